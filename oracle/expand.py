"""fp64 kv_b_proj latent expansion -- the plain definition (test infrastructure only).

NeMo AutoModel "dflash.draft_kimi_k3" page, KimiK3DFlashAttention class text,
and "dspark.draft_kimi_k3" page, KimiK3DSparkAttention class text: kv_b_proj
produces num_attention_heads slices of qk_nope_head_dim + v_head_dim, one per
query head.  Kimi K3 model page, MLA context-parallel forward: the compressed
latent the projection consumes is kv_lora_rank (+ the head-shared rope part,
which does not go through kv_b_proj) values per token.

Reading (the pages do not print the weight layout): kv_b_proj is a bias-free
Linear with weight [H * (Dn + Dv), R] (out x in); output column
h * (Dn + Dv) + e is head h's k_nope[e] for e < Dn and head h's v[e - Dn] after.

    kv[b, t, h, e] = sum_r latent[b, t, r] * W[h * (Dn + Dv) + e, r]
    k_nope[b, h, t, :] = kv[b, t, h, :Dn];   v[b, h, t, :] = kv[b, t, h, Dn:]
"""
from __future__ import annotations

import numpy as np

from ._arrays import f64


def latent_expand(latent, w_kv_b, H: int, Dn: int, Dv: int):
    lat = f64(latent)                    # [B, Lk, R]
    w = f64(w_kv_b)                      # [H*(Dn+Dv), R]
    B, Lk, R = lat.shape
    if w.shape != (H * (Dn + Dv), R):
        raise ValueError(f"w_kv_b must be [{H * (Dn + Dv)}, {R}], got {w.shape}")
    kv = (lat @ w.T).reshape(B, Lk, H, Dn + Dv)
    k_nope = np.ascontiguousarray(kv[..., :Dn].transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(kv[..., Dn:].transpose(0, 2, 1, 3))
    return k_nope, v
