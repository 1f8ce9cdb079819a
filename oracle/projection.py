"""fp64 projections around the draft attention -- the plain definitions (test infrastructure only).

DFlash page, module text: the draft's MLA has Q-LoRA and a compressed KV latent
and uses an RMSNorm whose variance is computed in fp32 (the Kimi RMSNorm; its
class text on the K3 model page says the same).  DSpark page,
KimiK3DSparkAttention attributes: q_a_proj, q_a_layernorm, q_b_proj,
kv_a_proj_with_mqa, kv_a_layernorm, kv_b_proj, q_head_dim = qk_nope + qk_rope,
kv_lora_rank; KimiK3DSparkAttention.forward: the frozen target context is
concatenated before the noise block to form the keys and values;
KimiK3DSparkModel._forward_backbone: the target hidden states are projected by
fc and normed once.  K3 model page, MLA context-parallel forward: the
compressed latent holds kv_lora_rank + qk_rope_head_dim values per token.

Readings (the pages name the modules, not their arithmetic):
  rms_norm(x)     = x / sqrt(mean(x^2) + eps) * gamma        (over the last axis)
  a Linear        = x @ W^T, W stored [out, in], no bias
  q               = rms_norm(x @ Wqa^T, gq) @ Wqb^T, split per head into q_head_dim
                    slices (heads outer), laid out [B, H, L, q_head_dim]
  c               = [ctx ; noise] @ Wkva^T, per token [latent (R) | k_rope (Dr)]
  k_nope, v       = kv_b_proj of rms_norm(latent, gkv)  (expand.latent_expand)
  context         = rms_norm(target_hidden @ Wfc^T, gh)
"""
from __future__ import annotations

import numpy as np

from ._arrays import f64
from .expand import latent_expand


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis, fp64."""
    x = f64(x)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * f64(gamma)


def linear(x, w) -> np.ndarray:
    """x @ W^T with W stored [out, in]."""
    return f64(x) @ f64(w).T


def context_project(target_hidden, w_fc, gamma, eps: float) -> np.ndarray:
    """[B, ctx, K_in] -> [B, ctx, hidden]: fc, then hidden_norm."""
    return rms_norm(linear(target_hidden, w_fc), gamma, eps)


def q_project(x, w_q_a, gamma_q, eps: float, w_q_b, H: int) -> np.ndarray:
    """[B, L, hidden] -> q [B, H, L, Dqk]: q_a_proj, q_a_layernorm, q_b_proj."""
    q = linear(rms_norm(linear(x, w_q_a), gamma_q, eps), w_q_b)      # [B, L, H*Dqk]
    B, L, N = q.shape
    return q.reshape(B, L, H, N // H).transpose(0, 2, 1, 3)


def kv_project(ctx_hidden, noise_hidden, w_kv_a, gamma_kv, eps: float, w_kv_b, H: int, R: int,
               Dn: int = 128, Dv: int = 128):
    """Keys and values over [context | noise]: (k_nope [B,H,Lk,Dn], k_rope [B,Lk,Dr], v [B,H,Lk,Dv])."""
    h = f64(noise_hidden) if ctx_hidden is None else np.concatenate([f64(ctx_hidden), f64(noise_hidden)], axis=1)
    c = linear(h, w_kv_a)
    latent = rms_norm(c[..., :R], gamma_kv, eps)
    k_nope, v = latent_expand(latent, w_kv_b, H, Dn, Dv)
    return k_nope, c[..., R:], v
