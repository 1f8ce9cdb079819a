"""fp64 masked softmax attention -- the plain definition (test infrastructure only).

NeMo AutoModel "dflash.draft_kimi_k3" page, KimiK3DFlashAttention.forward: the
draft's queries are the noise tokens, its keys/values span [context | noise],
and the dense additive mask is added to the scores unchanged.  Class text:
kv_b_proj emits one qk_nope + v slice per query head, so every query head has
its own K/V (no group repeat).  Module text: NoPE -- the qk_rope_head_dim slice
of the key is one vector per token shared by all heads, with no rotary.
"dspark.draft_kimi_k3" page, KimiK3DSparkAttention: q_head_dim =
qk_nope_head_dim + qk_rope_head_dim and scaling = q_head_dim ** -0.5.

For batch b, head h, query i and key j:

    s[j] = scale * (q[b,h,i,:Dn] . k_nope[b,h,j,:] + q[b,h,i,Dn:] . k_rope[b,j,:])
           + mask[b,0,i,j]                              (mask term absent if None)
    p[j] = exp(s[j] - max_j s) / sum_j exp(s[j] - max_j s)
    out[b,h,i,:] = sum_j p[j] * v[b,h,j,:]

A row whose scores are all -inf has no defined softmax; it returns zeros (a
reading -- the pages do not say).  exp(-inf) is exactly 0, so -inf entries drop
out of both sums.
"""
from __future__ import annotations

import numpy as np

from ._arrays import f64


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of an fp64 score matrix; an all -inf row gives all zeros."""
    m = s.max(axis=-1, keepdims=True)
    dead = m == -np.inf
    m = np.where(dead, 0.0, m)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return np.where(dead, 0.0, e / np.where(dead, 1.0, z))


def _scores(qb: np.ndarray, kn: np.ndarray, kr: np.ndarray, mrow, scale: float, dn: int):
    s = scale * (qb[:, :dn] @ kn.T + qb[:, dn:] @ kr.T)
    if mrow is not None:
        s = s + mrow
    return s


def softmax_weights(q, k_nope, k_rope, mask, scale: float, b: int, h: int) -> np.ndarray:
    """The [Lq, Lk] attention weights of one (batch, head) -- used by the pins."""
    dn = k_nope.shape[-1]
    qb = f64(q[b, h])
    s = _scores(qb, f64(k_nope[b, h]), f64(k_rope[b]),
                None if mask is None else f64(mask[b, 0]), scale, dn)
    return _softmax_rows(s)


def mla_attention(q, k_nope, k_rope, v, mask, scale: float, q_rows=None) -> np.ndarray:
    """out [B, H, n_rows, Dv] in fp64.

    q [B,H,Lq,Dn+Dr]; k_nope [B,H,Lk,Dn]; k_rope [B,Lk,Dr]; v [B,H,Lk,Dv];
    mask [B,1,Lq,Lk] or None.  `q_rows` (an index array into Lq) restricts the
    result to those query rows, for spot checks at full size; the arithmetic of
    each row is the same as without it.
    """
    B, H, Lq, _ = q.shape
    dn = k_nope.shape[-1]
    dv = v.shape[-1]
    rows = np.arange(Lq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    out = np.zeros((B, H, len(rows), dv), dtype=np.float64)
    for b in range(B):
        kr = f64(k_rope[b])
        mrow = None if mask is None else f64(mask[b, 0])[rows]
        for h in range(H):
            qb = f64(q[b, h])[rows]
            p = _softmax_rows(_scores(qb, f64(k_nope[b, h]), kr, mrow, scale, dn))
            out[b, h] = p @ f64(v[b, h])
    return out
