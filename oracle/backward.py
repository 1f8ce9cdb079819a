"""fp64 gradients of the draft attention -- the plain definition (test infrastructure only).

The draft is trained: the DFlash page's KimiK3DFlashDraftModel class text has the
DFlash trainer embed the anchor/mask blocks and decode the draft's output, and the
DSpark page's module text calls its backbone one for speculative-decoding
training.  Training needs the gradients of the attention of attention.py with
respect to its four tensor inputs.  The mask is an input the trainer builds, not
a parameter, so it gets no gradient.

With s, p and out as in attention.py (one batch row b, one head h, query i,
key j, and Dn the k_nope width) and dout the gradient arriving at out:

    dp[i,j]  = dout[i,:] . v[j,:]
    D[i]     = sum_j p[i,j] * dp[i,j]          (= dout[i,:] . out[i,:])
    ds[i,j]  = p[i,j] * (dp[i,j] - D[i])       (the softmax Jacobian applied to dp)
    dv[j,:]  = sum_i p[i,j] * dout[i,:]
    dq[i,:]  = scale * sum_j ds[i,j] * [k_nope[j,:] | k_rope[j,:]]
    dk_nope[j,:] = scale * sum_i ds[i,j] * q[i,:Dn]
    dk_rope[b,j,:] = scale * sum_h sum_i ds_h[i,j] * q_h[i,Dn:]   (the rope key is
                     one tensor used by every head, so its gradient sums over heads)

A row whose scores are all -inf returns the constant 0 (the reading of
attention.py), so it passes no gradient: its p and ds are 0.  Hidden entries
(mask -inf) have p = 0 and drop out of every sum.
"""
from __future__ import annotations

import numpy as np

from ._arrays import f64


def _probs(qb, kn, kr, mrow, scale, dn):
    """Row softmax of one (b, h) score matrix; an all -inf row gives zeros."""
    s = scale * (qb[:, :dn] @ kn.T + qb[:, dn:] @ kr.T)
    if mrow is not None:
        s = s + mrow
    m = s.max(axis=-1, keepdims=True)
    dead = m == -np.inf
    e = np.exp(s - np.where(dead, 0.0, m))
    z = e.sum(axis=-1, keepdims=True)
    return np.where(dead, 0.0, e / np.where(dead, 1.0, z))


def mla_attention_backward(q, k_nope, k_rope, v, mask, dout, scale: float, heads=None):
    """(dq, dk_nope, dk_rope, dv) in fp64, shaped like q, k_nope, k_rope, v.

    `heads` (a list of head indices) restricts dq / dk_nope / dv to those heads
    (the other heads' slices stay 0) for spot checks at large sizes; dk_rope sums
    over the heads computed, so it is complete only when `heads` is None.
    """
    B, H, Lq, _ = q.shape
    dn = k_nope.shape[-1]
    dq = np.zeros(q.shape, dtype=np.float64)
    dkn = np.zeros(k_nope.shape, dtype=np.float64)
    dkr = np.zeros(k_rope.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    hs = range(H) if heads is None else heads
    for b in range(B):
        kr = f64(k_rope[b])
        mrow = None if mask is None else f64(mask[b, 0])
        for h in hs:
            qb, kn, vb, do = f64(q[b, h]), f64(k_nope[b, h]), f64(v[b, h]), f64(dout[b, h])
            p = _probs(qb, kn, kr, mrow, scale, dn)
            dp = do @ vb.T
            D = (p * dp).sum(axis=-1, keepdims=True)
            ds = p * (dp - D)
            dv[b, h] = p.T @ do
            dq[b, h, :, :dn] = scale * (ds @ kn)
            dq[b, h, :, dn:] = scale * (ds @ kr)
            dkn[b, h] = scale * (ds.T @ qb[:, :dn])
            dkr[b] += scale * (ds.T @ qb[:, dn:])
    return dq, dkn, dkr, dv


def logsumexp_rows(q, k_nope, k_rope, mask, scale: float) -> np.ndarray:
    """[B, H, Lq] natural-log normaliser log(sum_j exp(s[i,j])) of each row; -inf
    for a row with no finite score.  Saved by a forward pass for its backward."""
    B, H, Lq, _ = q.shape
    dn = k_nope.shape[-1]
    out = np.empty((B, H, Lq), dtype=np.float64)
    for b in range(B):
        kr = f64(k_rope[b])
        mrow = None if mask is None else f64(mask[b, 0])
        for h in range(H):
            qb = f64(q[b, h])
            s = scale * (qb[:, :dn] @ f64(k_nope[b, h]).T + qb[:, dn:] @ kr.T)
            if mrow is not None:
                s = s + mrow
            m = s.max(axis=-1)
            dead = m == -np.inf
            mm = np.where(dead, 0.0, m)
            z = np.exp(s - mm[:, None]).sum(axis=-1)
            out[b, h] = np.where(dead, -np.inf, mm + np.log(np.where(dead, 1.0, z)))
    return out
