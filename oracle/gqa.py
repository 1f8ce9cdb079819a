"""fp64 GQA draft attention with yarn RoPE and qk-norm -- the plain definitions (test infrastructure only).

Modular MAX page, pipelines.architectures.dflash_kimi_k25 (module text): a
DFlash draft for a Kimi K2.5 (DeepSeek-V3 MLA) target.  The draft's own
attention is ordinary MHA/GQA with DeepSeek-yarn RoPE, so its KV cache has its
own layout, independent of the target's MLA cache.  The context K/V go into
the draft's cache once (DFlashKimiK25.materialize); each block then attends to
that cache plus its own keys (DFlashKimiK25.forward_block), as in the page's
llama3 DFlash draft.  construct_kv_params: the draft's cache is always bf16,
independent of the target's cache dtype, and is sized by the draft block it
stores.  The
config fields are num_attention_heads, num_key_value_heads, head_dim,
rms_norm_eps, rope_theta, rope_scaling and use_qk_norm
(DFlashKimiK25DraftConfig).

Readings (the page prints no arithmetic):
  * yarn RoPE as DeepSeek-V3 defines it: per frequency pair i of the rotary
    width d, the extrapolated 1 / theta^(2i/d) and the interpolated value
    divided by `factor` are blended by a linear ramp between the correction
    dimensions of beta_fast and beta_slow rotations at the original context
    length; cos and sin are scaled by mscale(factor, mscale) /
    mscale(factor, mscale_all_dim), mscale(s, m) = 0.1 m ln s + 1 (1 if s <= 1).
  * RoPE pairs dimension i with i + d/2 (rotate-half): x' = x cos + rot(x) sin,
    rot(x) = [-x[d/2:], x[:d/2]]; the angle of pair i at position p is p * inv_freq[i].
  * qk-norm: RMSNorm over head_dim of every head (one weight vector per q / k),
    before RoPE.  v is neither normed nor rotated.
  * positions: context token t sits at t; block token i of batch row b at
    ctx_len[b] + i.  The block sees every cached context key and every block key
    (non-causal); scale head_dim ** -0.5.
  * query head h reads KV head h // (num_attention_heads / num_key_value_heads).
"""
from __future__ import annotations

import math

import numpy as np

from ._arrays import f64
from .projection import linear, rms_norm


def yarn_mscale(scale: float, mscale: float) -> float:
    return 1.0 if scale <= 1.0 else 0.1 * mscale * math.log(scale) + 1.0


def _correction_dim(rotations: float, dim: int, base: float, max_pos: int) -> float:
    """The rotary dimension whose wavelength fits `rotations` turns in max_pos."""
    return dim * math.log(max_pos / (rotations * 2.0 * math.pi)) / (2.0 * math.log(base))


def yarn_inv_freq(dim: int, base: float, factor: float, orig_max_pos: int, beta_fast: float,
                  beta_slow: float) -> np.ndarray:
    """[dim / 2] inverse frequencies of yarn RoPE (fp64)."""
    i = np.arange(0, dim, 2, dtype=np.float64)
    extra = 1.0 / base ** (i / dim)
    inter = extra / factor
    low = max(math.floor(_correction_dim(beta_fast, dim, base, orig_max_pos)), 0)
    high = min(math.ceil(_correction_dim(beta_slow, dim, base, orig_max_pos)), dim - 1)
    if low == high:
        high += 0.001
    ramp = np.clip((np.arange(dim // 2, dtype=np.float64) - low) / (high - low), 0.0, 1.0)
    keep_extra = 1.0 - ramp
    return inter * (1.0 - keep_extra) + extra * keep_extra


def rope(x, positions, inv_freq, mscale: float = 1.0) -> np.ndarray:
    """Rotate-half RoPE of x [..., T, d] at positions broadcastable to [..., T]."""
    x = f64(x)
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[..., None] * f64(inv_freq)      # [..., T, d/2]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1) * mscale
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1) * mscale
    rot = np.concatenate([-x[..., d // 2:], x[..., :d // 2]], axis=-1)
    return x * cos + rot * sin


def gqa_attention(q, k, v, lens, scale: float) -> np.ndarray:
    """q [B, Hq, Lq, d]; k, v [B, Hkv, Lk, d]; row b sees keys j < lens[b] -> [B, Hq, Lq, d]."""
    q, k, v = f64(q), f64(k), f64(v)
    B, Hq, Lq, _ = q.shape
    g = Hq // k.shape[1]
    out = np.zeros(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // g, :n].T)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            out[b, h] = (p / p.sum(axis=-1, keepdims=True)) @ v[b, h // g, :n]
    return out


def _heads(x, H: int) -> np.ndarray:
    """[B, T, H*d] -> [B, H, T, d]."""
    B, T, N = x.shape
    return x.reshape(B, T, H, N // H).transpose(0, 2, 1, 3)


def materialize(ctx_hidden, w_k, w_v, gamma_k, eps: float, Hkv: int, inv_freq, mscale: float = 1.0):
    """Context K/V for the cache: k = rope(rms_norm(x W_k^T per head)) at positions
    0..Lc-1, v = x W_v^T; both [B, Hkv, Lc, d]."""
    x = f64(ctx_hidden)
    Lc = x.shape[1]
    k = rope(rms_norm(_heads(linear(x, w_k), Hkv), gamma_k, eps), np.arange(Lc), inv_freq, mscale)
    return k, _heads(linear(x, w_v), Hkv)


def forward_block(blk_hidden, w_q, w_k, w_v, gamma_q, gamma_k, eps: float, Hq: int, Hkv: int,
                  k_ctx, v_ctx, ctx_len, inv_freq, mscale: float = 1.0):
    """Attention output [B, Hq, bs, d] of a block over [cached context | block]:
    the block's q / k / v at positions ctx_len[b] + i, keys = the first ctx_len[b]
    cached context keys then the block's keys."""
    x = f64(blk_hidden)
    B, bs, _ = x.shape
    pos = np.asarray(ctx_len, dtype=np.float64)[:, None, None] + np.arange(bs)[None, None, :]   # [B, 1, bs]
    q = rope(rms_norm(_heads(linear(x, w_q), Hq), gamma_q, eps), pos, inv_freq, mscale)
    kb = rope(rms_norm(_heads(linear(x, w_k), Hkv), gamma_k, eps), pos, inv_freq, mscale)
    vb = _heads(linear(x, w_v), Hkv)
    d = q.shape[-1]
    out = np.zeros((B, Hq, bs, d), dtype=np.float64)
    for b in range(B):
        n = int(ctx_len[b])
        k = np.concatenate([f64(k_ctx[b:b + 1, :, :n]), kb[b:b + 1]], axis=2)
        v = np.concatenate([f64(v_ctx[b:b + 1, :, :n]), vb[b:b + 1]], axis=2)
        out[b] = gqa_attention(q[b:b + 1], k, v, [n + bs], d ** -0.5)[0]
    return out
