"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

This is what makes the pins meaningful: a dropped term, a wrong sign, a wrong
index or a transposed operand anywhere in the oracle must fail at least one.
"""
import math

import numpy as np
import pytest

import oracle
import pins
from oracle import attention as oatt
from oracle import expand as oexp
from oracle import occupancy as oocc
from oracle._arrays import f64


def _scores_no_rope(qb, kn, kr, mrow, scale, dn):
    s = scale * (qb[:, :dn] @ kn.T)
    return s if mrow is None else s + mrow


def _scores_rope_sign(qb, kn, kr, mrow, scale, dn):
    s = scale * (qb[:, :dn] @ kn.T - qb[:, dn:] @ kr.T)
    return s if mrow is None else s + mrow


def _scores_scale_after_mask(qb, kn, kr, mrow, scale, dn):
    s = qb[:, :dn] @ kn.T + qb[:, dn:] @ kr.T
    return scale * (s if mrow is None else s + mrow)


def _scores_mask_ignored(qb, kn, kr, mrow, scale, dn):
    return scale * (qb[:, :dn] @ kn.T + qb[:, dn:] @ kr.T)


def _scores_rope_into_nope_slot(qb, kn, kr, mrow, scale, dn):
    # pairs q_rope with the first Dr dims of k_nope instead of k_rope
    dr = kr.shape[1]
    s = scale * (qb[:, :dn] @ kn.T + qb[:, dn:] @ kn[:, :dr].T)
    return s if mrow is None else s + mrow


def _softmax_wrong_axis(s):
    e = np.exp(s - np.max(np.where(np.isfinite(s), s, -1e300), axis=0, keepdims=True))
    z = e.sum(axis=0, keepdims=True)
    return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def _softmax_uniform_dead_rows(s):
    m = s.max(axis=-1, keepdims=True)
    dead = m == -np.inf
    e = np.where(dead, 1.0, np.exp(s - np.where(dead, 0.0, m)))
    return e / e.sum(axis=-1, keepdims=True)


def _softmax_no_normalise(s):
    m = s.max(axis=-1, keepdims=True)
    dead = m == -np.inf
    return np.where(dead, 0.0, np.exp(s - np.where(dead, 0.0, m)))


def _attn_wrong_v_head(q, k_nope, k_rope, v, mask, scale, q_rows=None):
    H = v.shape[1]
    v2 = np.concatenate([f64(v)[:, 1:], f64(v)[:, :1]], axis=1) if H > 1 else f64(v)[..., ::-1]
    return _orig_attn(q, k_nope, k_rope, v2, mask, scale, q_rows)


def _attn_mask_transposed_rows(q, k_nope, k_rope, v, mask, scale, q_rows=None):
    if mask is not None:
        mask = f64(mask)[:, :, ::-1, :]
    return _orig_attn(q, k_nope, k_rope, v, mask, scale, q_rows)


def _expand_swapped_slices(latent, w, H, Dn, Dv):
    lat, ww = f64(latent), f64(w)
    B, Lk, R = lat.shape
    kv = (lat @ ww.T).reshape(B, Lk, H, Dn + Dv)
    return (np.ascontiguousarray(kv[..., Dv:].transpose(0, 2, 1, 3)),
            np.ascontiguousarray(kv[..., :Dv].transpose(0, 2, 1, 3)))


def _expand_slice_major(latent, w, H, Dn, Dv):
    lat, ww = f64(latent), f64(w)
    B, Lk, R = lat.shape
    kv = (lat @ ww.T).reshape(B, Lk, Dn + Dv, H).transpose(0, 1, 3, 2)
    return (np.ascontiguousarray(kv[..., :Dn].transpose(0, 2, 1, 3)),
            np.ascontiguousarray(kv[..., Dn:].transpose(0, 2, 1, 3)))


def _classes_positive_zero_only(mask, BM, BN):
    m = f64(mask)
    out = _orig_classes(m, BM, BN)
    B, _, Lq, Lk = m.shape
    for b in range(B):
        for qt in range(out.shape[1]):
            for kt in range(out.shape[2]):
                t = m[b, 0, qt * BM:(qt + 1) * BM, kt * BN:(kt + 1) * BN]
                if out[b, qt, kt] == 1 and np.any(np.signbit(t)):
                    out[b, qt, kt] = 2
    return out


def _classes_nan_as_masked(mask, BM, BN):
    m = f64(mask).copy()
    m[np.isnan(m)] = -np.inf
    return _orig_classes(m, BM, BN)


def _classes_square_tiles(mask, BM, BN):
    return _orig_classes(mask, BM, BM)


def _classes_binary_as_values(mask, BM, BN):
    out = _orig_classes(mask, BM, BN)
    out[out == 2] = 3
    return out


def _bits_transposed(mask, BM, BN, classes):
    out = _orig_bits(mask, BM, BN, classes)
    rev = np.zeros_like(out)
    for k in range(BN):
        rev |= ((out >> np.uint64(k)) & np.uint64(1)) << np.uint64(BN - 1 - k)
    return rev


def _bwd_variant(kind):
    """The backward with one planted mistake (test code, not the oracle)."""
    def f(q, k_nope, k_rope, v, mask, dout, scale, heads=None):
        from oracle._arrays import f64
        B, H = q.shape[:2]
        dn = k_nope.shape[-1]
        dq, dkn = np.zeros(q.shape), np.zeros(k_nope.shape)
        dkr, dv = np.zeros(k_rope.shape), np.zeros(v.shape)
        for b in range(B):
            for h in range(H) if heads is None else heads:
                p = oracle.softmax_weights(q, k_nope, k_rope, mask, scale, b, h)
                qb, kn, kr = f64(q[b, h]), f64(k_nope[b, h]), f64(k_rope[b])
                do, vb = f64(dout[b, h]), f64(v[b, h])
                dp = do @ vb.T
                D = 0.0 if kind == "no_D" else (p * dp).sum(axis=-1, keepdims=True)
                ds = p * (dp - D)
                dv[b, h] = (ds if kind == "dv_from_ds" else p).T @ do
                dq[b, h, :, :dn] = scale * (ds @ kn)
                dq[b, h, :, dn:] = (-scale if kind == "dq_rope_sign" else scale) * (ds @ kr)
                dkn[b, h] = (1.0 if kind == "dk_unscaled" else scale) * (ds.T @ qb[:, :dn])
                if kind == "rope_last_head":
                    dkr[b] = scale * (ds.T @ qb[:, dn:])
                else:
                    dkr[b] += scale * (ds.T @ qb[:, dn:])
        return dq, dkn, dkr, dv
    return f


def _lse_log2(q, k_nope, k_rope, mask, scale):
    return _orig_lse(q, k_nope, k_rope, mask, scale) / math.log(2.0)


from oracle import projection as oproj


def _rms_no_eps(x, gamma, eps):
    return _orig_rms(x, gamma, 0.0)


def _rms_no_gamma(x, gamma, eps):
    return _orig_rms(x, np.ones_like(f64(gamma)), eps)


def _rms_mean_abs(x, gamma, eps):
    x = f64(x)
    return x / (np.abs(x).mean(axis=-1, keepdims=True) + eps) * f64(gamma)


def _q_heads_inner(x, w_q_a, gamma_q, eps, w_q_b, H):
    q = oproj.linear(oproj.rms_norm(oproj.linear(x, w_q_a), gamma_q, eps), w_q_b)
    B, L, N = q.shape
    return q.reshape(B, L, N // H, H).transpose(0, 3, 1, 2)


def _kv_noise_first(ctx_hidden, noise_hidden, w_kv_a, gamma_kv, eps, w_kv_b, H, R, Dn=128, Dv=128):
    if ctx_hidden is None:
        return _orig_kv(None, noise_hidden, w_kv_a, gamma_kv, eps, w_kv_b, H, R, Dn, Dv)
    h = np.concatenate([f64(noise_hidden), f64(ctx_hidden)], axis=1)
    c = oproj.linear(h, w_kv_a)
    kn, v = oracle.latent_expand(oproj.rms_norm(c[..., :R], gamma_kv, eps), w_kv_b, H, Dn, Dv)
    return kn, c[..., R:], v


def _kv_rope_first(ctx_hidden, noise_hidden, w_kv_a, gamma_kv, eps, w_kv_b, H, R, Dn=128, Dv=128):
    h = f64(noise_hidden) if ctx_hidden is None else np.concatenate([f64(ctx_hidden), f64(noise_hidden)], axis=1)
    c = oproj.linear(h, w_kv_a)
    Dr = c.shape[-1] - R
    kn, v = oracle.latent_expand(oproj.rms_norm(c[..., Dr:], gamma_kv, eps), w_kv_b, H, Dn, Dv)
    return kn, c[..., :Dr], v


def _kv_norm_whole(ctx_hidden, noise_hidden, w_kv_a, gamma_kv, eps, w_kv_b, H, R, Dn=128, Dv=128):
    h = f64(noise_hidden) if ctx_hidden is None else np.concatenate([f64(ctx_hidden), f64(noise_hidden)], axis=1)
    c = oproj.linear(h, w_kv_a)
    Dr = c.shape[-1] - R
    cn = oproj.rms_norm(c, np.concatenate([f64(gamma_kv), np.ones(Dr)]), eps)
    kn, v = oracle.latent_expand(cn[..., :R], w_kv_b, H, Dn, Dv)
    return kn, cn[..., R:], v


from oracle import gqa as ogqa


def _rope_interleaved(x, positions, inv_freq, mscale=1.0):
    x = f64(x)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * f64(inv_freq)
    c, sn = np.cos(ang) * mscale, np.sin(ang) * mscale
    out = x.copy()
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * sn
    out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * sn
    return out


def _rope_sign(x, positions, inv_freq, mscale=1.0):
    return _orig_rope(x, -np.asarray(positions, dtype=np.float64), inv_freq, mscale)


def _gqa_head_modulo(q, k, v, lens, scale):
    q, k, v = f64(q), f64(k), f64(v)
    Hkv = k.shape[1]
    out = np.zeros(q.shape[:3] + (v.shape[-1],))
    for b in range(q.shape[0]):
        n = int(lens[b])
        for h in range(q.shape[1]):
            s_ = scale * (q[b, h] @ k[b, h % Hkv, :n].T)
            p_ = np.exp(s_ - s_.max(axis=-1, keepdims=True))
            out[b, h] = (p_ / p_.sum(axis=-1, keepdims=True)) @ v[b, h % Hkv, :n]
    return out


def _yarn_betas_swapped(dim, base, factor, orig, beta_fast, beta_slow):
    return _orig_yarn(dim, base, factor, orig, beta_slow, beta_fast)


def _correction_dim_no_two_pi(rotations, dim, base, max_pos):
    return dim * math.log(max_pos / rotations) / (2.0 * math.log(base))


def _yarn_floor_ceil_swapped(dim, base, factor, orig, beta_fast, beta_slow):
    i = np.arange(0, dim, 2, dtype=np.float64)
    extra = 1.0 / base ** (i / dim)
    low = max(math.ceil(ogqa._correction_dim(beta_fast, dim, base, orig)), 0)
    high = min(math.floor(ogqa._correction_dim(beta_slow, dim, base, orig)), dim - 1)
    if low == high:
        high += 0.001
    w = np.clip((np.arange(dim // 2, dtype=np.float64) - low) / (high - low), 0.0, 1.0)
    return extra * (1.0 - w) + extra / factor * w


def _fb_zero(blk_hidden, w_q, w_k, w_v, gamma_q, gamma_k, eps, Hq, Hkv, k_ctx, v_ctx, ctx_len, inv_freq, mscale):
    x = f64(blk_hidden)
    B, bs, _ = x.shape
    pos = np.arange(bs)[None, None, :]
    q = ogqa.rope(oproj.rms_norm(ogqa._heads(oproj.linear(x, w_q), Hq), gamma_q, eps), pos, inv_freq, mscale)
    kb = ogqa.rope(oproj.rms_norm(ogqa._heads(oproj.linear(x, w_k), Hkv), gamma_k, eps), pos, inv_freq, mscale)
    vb = ogqa._heads(oproj.linear(x, w_v), Hkv)
    out = np.zeros((B, Hq, bs, q.shape[-1]))
    for b in range(B):
        n = int(ctx_len[b])
        k = np.concatenate([f64(k_ctx[b:b + 1, :, :n]), kb[b:b + 1]], axis=2)
        v = np.concatenate([f64(v_ctx[b:b + 1, :, :n]), vb[b:b + 1]], axis=2)
        out[b] = ogqa.gqa_attention(q[b:b + 1], k, v, [n + bs], q.shape[-1] ** -0.5)[0]
    return out


def _materialize_norm_after_rope(ctx_hidden, w_k, w_v, gamma_k, eps, Hkv, inv_freq, mscale=1.0):
    x = f64(ctx_hidden)
    k = oproj.rms_norm(ogqa.rope(ogqa._heads(oproj.linear(x, w_k), Hkv), np.arange(x.shape[1]), inv_freq, mscale),
                       gamma_k, eps)
    return k, ogqa._heads(oproj.linear(x, w_v), Hkv)


_orig_rope = ogqa.rope
_orig_yarn = ogqa.yarn_inv_freq
_orig_fb = ogqa.forward_block
_orig_rms = oproj.rms_norm
_orig_kv = oracle.kv_project
_orig_lse = oracle.logsumexp_rows
_orig_attn = oracle.mla_attention
_orig_classes = oracle.tile_classes
_orig_bits = oracle.tile_bits

MUTANTS = {
    "drop_rope_term": [(oatt, "_scores", _scores_no_rope)],
    "rope_sign": [(oatt, "_scores", _scores_rope_sign)],
    "scale_after_mask": [(oatt, "_scores", _scores_scale_after_mask)],
    "mask_ignored": [(oatt, "_scores", _scores_mask_ignored)],
    "rope_paired_with_nope": [(oatt, "_scores", _scores_rope_into_nope_slot)],
    "softmax_wrong_axis": [(oatt, "_softmax_rows", _softmax_wrong_axis)],
    "dead_row_uniform": [(oatt, "_softmax_rows", _softmax_uniform_dead_rows)],
    "no_normalisation": [(oatt, "_softmax_rows", _softmax_no_normalise)],
    "wrong_v_head": [(oracle, "mla_attention", _attn_wrong_v_head)],
    "mask_rows_reversed": [(oracle, "mla_attention", _attn_mask_transposed_rows)],
    "expand_swapped_slices": [(oracle, "latent_expand", _expand_swapped_slices)],
    "expand_slice_major": [(oracle, "latent_expand", _expand_slice_major)],
    "occupancy_neg_zero": [(oracle, "tile_classes", _classes_positive_zero_only)],
    "occupancy_nan_masked": [(oracle, "tile_classes", _classes_nan_as_masked)],
    "occupancy_square_tiles": [(oracle, "tile_classes", _classes_square_tiles)],
    "occupancy_binary_as_values": [(oracle, "tile_classes", _classes_binary_as_values)],
    "occupancy_bits_reversed": [(oracle, "tile_bits", _bits_transposed)],
    "backward_no_D": [(oracle, "mla_attention_backward", _bwd_variant("no_D"))],
    "backward_dv_from_ds": [(oracle, "mla_attention_backward", _bwd_variant("dv_from_ds"))],
    "backward_dq_rope_sign": [(oracle, "mla_attention_backward", _bwd_variant("dq_rope_sign"))],
    "backward_dk_unscaled": [(oracle, "mla_attention_backward", _bwd_variant("dk_unscaled"))],
    "backward_rope_last_head": [(oracle, "mla_attention_backward", _bwd_variant("rope_last_head"))],
    "lse_in_log2": [(oracle, "logsumexp_rows", _lse_log2)],
    "rms_no_eps": [(oproj, "rms_norm", _rms_no_eps), (oracle, "rms_norm", _rms_no_eps)],
    "rms_no_gamma": [(oproj, "rms_norm", _rms_no_gamma), (oracle, "rms_norm", _rms_no_gamma)],
    "rms_mean_abs": [(oproj, "rms_norm", _rms_mean_abs), (oracle, "rms_norm", _rms_mean_abs)],
    "q_heads_inner": [(oracle, "q_project", _q_heads_inner)],
    "kv_noise_first": [(oracle, "kv_project", _kv_noise_first)],
    "kv_rope_first": [(oracle, "kv_project", _kv_rope_first)],
    "kv_norm_whole_row": [(oracle, "kv_project", _kv_norm_whole)],
    "rope_interleaved_pairs": [(ogqa, "rope", _rope_interleaved), (oracle, "rope", _rope_interleaved)],
    "rope_sign": [(ogqa, "rope", _rope_sign), (oracle, "rope", _rope_sign)],
    "gqa_head_modulo": [(ogqa, "gqa_attention", _gqa_head_modulo), (oracle, "gqa_attention", _gqa_head_modulo)],
    "yarn_betas_swapped": [(ogqa, "yarn_inv_freq", _yarn_betas_swapped), (oracle, "yarn_inv_freq", _yarn_betas_swapped)],
    "yarn_no_two_pi": [(ogqa, "_correction_dim", _correction_dim_no_two_pi)],
    "yarn_floor_ceil_swapped": [(ogqa, "yarn_inv_freq", _yarn_floor_ceil_swapped),
                                (oracle, "yarn_inv_freq", _yarn_floor_ceil_swapped)],
    "block_positions_from_zero": [(oracle, "forward_block", _fb_zero)],
    "qk_norm_after_rope": [(oracle, "materialize", _materialize_norm_after_rope)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
