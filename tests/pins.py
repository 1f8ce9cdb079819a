"""Checks that pin the fp64 oracle to things other than itself.

Each check calls the oracle through the `oracle` package attributes, so a test
can plant a mistake inside the oracle (monkeypatching one of its internals)
and confirm that at least one check catches it.  None of these re-types the
oracle's formula: they use closed forms derived by hand, invariants of the
definition, a pure-Python brute force on tiny shapes, an explicit gather of
the keys a DFlash block may see, and PyTorch's own fused attention routine.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import attention as oatt
from oracle import expand as oexp
from oracle import occupancy as oocc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NINF = -np.inf


def _rand(seed, B, H, Lq, Lk, dn=8, dr=4, dv=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Lq, dn + dr))
    kn = rng.standard_normal((B, H, Lk, dn))
    kr = rng.standard_normal((B, Lk, dr))
    v = rng.standard_normal((B, H, Lk, dv))
    return q, kn, kr, v


def _rand_mask(seed, B, Lq, Lk, p_masked=0.5, finite_noise=True, keep_one=True):
    """Random additive mask with -inf entries; every row keeps >= 1 finite entry."""
    rng = np.random.default_rng(seed + 1000)
    m = rng.standard_normal((B, 1, Lq, Lk)) if finite_noise else np.zeros((B, 1, Lq, Lk))
    hide = rng.random((B, 1, Lq, Lk)) < p_masked
    if keep_one:
        keep = rng.integers(0, Lk, size=(B, 1, Lq))
        for b in range(B):
            for i in range(Lq):
                hide[b, 0, i, keep[b, 0, i]] = False
    m[hide] = NINF
    return m


# ---------------------------------------------------------------- attention

def pin_closed_form_golden():
    """Hand-derived cases in tests/golden/closed_form_attention.json."""
    with open(os.path.join(GOLDEN, "closed_form_attention.json")) as f:
        data = json.load(f)
    scale = 3.0 ** -0.5
    conv = {"-inf": NINF, "ln2": math.log(2.0)}
    for case in data["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, None]          # [1,1,Lq,3]
        a = np.log(np.array(case["k_nope_a"], dtype=np.float64) + 1.0) / (2.0 * scale)
        kn = np.stack([a, np.zeros_like(a)], axis=1)[None, None]        # [1,1,3,2]
        kr = a[:, None][None]                                           # [1,3,1]
        v = np.array(case["v"], dtype=np.float64)[None, None]
        mask = None
        if case["mask"] is not None:
            mask = np.array([[conv.get(x, x) if isinstance(x, str) else x for x in row]
                             for row in case["mask"]], dtype=np.float64)[None, None]
        out = oracle.mla_attention(q, kn, kr, v, mask, scale)[0, 0]
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12,
                                   err_msg=case["name"])


def pin_rows_sum_to_one():
    """Softmax weights: each row with a finite score sums to 1; -inf entries weigh 0."""
    q, kn, kr, v = _rand(1, 2, 3, 7, 11)
    mask = _rand_mask(1, 2, 7, 11)
    for b in range(2):
        for h in range(3):
            p = oracle.softmax_weights(q, kn, kr, mask, 0.3, b, h)
            np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
            assert np.all(p[mask[b, 0] == NINF] == 0.0)
            assert np.all(p >= 0.0)


def pin_zero_mask_equals_no_mask():
    q, kn, kr, v = _rand(2, 1, 2, 5, 9)
    a = oracle.mla_attention(q, kn, kr, v, np.zeros((1, 1, 5, 9)), 0.25)
    b = oracle.mla_attention(q, kn, kr, v, None, 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_single_visible_key_returns_its_value():
    q, kn, kr, v = _rand(3, 2, 2, 6, 10)
    mask = np.full((2, 1, 6, 10), NINF)
    rng = np.random.default_rng(3)
    js = rng.integers(0, 10, size=(2, 6))
    for b in range(2):
        for i in range(6):
            mask[b, 0, i, js[b, i]] = rng.standard_normal() * 5.0
    out = oracle.mla_attention(q, kn, kr, v, mask, 0.7)
    for b in range(2):
        for h in range(2):
            for i in range(6):
                np.testing.assert_array_equal(out[b, h, i], v[b, h, js[b, i]])


def pin_key_permutation_invariance():
    q, kn, kr, v = _rand(4, 1, 3, 8, 13)
    mask = _rand_mask(4, 1, 8, 13)
    perm = np.random.default_rng(4).permutation(13)
    a = oracle.mla_attention(q, kn, kr, v, mask, 0.4)
    b = oracle.mla_attention(q, kn[:, :, perm], kr[:, perm], v[:, :, perm], mask[..., perm], 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_row_shift_invariance():
    """Adding c to every finite mask entry of a row leaves that row unchanged."""
    q, kn, kr, v = _rand(5, 1, 2, 6, 9)
    mask = _rand_mask(5, 1, 6, 9)
    shifted = mask.copy()
    c = np.array([3.0, -7.5, 0.25, 40.0, -1.0, 12.0])
    shifted[0, 0] += c[:, None]          # -inf + c stays -inf
    a = oracle.mla_attention(q, kn, kr, v, mask, 0.5)
    b = oracle.mla_attention(q, kn, kr, v, shifted, 0.5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_zero_query_gives_mean_of_visible_values():
    _, kn, kr, v = _rand(6, 2, 2, 5, 12)
    q = np.zeros((2, 2, 5, 12))
    vis = np.random.default_rng(6).random((2, 5, 12)) < 0.6
    vis[:, :, 0] = True
    mask = np.where(vis, 0.0, NINF)[:, None]
    out = oracle.mla_attention(q, kn, kr, v, mask, 0.9)
    for b in range(2):
        for h in range(2):
            for i in range(5):
                np.testing.assert_allclose(out[b, h, i], v[b, h, vis[b, i]].mean(0), atol=1e-12)


def pin_value_shift_adds_constant():
    q, kn, kr, v = _rand(7, 1, 2, 4, 7)
    mask = _rand_mask(7, 1, 4, 7)
    c = 2.5
    a = oracle.mla_attention(q, kn, kr, v, mask, 0.35)
    b = oracle.mla_attention(q, kn, kr, v + c, mask, 0.35)
    np.testing.assert_allclose(b, a + c, atol=1e-12)


def pin_matches_torch_sdpa():
    """PyTorch's scaled_dot_product_attention (fp64, CPU) on explicit keys
    [k_nope | k_rope broadcast to every head] with the same float mask."""
    import torch
    import torch.nn.functional as F
    q, kn, kr, v = _rand(8, 2, 3, 9, 14, dn=16, dr=8, dv=12)
    mask = _rand_mask(8, 2, 9, 14)
    scale = 24 ** -0.5
    k = np.concatenate([kn, np.broadcast_to(kr[:, None], (2, 3, 14, 8))], axis=-1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(np.ascontiguousarray(k)),
                                         torch.from_numpy(v), attn_mask=torch.from_numpy(mask),
                                         scale=scale).numpy()
    out = oracle.mla_attention(q, kn, kr, v, mask, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_dflash_block_gather():
    """With the DFlash block mask, block j's rows equal plain softmax attention
    over the explicitly gathered keys context[0..anchor_j] + block j's own keys."""
    from scipy.special import softmax
    from dflash_block_draft_amd import workloads as W
    rng = np.random.default_rng(9)
    ctx, A, bs, H = 40, 3, 4, 2
    anchors = W.draw_anchors(rng, 1, A, ctx)
    vis = W.visibility(anchors, ctx, ctx, bs)
    mask = np.where(vis, 0.0, NINF)[:, None]
    Lq, Lk = A * bs, ctx + A * bs
    q, kn, kr, v = _rand(9, 1, H, Lq, Lk)
    scale = 12 ** -0.5
    out = oracle.mla_attention(q, kn, kr, v, mask, scale)
    for h in range(H):
        for j in range(A):
            keys = np.concatenate([np.arange(anchors[0, j] + 1), ctx + j * bs + np.arange(bs)])
            kfull = np.concatenate([kn[0, h][keys], kr[0][keys]], axis=1)
            for i in range(j * bs, (j + 1) * bs):
                w = softmax(scale * (kfull @ q[0, h, i]))
                np.testing.assert_allclose(out[0, h, i], w @ v[0, h][keys], atol=1e-12)


def pin_brute_force_tiny():
    """Pure-Python loops (math.exp, explicit sums) on tiny shapes."""
    q, kn, kr, v = _rand(10, 2, 2, 3, 5, dn=3, dr=2, dv=2)
    mask = _rand_mask(10, 2, 3, 5)
    mask[1, 0, 2, :] = NINF                               # one dead row
    scale = 0.6
    out = oracle.mla_attention(q, kn, kr, v, mask, scale)
    for b in range(2):
        for h in range(2):
            for i in range(3):
                s = []
                for j in range(5):
                    acc = 0.0
                    for d in range(3):
                        acc += q[b, h, i, d] * kn[b, h, j, d]
                    for d in range(2):
                        acc += q[b, h, i, 3 + d] * kr[b, j, d]
                    s.append(acc * scale + mask[b, 0, i, j])
                fin = [x for x in s if x != -math.inf]
                if not fin:
                    exp_out = [0.0, 0.0]
                else:
                    mx = max(fin)
                    e = [math.exp(x - mx) if x != -math.inf else 0.0 for x in s]
                    z = sum(e)
                    exp_out = [sum(e[j] * v[b, h, j, c] for j in range(5)) / z for c in range(2)]
                np.testing.assert_allclose(out[b, h, i], exp_out, atol=1e-12)


def pin_query_rows_subset():
    """Restricting to a subset of query rows returns exactly those rows."""
    q, kn, kr, v = _rand(11, 1, 2, 10, 8)
    mask = _rand_mask(11, 1, 10, 8)
    full = oracle.mla_attention(q, kn, kr, v, mask, 0.3)
    rows = np.array([7, 0, 3])
    sub = oracle.mla_attention(q, kn, kr, v, mask, 0.3, q_rows=rows)
    np.testing.assert_array_equal(sub, full[:, :, rows])


ATTENTION_PINS = [
    pin_closed_form_golden, pin_rows_sum_to_one, pin_zero_mask_equals_no_mask,
    pin_single_visible_key_returns_its_value, pin_key_permutation_invariance,
    pin_row_shift_invariance, pin_zero_query_gives_mean_of_visible_values,
    pin_value_shift_adds_constant, pin_matches_torch_sdpa, pin_dflash_block_gather,
    pin_brute_force_tiny, pin_query_rows_subset,
]


# ---------------------------------------------------------------- expand

def pin_expand_brute_force():
    rng = np.random.default_rng(20)
    B, Lk, R, H, Dn, Dv = 2, 3, 5, 2, 3, 2
    lat = rng.standard_normal((B, Lk, R))
    w = rng.standard_normal((H * (Dn + Dv), R))
    kn, v = oracle.latent_expand(lat, w, H, Dn, Dv)
    for b in range(B):
        for t in range(Lk):
            for h in range(H):
                for e in range(Dn + Dv):
                    acc = 0.0
                    for r in range(R):
                        acc += lat[b, t, r] * w[h * (Dn + Dv) + e, r]
                    got = kn[b, h, t, e] if e < Dn else v[b, h, t, e - Dn]
                    assert abs(got - acc) < 1e-12


def pin_expand_one_hot_layout():
    """A one-hot weight row copies one latent column to a known (head, slot)."""
    B, Lk, R, H, Dn, Dv = 1, 4, 6, 3, 2, 2
    lat = np.arange(B * Lk * R, dtype=np.float64).reshape(B, Lk, R) + 1.0
    w = np.zeros((H * (Dn + Dv), R))
    w[1 * (Dn + Dv) + 0, 4] = 1.0       # head 1, k_nope[0] <- latent[:, :, 4]
    w[2 * (Dn + Dv) + Dn + 1, 2] = 1.0  # head 2, v[1]      <- latent[:, :, 2]
    kn, v = oracle.latent_expand(lat, w, H, Dn, Dv)
    np.testing.assert_array_equal(kn[0, 1, :, 0], lat[0, :, 4])
    np.testing.assert_array_equal(v[0, 2, :, 1], lat[0, :, 2])
    assert np.count_nonzero(kn) == Lk and np.count_nonzero(v) == Lk


EXPAND_PINS = [pin_expand_brute_force, pin_expand_one_hot_layout]


# ---------------------------------------------------------------- occupancy

def pin_occupancy_brute_force():
    rng = np.random.default_rng(30)
    B, Lq, Lk, BM, BN = 2, 11, 23, 4, 5
    m = np.zeros((B, 1, Lq, Lk))
    m[rng.random(m.shape) < 0.7] = NINF
    m[0, 0, 0:4, 0:5] = NINF                       # one tile all -inf
    m[0, 0, 4:8, 5:10] = 0.0                       # one tile all zero
    m[0, 0, 4:8, 10:15] = -0.0                     # negative zeros count as zero
    m[1, 0, 8:11, 20:23] = NINF                    # a ragged corner tile, all -inf
    m[1, 0, 4:8, 0:5] = NINF
    m[1, 0, 5, 2] = np.nan                         # NaN alone in an otherwise -inf tile
    m[1, 0, 0:4, 10:15] = 0.0
    m[1, 0, 2, 11] = np.inf                        # +inf alone in an otherwise zero tile
    m[1, 0, 1, 6] = -3.0e38                        # large finite negatives are values
    cls = oracle.tile_classes(m, BM, BN)
    assert cls.shape == (B, 3, 5)
    for b in range(B):
        for qt in range(3):
            for kt in range(5):
                vals = [m[b, 0, i, j] for i in range(qt * BM, min(qt * BM + BM, Lq))
                        for j in range(kt * BN, min(kt * BN + BN, Lk))]
                if all(x == -math.inf for x in vals):
                    want = 0
                elif all(x == 0.0 for x in vals):
                    want = 1
                elif all(x == 0.0 or x == -math.inf for x in vals):
                    want = 2
                else:
                    want = 3
                assert cls[b, qt, kt] == want, (b, qt, kt)
    assert cls[0, 0, 0] == 0 and cls[0, 1, 1] == 1 and cls[0, 1, 2] == 1 and cls[1, 2, 4] == 0
    assert cls[1, 1, 0] == 3 and cls[1, 0, 2] == 3            # NaN / +inf make a tile "values"
    assert (cls == 2).sum() > 0                                # the random 0/-inf tiles are binary
    bits = oracle.tile_bits(m, BM, BN, cls)
    for b, qt, kt in zip(*np.nonzero(cls == 2)):
        for r in range(BM):
            i = qt * BM + r
            want = 0
            if i < Lq:
                for k in range(BN):
                    j = kt * BN + k
                    if j < Lk and m[b, 0, i, j] == 0.0:
                        want += 2 ** k
            assert int(bits[b, qt, kt, r]) == want, (b, qt, kt, r)
    lists = oracle.tile_lists(cls)
    for b in range(B):
        for qt in range(3):
            idx, c = lists[b][qt]
            assert list(idx) == [kt for kt in range(5) if cls[b, qt, kt] != 0]
            assert all(c == cls[b, qt, idx])


OCCUPANCY_PINS = [pin_occupancy_brute_force]


# ---------------------------------------------------------------- backward

def _mask_with_dead_row(seed, B, Lq, Lk):
    m = _rand_mask(seed, B, Lq, Lk, p_masked=0.45)
    m[0, 0, Lq - 1, :] = NINF                      # one row sees nothing: constant 0 output
    return m


def pin_backward_finite_differences():
    """Central differences of the (separately pinned) forward oracle: for
    f = sum(dout * out), df/dx at every entry of q, k_nope, k_rope and v."""
    q, kn, kr, v = _rand(40, 2, 2, 3, 5, dn=4, dr=3, dv=3)
    mask = _mask_with_dead_row(40, 2, 3, 5)
    dout = np.random.default_rng(41).standard_normal((2, 2, 3, 3))
    scale = 0.41
    grads = oracle.mla_attention_backward(q, kn, kr, v, mask, dout, scale)
    args = [q, kn, kr, v]
    eps = 1e-6
    for slot, g in enumerate(grads):
        x = args[slot]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[slot], am[slot] = xp, xm
            fp = (dout * oracle.mla_attention(*ap, mask, scale)).sum()
            fm = (dout * oracle.mla_attention(*am, mask, scale)).sum()
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=f"input {slot}")


def pin_backward_matches_torch_autograd():
    """torch.autograd (fp64, CPU) through scaled_dot_product_attention on explicit
    keys [k_nope | k_rope broadcast to every head]; rows with a finite score only
    (the library's softmax of an all -inf row is NaN, not the 0 this reading uses)."""
    import torch
    import torch.nn.functional as F
    B, H, Lq, Lk, dn, dr, dv = 2, 3, 9, 14, 16, 8, 12
    q, kn, kr, v = _rand(42, B, H, Lq, Lk, dn=dn, dr=dr, dv=dv)
    mask = _rand_mask(42, B, Lq, Lk)
    dout = np.random.default_rng(43).standard_normal((B, H, Lq, dv))
    scale = 24 ** -0.5
    tq, tkn, tkr, tv = (torch.tensor(a, requires_grad=True) for a in (q, kn, kr, v))
    k = torch.cat([tkn, tkr[:, None].expand(B, H, Lk, dr)], dim=-1)
    out = F.scaled_dot_product_attention(tq, k, tv, attn_mask=torch.from_numpy(mask), scale=scale)
    out.backward(torch.from_numpy(dout))
    got = oracle.mla_attention_backward(q, kn, kr, v, mask, dout, scale)
    for g, t in zip(got, (tq, tkn, tkr, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=0, atol=1e-11)


def pin_backward_invariants():
    """Softmax rows sum to 1, so the gradient rows of s sum to 0: the key
    gradients sum to 0 over the keys, and the value gradients sum to the
    output gradient of the rows that see anything.  A dead row passes nothing."""
    B, H, Lq, Lk = 2, 2, 6, 11
    q, kn, kr, v = _rand(44, B, H, Lq, Lk)
    mask = _mask_with_dead_row(44, B, Lq, Lk)
    dout = np.random.default_rng(45).standard_normal((B, H, Lq, v.shape[-1]))
    dq, dkn, dkr, dv = oracle.mla_attention_backward(q, kn, kr, v, mask, dout, 0.3)
    np.testing.assert_allclose(dkn.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dkr.sum(axis=1), 0.0, atol=1e-12)
    live = np.isfinite(mask).any(axis=-1)[:, 0]                  # [B, Lq]
    want_dv = (dout * live[:, None, :, None]).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), want_dv, atol=1e-12)
    assert not live[0, Lq - 1] and np.all(dq[0, :, Lq - 1] == 0.0)
    # per-head restriction: the same slices, and the rope gradient of one head
    one = oracle.mla_attention_backward(q, kn, kr, v, mask, dout, 0.3, heads=[1])
    np.testing.assert_allclose(one[0][:, 1], dq[:, 1], atol=0)
    np.testing.assert_allclose(one[3][:, 1], dv[:, 1], atol=0)
    zero = oracle.mla_attention_backward(q, kn, kr, v, mask, dout, 0.3, heads=[0])
    np.testing.assert_allclose(one[2] + zero[2], dkr, atol=1e-12)


def pin_logsumexp_normalises_the_forward():
    """exp(s - lse) over explicitly formed scores sums to 1 per live row and,
    applied to v, reproduces the forward oracle; dead rows have lse = -inf."""
    B, H, Lq, Lk, dn = 2, 2, 5, 9, 8
    q, kn, kr, v = _rand(46, B, H, Lq, Lk, dn=dn)
    mask = _mask_with_dead_row(46, B, Lq, Lk)
    lse = oracle.logsumexp_rows(q, kn, kr, mask, 0.37)
    out = oracle.mla_attention(q, kn, kr, v, mask, 0.37)
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                s = [0.37 * (float(np.dot(q[b, h, i, :dn], kn[b, h, j])) + float(np.dot(q[b, h, i, dn:], kr[b, j])))
                     + mask[b, 0, i, j] for j in range(Lk)]
                if all(x == NINF for x in s):
                    assert lse[b, h, i] == NINF
                    continue
                p = [math.exp(x - lse[b, h, i]) for x in s]
                assert abs(sum(p) - 1.0) < 1e-12
                np.testing.assert_allclose(np.dot(p, v[b, h]), out[b, h, i], atol=1e-12)


# ---------------------------------------------------------------- projections

def _brute_rms(row, gamma, eps):
    ms = sum(float(x) * float(x) for x in row) / len(row)
    return [float(x) / math.sqrt(ms + eps) * float(g) for x, g in zip(row, gamma)]


def pin_rms_norm():
    """Constant rows, a pure-Python loop, and torch's rms_norm (fp64, CPU)."""
    import torch
    rng = np.random.default_rng(70)
    g = rng.standard_normal(5)
    for c in (2.0, -0.5):
        out = oracle.rms_norm(np.full((1, 5), c), g, 0.25)
        np.testing.assert_allclose(out, c / math.sqrt(c * c + 0.25) * g[None], atol=1e-14)
    x = rng.standard_normal((3, 4, 7))
    gam = rng.standard_normal(7)
    out = oracle.rms_norm(x, gam, 0.3)
    for i in range(3):
        for j in range(4):
            np.testing.assert_allclose(out[i, j], _brute_rms(x[i, j], gam, 0.3), atol=1e-13)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (7,), weight=torch.from_numpy(gam), eps=0.3)
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-13)


def pin_context_project_brute_force():
    rng = np.random.default_rng(71)
    B, ctx, K, Hd = 2, 3, 5, 4
    th = rng.standard_normal((B, ctx, K))
    w = rng.standard_normal((Hd, K))
    g = rng.standard_normal(Hd)
    out = oracle.context_project(th, w, g, 0.2)
    for b in range(B):
        for t in range(ctx):
            y = [sum(th[b, t, k] * w[n, k] for k in range(K)) for n in range(Hd)]
            np.testing.assert_allclose(out[b, t], _brute_rms(y, g, 0.2), atol=1e-12)


def pin_q_project_brute_force():
    """Head-major output: q[b,h,t,d] uses row h*Dqk + d of q_b_proj."""
    rng = np.random.default_rng(72)
    B, L, Hd, Rq, H, Dqk = 2, 3, 5, 6, 2, 3
    x = rng.standard_normal((B, L, Hd))
    wa = rng.standard_normal((Rq, Hd))
    ga = rng.standard_normal(Rq)
    wb = rng.standard_normal((H * Dqk, Rq))
    q = oracle.q_project(x, wa, ga, 0.1, wb, H)
    assert q.shape == (B, H, L, Dqk)
    for b in range(B):
        for t in range(L):
            qa = _brute_rms([sum(x[b, t, k] * wa[r, k] for k in range(Hd)) for r in range(Rq)], ga, 0.1)
            for h in range(H):
                for d in range(Dqk):
                    want = sum(qa[r] * wb[h * Dqk + d, r] for r in range(Rq))
                    assert abs(q[b, h, t, d] - want) < 1e-11, (b, h, t, d)


def pin_kv_project_brute_force():
    """Context rows first, then noise; latent = the first R outputs (normed),
    k_rope = the last Dr (not normed); per head [k_nope | v] rows of kv_b_proj."""
    rng = np.random.default_rng(73)
    B, ctx, L, Hd, R, Dr, H, Dn, Dv = 2, 2, 3, 5, 4, 2, 2, 2, 3
    ch = rng.standard_normal((B, ctx, Hd))
    nh = rng.standard_normal((B, L, Hd))
    wa = rng.standard_normal((R + Dr, Hd))
    g = rng.standard_normal(R)
    wb = rng.standard_normal((H * (Dn + Dv), R))
    kn, kr, v = oracle.kv_project(ch, nh, wa, g, 0.15, wb, H, R, Dn, Dv)
    assert kn.shape == (B, H, ctx + L, Dn) and kr.shape == (B, ctx + L, Dr) and v.shape == (B, H, ctx + L, Dv)
    for b in range(B):
        for t in range(ctx + L):
            hrow = ch[b, t] if t < ctx else nh[b, t - ctx]
            c = [sum(hrow[k] * wa[n, k] for k in range(Hd)) for n in range(R + Dr)]
            np.testing.assert_allclose(kr[b, t], c[R:], atol=1e-12)
            lat = _brute_rms(c[:R], g, 0.15)
            for h in range(H):
                for d in range(Dn):
                    assert abs(kn[b, h, t, d] - sum(lat[r] * wb[h * (Dn + Dv) + d, r] for r in range(R))) < 1e-11
                for d in range(Dv):
                    assert abs(v[b, h, t, d] - sum(lat[r] * wb[h * (Dn + Dv) + Dn + d, r] for r in range(R))) < 1e-11
    kn0, kr0, v0 = oracle.kv_project(None, nh, wa, g, 0.15, wb, H, R, Dn, Dv)
    np.testing.assert_allclose(kn0, kn[:, :, ctx:], atol=1e-12)
    np.testing.assert_allclose(kr0, kr[:, ctx:], atol=1e-12)


PROJECTION_PINS = [pin_rms_norm, pin_context_project_brute_force, pin_q_project_brute_force,
                   pin_kv_project_brute_force]

# ---------------------------------------------------------------- GQA draft (yarn RoPE, qk-norm)

def pin_yarn_limits():
    """factor 1 is plain RoPE; otherwise the first pairs keep 1/theta^(2i/d), the last
    are divided by the factor, and the ratio in between never decreases."""
    d, base = 64, 10000.0
    plain = 1.0 / base ** (np.arange(0, d, 2) / d)
    np.testing.assert_allclose(oracle.yarn_inv_freq(d, base, 1.0, 4096, 32, 1), plain, rtol=1e-15)
    inv = oracle.yarn_inv_freq(d, base, 8.0, 4096, 32, 1)
    ratio = plain / inv
    assert abs(ratio[0] - 1.0) < 1e-15 and abs(ratio[-1] - 8.0) < 1e-12
    assert np.all(np.diff(ratio) >= -1e-12) and (ratio == 1.0).sum() >= 2 and (abs(ratio - 8.0) < 1e-12).sum() >= 2
    assert abs(oracle.yarn_mscale(1.0, 0.7) - 1.0) < 1e-15
    assert abs(oracle.yarn_mscale(math.e, 1.0) - 1.1) < 1e-15


def _rotations(j, d, theta, orig):
    """Turns pair j makes over orig positions at its unscaled frequency theta^(-2j/d)."""
    return orig * theta ** (-2.0 * j / d) / (2.0 * math.pi)


def pin_yarn_ntk_by_parts():
    """yarn's frequency split, from its defining rule (YaRN paper, section 3.2,
    "NTK-by-parts"; the MAX page's DFlashKimiK25DraftConfig names the Deepseek-yarn
    variant through rope_scaling): a pair that turns at least beta_fast times over
    the original context keeps theta^(-2j/d); a pair that turns at most beta_slow
    times is divided by factor; pairs in between are blended with a weight linear
    in the pair index between the first and last pair of the two kinds.

    Hand-derived case (the GQA draft's rope settings: d 128, theta 5e4, factor 32,
    original context 4096, beta_fast 32, beta_slow 1).  Pair j turns
    r_j = 4096 * 5e4^(-j/64) / (2 pi) times, so r_j = beta at
    j = 128 ln(4096 / (2 pi beta)) / (2 ln 5e4):
      beta 32: ln(20.37183) = 3.014153 -> j = 128 * 3.014153 / 21.639557 = 17.829
      beta 1:  ln(651.8986) = 6.479889 -> j = 128 * 6.479889 / 21.639557 = 38.329
    Pair 17 turns 36.81 times (kept), pair 18 31.09 (on the ramp), pair 38 1.057
    (on the ramp), pair 39 0.893 (divided).  The ramp runs from pair 17 (weight 0)
    to pair 39 (weight 1) in steps of 1/22, so pair 20 is e (1 - 3/22) + e/32 * 3/22
    = e * 611/704 and pair 30 is e (1 - 13/22) + e/32 * 13/22 = e * 301/704,
    e = 5e4^(-j/64)."""
    d, th, fac, orig = 128, 50000.0, 32.0, 4096
    inv = oracle.yarn_inv_freq(d, th, fac, orig, 32, 1)
    e = lambda j: th ** (-j / 64.0)   # noqa: E731
    assert abs(inv[17] / e(17) - 1.0) < 1e-14 and abs(inv[39] * 32.0 / e(39) - 1.0) < 1e-14
    assert inv[18] < e(18) * (1.0 - 1e-3) and inv[38] > e(38) / 32.0 * (1.0 + 1e-3)
    assert abs(inv[18] / (e(18) * (21.0 / 22.0 + 1.0 / 704.0)) - 1.0) < 1e-14
    assert abs(inv[20] / (e(20) * 611.0 / 704.0) - 1.0) < 1e-14
    assert abs(inv[30] / (e(30) * 301.0 / 704.0) - 1.0) < 1e-14
    # the rule itself, over several settings whose boundaries fall between pairs
    for d, th, fac, orig, bf, bs in ((128, 50000.0, 32.0, 4096, 32, 1), (64, 10000.0, 8.0, 4096, 32, 1),
                                     (128, 10000.0, 40.0, 4096, 32, 1), (96, 1e6, 4.0, 8192, 16, 2),
                                     (32, 500.0, 4.0, 256, 8, 1)):
        inv = oracle.yarn_inv_freq(d, th, fac, orig, bf, bs)
        ext = th ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        w = (ext - inv) / (ext - ext / fac)            # blend weight of the divided frequency
        r = np.array([_rotations(j, d, th, orig) for j in range(d // 2)])
        assert np.all((np.abs(w) < 1e-12) == (r >= bf)), (d, th, fac, orig)
        assert np.all((np.abs(w - 1.0) < 1e-12) == (r <= bs)), (d, th, fac, orig)
        mid = np.nonzero((r < bf) & (r > bs))[0]
        lo, hi = mid[0] - 1, mid[-1] + 1               # last kept pair, first divided pair
        np.testing.assert_allclose(w[mid], (mid - lo) / (hi - lo), rtol=1e-12, atol=1e-13)
    # an independent implementation: transformers' yarn initialiser (fp32)
    try:
        import torch
        from transformers import PretrainedConfig
        from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    except ImportError:
        return
    for d, th, fac, orig, bf, bs in ((128, 50000.0, 32.0, 4096, 32, 1), (64, 10000.0, 8.0, 4096, 32, 1),
                                     (16, 500.0, 4.0, 64, 8, 1)):
        rp = {"rope_type": "yarn", "rope_theta": th, "factor": fac, "original_max_position_embeddings": orig,
              "beta_fast": bf, "beta_slow": bs, "mscale": 0.707, "mscale_all_dim": 1.0}
        cfg = PretrainedConfig(head_dim=d, hidden_size=4 * d, num_attention_heads=4,
                               max_position_embeddings=int(orig * fac), rope_parameters=rp, rope_theta=th)
        hf_inv, hf_att = ROPE_INIT_FUNCTIONS["yarn"](cfg, torch.device("cpu"))
        np.testing.assert_allclose(oracle.yarn_inv_freq(d, th, fac, orig, bf, bs), hf_inv.double().numpy(),
                                   rtol=1e-6)
        assert abs(oracle.yarn_mscale(fac, 0.707) / oracle.yarn_mscale(fac, 1.0) - hf_att) < 1e-12


def pin_rope_properties():
    """Dimension i pairs with i + d/2; rotation keeps the norm; the product of a
    rotated query and key depends only on their position difference."""
    rng = np.random.default_rng(74)
    d = 16
    inv = oracle.yarn_inv_freq(d, 500.0, 4.0, 64, 8, 1)
    for i in (0, 3, d // 2 - 1):
        e = np.zeros(d)
        e[i] = 1.0
        out = oracle.rope(e[None], [37], inv)[0]
        want = np.zeros(d)
        want[i] = math.cos(37 * inv[i])
        want[i + d // 2] = math.sin(37 * inv[i])
        np.testing.assert_allclose(out, want, atol=1e-14)
    x = rng.standard_normal((5, d))
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(x, np.arange(5) * 101, inv), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n, sh in ((5, 2, 40), (0, 17, 1000)):
        a = oracle.rope(q[None], [m], inv)[0] @ oracle.rope(k[None], [n], inv)[0]
        b = oracle.rope(q[None], [m + sh], inv)[0] @ oracle.rope(k[None], [n + sh], inv)[0]
        assert abs(a - b) < 1e-11
    np.testing.assert_allclose(oracle.rope(x, [0] * 5, inv, 1.5), 1.5 * x, atol=1e-14)


def pin_gqa_matches_torch_sdpa():
    """PyTorch's attention (fp64, CPU) with the KV heads repeated over their query
    group and a key-length mask per batch row."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(75)
    B, Hq, Hkv, Lq, Lk, d = 2, 6, 2, 5, 11, 8
    q = rng.standard_normal((B, Hq, Lq, d))
    k = rng.standard_normal((B, Hkv, Lk, d))
    v = rng.standard_normal((B, Hkv, Lk, d))
    lens = [11, 7]
    mask = np.zeros((B, 1, Lq, Lk))
    mask[1, :, :, 7:] = -np.inf
    kr = torch.from_numpy(k).repeat_interleave(3, dim=1)
    vr = torch.from_numpy(v).repeat_interleave(3, dim=1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), kr, vr, attn_mask=torch.from_numpy(mask),
                                         scale=0.3).numpy()
    np.testing.assert_allclose(oracle.gqa_attention(q, k, v, lens, 0.3), ref, atol=1e-12)


def _gqa_case(seed, B=2, Lc=7, bs=3, hidden=8, Hq=4, Hkv=2, d=8):
    rng = np.random.default_rng(seed)
    return dict(ctx=rng.standard_normal((B, Lc, hidden)), blk=rng.standard_normal((B, bs, hidden)),
                wq=rng.standard_normal((Hq * d, hidden)) * 0.3, wk=rng.standard_normal((Hkv * d, hidden)) * 0.3,
                wv=rng.standard_normal((Hkv * d, hidden)) * 0.3, gq=1 + 0.1 * rng.standard_normal(d),
                gk=1 + 0.1 * rng.standard_normal(d), inv=oracle.yarn_inv_freq(d, 100.0, 2.0, 16, 4, 1),
                Hq=Hq, Hkv=Hkv, d=d, B=B, Lc=Lc, bs=bs)


def pin_forward_block_equals_whole_sequence():
    """With ctx_len = Lc, a block over the materialised context equals attention
    over the K/V materialised from the whole [context | block] sequence (positions
    continue across the boundary, context first); cached keys past ctx_len[b]
    are never read; the block's queries come from the q chain at those positions."""
    c = _gqa_case(76)
    kc, vc = oracle.materialize(c["ctx"], c["wk"], c["wv"], c["gk"], 0.1, c["Hkv"], c["inv"], 1.2)
    out = oracle.forward_block(c["blk"], c["wq"], c["wk"], c["wv"], c["gq"], c["gk"], 0.1, c["Hq"], c["Hkv"],
                               kc, vc, [c["Lc"]] * c["B"], c["inv"], 1.2)
    whole = np.concatenate([c["ctx"], c["blk"]], axis=1)
    kw, vw = oracle.materialize(whole, c["wk"], c["wv"], c["gk"], 0.1, c["Hkv"], c["inv"], 1.2)
    L = c["Lc"] + c["bs"]
    qw, _ = oracle.materialize(whole, c["wq"], c["wq"], c["gq"], 0.1, c["Hq"], c["inv"], 1.2)
    want = oracle.gqa_attention(qw[:, :, c["Lc"]:], kw, vw, [L] * c["B"], c["d"] ** -0.5)
    np.testing.assert_allclose(out, want, atol=1e-12)
    # a shorter context in row 1: garbage past ctx_len is ignored, positions restart at ctx_len
    kg, vg = kc.copy(), vc.copy()
    kg[1, :, 4:] = 1e3
    vg[1, :, 4:] = -1e3
    out2 = oracle.forward_block(c["blk"], c["wq"], c["wk"], c["wv"], c["gq"], c["gk"], 0.1, c["Hq"], c["Hkv"],
                                kg, vg, [c["Lc"], 4], c["inv"], 1.2)
    whole1 = np.concatenate([c["ctx"][1:2, :4], c["blk"][1:2]], axis=1)
    kw1, vw1 = oracle.materialize(whole1, c["wk"], c["wv"], c["gk"], 0.1, c["Hkv"], c["inv"], 1.2)
    qw1, _ = oracle.materialize(whole1, c["wq"], c["wq"], c["gq"], 0.1, c["Hq"], c["inv"], 1.2)
    want1 = oracle.gqa_attention(qw1[:, :, 4:], kw1, vw1, [4 + c["bs"]], c["d"] ** -0.5)
    np.testing.assert_allclose(out2[1:2], want1, atol=1e-12)
    np.testing.assert_allclose(out2[0], out[0], atol=0)


def pin_materialize_brute_force():
    """k = RoPE(RMSNorm(x W_k^T per head)), v = x W_v^T, written out with loops."""
    c = _gqa_case(77, B=1, Lc=4, hidden=5, Hkv=2, d=4)
    k, v = oracle.materialize(c["ctx"], c["wk"], c["wv"], c["gk"], 0.2, 2, c["inv"], 1.0)
    d = 4
    for t in range(4):
        x = c["ctx"][0, t]
        for h in range(2):
            raw = [sum(x[j] * c["wk"][h * d + e, j] for j in range(5)) for e in range(d)]
            nk = _brute_rms(raw, c["gk"], 0.2)
            for e in range(d):
                ang = t * c["inv"][e % (d // 2)]
                partner = -nk[e + d // 2] if e < d // 2 else nk[e - d // 2]
                assert abs(k[0, h, t, e] - (nk[e] * math.cos(ang) + partner * math.sin(ang))) < 1e-12
                assert abs(v[0, h, t, e] - sum(x[j] * c["wv"][h * d + e, j] for j in range(5))) < 1e-12


GQA_PINS = [pin_yarn_limits, pin_yarn_ntk_by_parts, pin_rope_properties, pin_gqa_matches_torch_sdpa,
            pin_forward_block_equals_whole_sequence, pin_materialize_brute_force]

BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_matches_torch_autograd,
                 pin_backward_invariants, pin_logsumexp_normalises_the_forward]

ALL_PINS = ATTENTION_PINS + EXPAND_PINS + OCCUPANCY_PINS + BACKWARD_PINS + PROJECTION_PINS + GQA_PINS
