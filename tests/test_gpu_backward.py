"""The attention backward and the forward's row log-normaliser on the GPU,
against the fp64 oracle (oracle.mla_attention_backward / logsumexp_rows).

Tolerances, from the arithmetic.  The lse of the bf16 forward sums fp32
probabilities, or on its exact-path steps their bf16 roundings (relative error
<= 2^-9 each, all positive, so the sum too), so |lse - exact| <= ~2^-9: bound
4e-3.  The backward rounds p and ds to
bf16 as MFMA operands and every output to bf16 (each a relative 2^-9
perturbation of a term or a result), recomputes p from that lse (another
relative 2^-9) and takes D from the bf16
output; the gradients therefore carry a few units of 2^-9 relative error
norm-wise: bound 1e-2 on ||got - ref|| / ||ref|| per tensor, and 2e-2 * max|ref|
on any single element (measured: about 2.5e-3 and at most 7e-3).  A wrong
index, sign, missing term or scale gives errors of order 1.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

LSE_TOL_BF16 = 4e-3
LSE_TOL_F32 = 1e-5
REL_FRO = 1e-2
REL_MAX = 2e-2


def say(msg):
    print(f"[gpu-bwd] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _general_mask(rng, B, Lq, Lk, dtype):
    """Finite values, -inf entries, and one row that sees nothing."""
    m = rng.standard_normal((B, 1, Lq, Lk)).astype(np.float32)
    m[rng.random(m.shape) < 0.4] = -np.inf
    m[0, 0, Lq // 2, :] = -np.inf
    return torch.from_numpy(m).to(dtype)


def _grad_check(name, got, ref):
    g = got.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / max(nrm, 1e-30)
    mx = err.max() / max(np.abs(ref).max(), 1e-30)
    say(f"  {name}: rel_fro={rel:.2e} max_err/max_ref={mx:.2e}")
    assert np.all(np.isfinite(g)), name
    assert rel <= REL_FRO and mx <= REL_MAX, name


def _cases():
    rng = np.random.default_rng(50)
    wl = W.custom(seed=51, B=2, H=3, ctx=300, A=7, bs=16, dtype="bf16", mask_dtype="bf16")   # Lq 112, Lk 412
    yield "dflash_bf16mask", wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask
    wl = W.custom(seed=52, B=1, H=2, ctx=450, A=9, bs=16, dtype="bf16", mask_dtype="f32")    # Lq 144, Lk 594
    yield "dflash_f32mask_ragged", wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask
    q, kn, kr, v = W.random_attention_inputs(53, 2, 2, 150, 201, dtype="bf16")
    yield "general_values_dead_row", q, kn, kr, v, _general_mask(rng, 2, 150, 201, torch.float32)
    q, kn, kr, v = W.random_attention_inputs(54, 1, 3, 37, 70, dtype="bf16")
    yield "no_mask_tiny", q, kn, kr, v, None
    wl = W.custom(seed=55, B=1, H=2, ctx=700, A=12, bs=24, dtype="bf16", mask_dtype="bf16")  # Lq 288, Lk 988
    yield "dflash_bs24", wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask


def _forward_lse(dev, q, kn, kr, v, m, scale, ws=None):
    B, H, Lq, _ = q.shape
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(q, kn, kr, v, m, scale, lse=lse, workspace=ws)
    return out, lse


@pytest.mark.parametrize("case", list(range(5)))
def test_lse_and_backward_small(dev, case):
    name, q, kn, kr, v, m = list(_cases())[case]
    B, H, Lq, _ = q.shape
    Lk = kn.shape[2]
    scale = 192 ** -0.5
    say(f"{name}: B={B} H={H} Lq={Lq} Lk={Lk} mask={None if m is None else m.dtype}")
    dout = W.normal(np.random.default_rng(60 + case), (B, H, Lq, 128), 1.0, "bf16")
    qd, knd, krd, vd, dod = (t.to(dev) for t in (q, kn, kr, v, dout))
    md = None if m is None else m.to(dev)
    out, lse = _forward_lse(dev, qd, knd, krd, vd, md, scale)
    plain = mla.mla_attn(qd, knd, krd, vd, md, scale)
    grads = mla.mla_attn_bwd(qd, knd, krd, vd, md, out, dod, lse, scale)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)                       # writing lse changes nothing else
    want_lse = oracle.logsumexp_rows(q, kn, kr, m, scale)
    got_lse = lse.cpu().double().numpy()
    dead = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), dead)
    lerr = np.abs(got_lse[~dead] - want_lse[~dead]).max()
    say(f"  lse max|err|={lerr:.2e}")
    assert lerr <= LSE_TOL_BF16
    ref = oracle.mla_attention_backward(q, kn, kr, v, m, dout, scale)
    for nm, g, r in zip(("dq", "dk_nope", "dk_rope", "dv"), grads, ref):
        _grad_check(nm, g, r)
    if dead.any():                                       # a row that sees nothing passes no gradient
        b, h, i = np.argwhere(dead)[0]
        assert torch.count_nonzero(grads[0][b, h, i]).item() == 0


def test_lse_f32(dev):
    wl = W.config(0)
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    out, lse = _forward_lse(dev, q, kn, kr, v, m, wl.scale)
    torch.cuda.synchronize()
    want = oracle.logsumexp_rows(wl.q, wl.k_nope, wl.k_rope, wl.mask, wl.scale)
    err = np.abs(lse.cpu().double().numpy() - want).max()
    say(f"f32 lse max|err|={err:.2e}")
    assert err <= LSE_TOL_F32


def test_backward_deterministic_and_reuse(dev):
    wl = W.custom(seed=56, B=1, H=4, ctx=1000, A=16, bs=16, dtype="bf16", mask_dtype="bf16")
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    dout = W.normal(np.random.default_rng(57), (1, 4, wl.Lq, 128), 1.0, "bf16").to(dev)
    ws = mla.new_bwd_workspace(1, 4, wl.Lq, wl.Lk, dev)
    out, lse = _forward_lse(dev, q, kn, kr, v, m, wl.scale, ws=ws)
    a = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse, wl.scale, workspace=ws, reuse_tile_map=True)
    b = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse, wl.scale)
    c = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse, wl.scale)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(y, z)


def test_backward_config2(dev):
    """The training-shaped workload at full size against the full oracle."""
    wl = W.config(2)
    say(f"{wl.name}: backward vs oracle (all heads)")
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    dout = W.normal(np.random.default_rng(58), (wl.B, wl.H, wl.Lq, 128), 1.0, "bf16")
    out, lse = _forward_lse(dev, q, kn, kr, v, m, wl.scale)
    grads = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout.to(dev), lse, wl.scale)
    torch.cuda.synchronize()
    ref = oracle.mla_attention_backward(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, dout, wl.scale)
    for nm, g, r in zip(("dq", "dk_nope", "dk_rope", "dv"), grads, ref):
        _grad_check(nm, g, r)


def test_backward_config4(dev):
    """The long-context workload: dq, dk_nope and dv of three heads (all rows and
    keys) against the oracle, plus properties that hold at any size over every
    head -- the key gradients of every (b, h) sum to 0 over the keys, the value
    gradients sum to the sum of dout over the rows.  (dk_rope sums over all 32
    heads, so it is checked by the invariant here and against the oracle on the
    training-shaped workload.)"""
    wl = W.config(4)
    say(f"{wl.name}: backward vs oracle on heads 0, 13, 31, invariants on all")
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    dout = W.normal(np.random.default_rng(59), (wl.B, wl.H, wl.Lq, 128), 1.0, "bf16").to(dev)
    out, lse = _forward_lse(dev, q, kn, kr, v, m, wl.scale)
    dq, dkn, dkr, dv = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse, wl.scale)
    torch.cuda.synchronize()
    for t in (dq, dkn, dkr, dv):
        assert torch.isfinite(t.float()).all()
    sk = dkn.double().sum(dim=2)                       # [B, H, 128]
    scale_k = dkn.double().abs().sum(dim=2)
    assert (sk.abs() <= 2e-2 * scale_k + 1e-3).all()
    sr = dkr.double().sum(dim=1)
    assert (sr.abs() <= 2e-2 * dkr.double().abs().sum(dim=1) + 1e-3).all()
    sv = dv.double().sum(dim=2)
    want = dout.double().sum(dim=2)
    assert ((sv - want).abs() <= 2e-2 * dout.double().abs().sum(dim=2) + 1e-3).all()
    heads = [0, 13, 31]
    ref = oracle.mla_attention_backward(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, dout.cpu(), wl.scale,
                                        heads=heads)
    for nm, g, r in (("dq", dq, ref[0]), ("dk_nope", dkn, ref[1]), ("dv", dv, ref[3])):
        _grad_check(f"{nm} heads {heads}", g[:, heads], r[:, heads])


def test_backward_largest_key_count(dev):
    """The largest key count the backward takes, 5592383 (the padded k^T copy of
    one (batch, head) just under 2^31 bytes), one block of 16 queries whose
    anchor is 1000: 1001 context keys and the last 16 keys are visible, the last
    key tile is ragged.  Keys nobody sees get exactly zero gradients; the visible
    keys' gradients and dq match the oracle run on the visible keys alone (the
    other keys' probabilities are exactly 0)."""
    Lk, bs, anchor = 5592383, 16, 1000
    ctx = Lk - bs
    gen = torch.Generator(device=dev)
    gen.manual_seed(61)
    say(f"backward, largest key count: Lk={Lk}")
    q = torch.randn((1, 1, bs, 192), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((1, 1, Lk, 128), generator=gen, device=dev).to(torch.bfloat16)
    kr = torch.randn((1, Lk, 64), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((1, 1, Lk, 128), generator=gen, device=dev).to(torch.bfloat16)
    dout = torch.randn((1, 1, bs, 128), generator=gen, device=dev).to(torch.bfloat16)
    mask = torch.full((1, 1, bs, Lk), float("-inf"), dtype=torch.bfloat16, device=dev)
    mask[..., :anchor + 1] = 0
    mask[..., ctx:] = 0
    scale = 192 ** -0.5
    out, lse = _forward_lse(dev, q, kn, kr, v, mask, scale)
    dq, dkn, dkr, dv = mla.mla_attn_bwd(q, kn, kr, v, mask, out, dout, lse, scale)
    torch.cuda.synchronize()
    hidden = slice(anchor + 1, ctx)
    for t, nm in ((dkn[:, :, hidden], "dk_nope"), (dkr[:, hidden], "dk_rope"), (dv[:, :, hidden], "dv")):
        assert torch.count_nonzero(t).item() == 0, nm
    cols = torch.cat([torch.arange(anchor + 1), torch.arange(ctx, Lk)]).to(dev)
    ref = oracle.mla_attention_backward(q.cpu(), kn[:, :, cols].cpu(), kr[:, cols].cpu(), v[:, :, cols].cpu(),
                                        mask[..., cols].cpu(), dout.cpu(), scale)
    got = (dq, dkn[:, :, cols], dkr[:, cols], dv[:, :, cols])
    for nm, g, r in zip(("dq", "dk_nope", "dk_rope", "dv"), got, ref):
        _grad_check(nm, g, r)
    del q, kn, kr, v, dout, mask, out, lse, dq, dkn, dkr, dv, got
    torch.cuda.empty_cache()
