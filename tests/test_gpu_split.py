"""The bf16 forward split over key ranges (small work grids) against the fp64 oracle.

A split run is the pages' softmax regrouped: each run normalises its own keys
and the runs are merged with weights exp(lse_run - lse) in a fixed order.  The
tolerances are those of the unsplit bf16 path (max 1.5e-2, mean 1e-3 on out;
4e-3 on lse, from the bf16 rounding of the probabilities it sums); split and
unsplit outputs are also compared with each other (they round the
probabilities relative to different stabilisers).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16_MAX = 1.5e-2
TOL_BF16_MEAN = 1e-3
LSE_TOL = 4e-3


def say(msg):
    print(f"[gpu-split] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _runs(B, H, Lq, Lk):
    """Number of key runs the library picks (from the workspace size it asks for)."""
    extra = mla.attn_split_workspace_bytes(B, H, Lq, Lk) - mla.attn_workspace_bytes(B, Lq, Lk)
    if extra <= 0:
        return 1
    per_run = B * H * Lq * (128 * 2 + 4)   # bf16 output + f32 normaliser per row and run
    return int(round(extra / per_run))


def _check_out(got, ref, what):
    d = np.abs(got.to("cpu", torch.float64).numpy() - ref)
    say(f"  {what}: max|err|={d.max():.3e} mean|err|={d.mean():.3e}")
    assert d.max() <= TOL_BF16_MAX and d.mean() <= TOL_BF16_MEAN, what


def _split_vs_unsplit(a, b):
    # The probabilities are rounded to bf16 relative to each run's own stabiliser
    # instead of the whole row's, so a weight moves by up to 2^-8 of itself and an
    # output by up to 2^-8 * max|v| (about 2e-2 for N(0,1) values), on average far less.
    d = (a.float() - b.float()).abs()
    say(f"  split vs unsplit: max|diff|={d.max().item():.3e} mean={d.mean().item():.3e}")
    assert d.max().item() <= 1.5e-2 and d.mean().item() <= 5e-4


def _dense(anchors, ctx, bs, dtype="bf16"):
    return W.additive_mask(W.visibility(np.asarray(anchors, dtype=np.int64), ctx, ctx, bs), dtype)


@pytest.mark.parametrize("case", ["expand_shape", "one_block_long_ctx", "few_tiles_empty_runs"])
def test_split_forward_and_lse(dev, case):
    rng = np.random.default_rng({"expand_shape": 70, "one_block_long_ctx": 71, "few_tiles_empty_runs": 72}[case])
    if case == "expand_shape":          # 2 x 2 q-tiles x 16 heads over 36 k-tiles
        B, H, ctx, A, bs = 2, 16, 2048, 16, 16
        anchors = W.draw_anchors(rng, B, A, ctx)
    elif case == "one_block_long_ctx":  # one draft block per row, 8 heads, 130 k-tiles
        B, H, ctx, A, bs = 1, 8, 8192, 1, 16
        anchors = np.array([[8000]])
    else:                               # every anchor early: most rows see 1-2 k-tiles, most runs empty
        B, H, ctx, A, bs = 1, 8, 8192, 4, 16
        anchors = np.array([[3, 20, 41, 90]])
    Lq, Lk = A * bs, ctx + A * bs
    S = _runs(B, H, Lq, Lk)
    say(f"{case}: B={B} H={H} Lq={Lq} Lk={Lk} runs={S}")
    assert S > 1
    q, kn, kr, v = W.random_attention_inputs(73, B, H, Lq, Lk, dtype="bf16")
    mask = _dense(anchors, ctx, bs)
    qd, knd, krd, vd, md = (t.to(dev) for t in (q, kn, kr, v, mask))
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(qd, knd, krd, vd, md, lse=lse)
    lse1 = torch.empty_like(lse)
    out1 = mla.mla_attn(qd, knd, krd, vd, md, lse=lse1, split_keys=False)
    blk = mla.mla_attn_blocks(qd, knd, krd, vd, torch.from_numpy(anchors.astype(np.int32)).to(dev), bs, ctx)
    torch.cuda.synchronize()
    assert torch.equal(out, blk)                 # the block-structure map splits the same way
    _split_vs_unsplit(out, out1)
    # each lse sums probabilities rounded to bf16 (relative error <= 2^-9 each, all
    # terms positive: the sum and so exp(lse) within 2^-9), relative to different
    # stabilisers in the two calls: they differ by at most about 2 * 2^-9
    dl = (lse - lse1).abs().max().item()
    say(f"  lse split vs unsplit: max|diff|={dl:.2e}")
    assert dl <= 4e-3
    _check_out(out, oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5), "split out vs oracle")
    want = oracle.logsumexp_rows(q, kn, kr, mask, 192 ** -0.5)
    lerr = np.abs(lse.cpu().double().numpy() - want).max()
    say(f"  lse max|err|={lerr:.2e}")
    assert lerr <= LSE_TOL


def test_split_dead_rows_and_no_mask(dev):
    """A row with no visible key returns 0 and lse -inf through the merge; without
    a mask every run is a full list of k-tiles."""
    B, H, Lq, Lk = 1, 4, 64, 1500
    q, kn, kr, v = W.random_attention_inputs(74, B, H, Lq, Lk, dtype="bf16")
    vis = np.ones((B, 1, Lq, Lk), dtype=bool)
    vis[0, 0, 5] = False                       # dead row
    vis[0, 0, 6, :1400] = False                # sees only the last run's keys
    mask = W.additive_mask(vis[:, 0], "f32")
    assert _runs(B, H, Lq, Lk) > 1
    qd, knd, krd, vd, md = (t.to(dev) for t in (q, kn, kr, v, mask))
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(qd, knd, krd, vd, md, lse=lse)
    nm = mla.mla_attn(qd, knd, krd, vd, None)
    nm1 = mla.mla_attn(qd, knd, krd, vd, None, split_keys=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0, :, 5]).item() == 0
    assert bool(torch.isneginf(lse[0, :, 5]).all())
    _check_out(out, oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5), "split, dead rows")
    _split_vs_unsplit(nm, nm1)
    _check_out(nm, oracle.mla_attention(q, kn, kr, v, None, 192 ** -0.5), "split, no mask")


def test_split_backward_matches_unsplit_forward(dev):
    """The backward takes out / lse of a split forward: gradients within the
    oracle's tolerance of those it takes from the unsplit forward."""
    rng = np.random.default_rng(75)
    B, H, ctx, A, bs = 1, 8, 1500, 8, 16
    anchors = W.draw_anchors(rng, B, A, ctx)
    Lq, Lk = A * bs, ctx + A * bs
    assert _runs(B, H, Lq, Lk) > 1
    q, kn, kr, v = (t.to(dev) for t in W.random_attention_inputs(76, B, H, Lq, Lk, dtype="bf16"))
    dout = W.normal(rng, (B, H, Lq, 128), 1.0, "bf16").to(dev)
    m = _dense(anchors, ctx, bs).to(dev)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(q, kn, kr, v, m, lse=lse)
    lse1 = torch.empty_like(lse)
    out1 = mla.mla_attn(q, kn, kr, v, m, lse=lse1, split_keys=False)
    g = mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse)
    g1 = mla.mla_attn_bwd(q, kn, kr, v, m, out1, dout, lse1)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk_nope", "dk_rope", "dv"), g, g1):
        d = (x.float() - y.float()).abs().max().item()
        ref = y.float().abs().max().item()
        say(f"  {name}: split vs unsplit max|diff|={d:.3e} (max|g|={ref:.3e})")
        assert d <= 2e-2 * ref + 1e-3
