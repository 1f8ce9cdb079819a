"""The block-structure entry points on the GPU: the tile map computed from
(anchors, ctx_valid, block_size) equals the occupancy pass over the dense
0 / -inf mask of the same visibility and the oracle's classification of it,
and the attention equals the dense-mask call bitwise and the oracle within the
bf16 tolerance."""
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


def say(msg):
    print(f"[gpu-blocks] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _i32(x, dev):
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(dev)


def _structures():
    """(name, anchors [B, A], ctx, ctx_valid [B] or None, block_size): the drawn
    recipe plus degenerate structures -- anchors below 0 and beyond the context,
    ctx_valid of 0, beyond ctx and below an anchor, no context at all, block
    sizes that do not divide a tile, ragged last tiles."""
    rng = np.random.default_rng(40)
    yield "drawn", W.draw_anchors(rng, 2, 9, 430), 452, np.array([430, 452]), 16
    yield "odd", np.array([[-7, 0, 3, 199, 200, 5000, -1]]), 200, None, 24
    yield "cv_edge", np.array([[5, 60, 130, 131], [-2, 0, 64, 2 ** 31 - 1]]), 131, np.array([0, 2 ** 30]), 5
    yield "cv_below", np.array([[10, 100, 300], [7, 8, 9]]), 320, np.array([50, -4]), 32
    yield "no_ctx", np.array([[0, 0, 0]]), 0, None, 48
    yield "bs1", rng.integers(-2, 140, size=(1, 70)), 130, np.array([129]), 1


def _dense_mask(anchors, ctx, ctx_valid, bs):
    cv = ctx if ctx_valid is None else ctx_valid
    return W.additive_mask(W.visibility(np.asarray(anchors, dtype=np.int64), ctx, cv, bs), "bf16")


def _map(ws, B, Lq, Lk):
    tm = mla.tile_map_view(ws, B, Lq, Lk)
    return {k: v.cpu().numpy() for k, v in tm.items() if isinstance(v, torch.Tensor)}


@pytest.mark.parametrize("case", list(range(6)))
def test_block_tile_map_equals_dense(dev, case):
    name, anchors, ctx, cv, bs = list(_structures())[case]
    B, A = anchors.shape
    Lq, Lk = A * bs, ctx + A * bs
    say(f"block tile map {name}: B={B} A={A} bs={bs} ctx={ctx} ctx_valid={cv}")
    ws = mla.block_occupancy(_i32(anchors, dev), bs, ctx, None if cv is None else _i32(cv, dev))
    mask = _dense_mask(anchors, ctx, cv, bs)
    wd = mla.mask_occupancy(mask.to(dev))
    torch.cuda.synchronize()
    got, ref = _map(ws, B, Lq, Lk), _map(wd, B, Lq, Lk)
    want = oracle.tile_classes(mask, mla.TILE_M, mla.TILE_N)
    assert np.array_equal(got["classes"], want)
    for k in ("classes", "counts", "order"):
        assert np.array_equal(got[k], ref[k]), k
    sel = want == 2
    gb, rb = got["bits"].view(np.uint64), ref["bits"].view(np.uint64)
    assert np.array_equal(gb[sel], rb[sel])
    assert np.array_equal(gb[sel], oracle.tile_bits(mask, mla.TILE_M, mla.TILE_N, want)[sel])
    counts = got["counts"]
    for b in range(B):
        for qt in range(counts.shape[1]):
            n = counts[b, qt]
            assert np.array_equal(got["lists"][b, qt, :n], ref["lists"][b, qt, :n])


@pytest.mark.parametrize("case", list(range(6)))
def test_block_attention_small(dev, case):
    name, anchors, ctx, cv, bs = list(_structures())[case]
    B, A = anchors.shape
    Lq, Lk, H = A * bs, ctx + A * bs, 3
    say(f"block attention {name}: B={B} H={H} Lq={Lq} Lk={Lk}")
    q, kn, kr, v = W.random_attention_inputs(41 + case, B, H, Lq, Lk, dtype="bf16")
    mask = _dense_mask(anchors, ctx, cv, bs)
    qd, knd, krd, vd, md = (t.to(dev) for t in (q, kn, kr, v, mask))
    out = mla.mla_attn_blocks(qd, knd, krd, vd, _i32(anchors, dev), bs, ctx,
                              None if cv is None else _i32(cv, dev))
    dense = mla.mla_attn(qd, knd, krd, vd, md)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    ref = oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5)
    d = np.abs(out.to("cpu", torch.float64).numpy() - ref)
    say(f"  max|err|={d.max():.3e} mean|err|={d.mean():.3e}")
    assert d.max() <= TOL_BF16_MAX and d.mean() <= TOL_BF16_MEAN


@pytest.mark.parametrize("idx,bs", [(2, None), (3, 8), (3, 32), (4, None)])
def test_block_attention_workloads(dev, idx, bs):
    """The bf16 workloads at full size: bitwise equal to the dense-mask call,
    whose whole output the parity tests compare with the oracle."""
    wl = W.config(idx, bs)
    say(f"{wl.name}: block structure vs dense mask")
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    anchors = _i32(wl.anchors, dev)
    cv = _i32(np.full(wl.B, wl.ctx_valid), dev)
    out = mla.mla_attn_blocks(q, kn, kr, v, anchors, wl.block_size, wl.ctx, cv, wl.scale)
    dense = mla.mla_attn(q, kn, kr, v, m, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)


def test_block_reuse_tile_map(dev):
    rng = np.random.default_rng(42)
    B, A, bs, ctx, H = 2, 10, 16, 700, 4
    anchors = W.draw_anchors(rng, B, A, ctx)
    Lq, Lk = A * bs, ctx + A * bs
    q, kn, kr, v = (t.to(dev) for t in W.random_attention_inputs(43, B, H, Lq, Lk, dtype="bf16"))
    ad = _i32(anchors, dev)
    ws = mla.new_workspace(B, Lq, Lk, dev)
    a = mla.mla_attn_blocks(q, kn, kr, v, ad, bs, ctx, workspace=ws)
    q2 = torch.flip(q, dims=[1]).contiguous()
    b = mla.mla_attn_blocks(q2, kn, kr, v, ad, bs, ctx, workspace=ws, reuse_tile_map=True)
    # (the map-only workspace gives unsplit calls; the fresh calls match that)
    c = mla.mla_attn_blocks(q2, kn, kr, v, ad, bs, ctx, split_keys=False)
    a2 = mla.mla_attn_blocks(q, kn, kr, v, ad, bs, ctx, split_keys=False)
    torch.cuda.synchronize()
    assert torch.equal(b, c)
    assert torch.equal(a, a2)


def test_block_structure_training_step(dev):
    """The block-structure map on a backward workspace drives the forward with lse
    and the backward through the map alone (no mask): bitwise equal to the same
    calls with the dense 0 / -inf mask."""
    rng = np.random.default_rng(44)
    B, A, bs, ctx, H = 2, 9, 16, 500, 3
    anchors = W.draw_anchors(rng, B, A, ctx)
    Lq, Lk = A * bs, ctx + A * bs
    q, kn, kr, v = (t.to(dev) for t in W.random_attention_inputs(45, B, H, Lq, Lk, dtype="bf16"))
    dout = W.normal(rng, (B, H, Lq, 128), 1.0, "bf16").to(dev)
    mask = _dense_mask(anchors, ctx, None, bs).to(dev)
    ws = mla.new_bwd_workspace(B, H, Lq, Lk, dev)
    mla.block_occupancy(_i32(anchors, dev), bs, ctx, workspace=ws)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    # (unsplit forwards throughout: whether a call may split its key list depends
    # on its workspace, and split and unsplit outputs differ by bf16 rounding)
    out = mla.mla_attn(q, kn, kr, v, None, lse=lse, workspace=ws, reuse_tile_map=True, split_keys=False)
    g = mla.mla_attn_bwd(q, kn, kr, v, None, out, dout, lse, workspace=ws, reuse_tile_map=True)
    lse_d = torch.empty_like(lse)
    out_d = mla.mla_attn(q, kn, kr, v, mask, lse=lse_d, split_keys=False)
    g_d = mla.mla_attn_bwd(q, kn, kr, v, mask, out_d, dout, lse_d)
    blk = mla.mla_attn_blocks(q, kn, kr, v, _i32(anchors, dev), bs, ctx, split_keys=False)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(out, blk) and torch.equal(lse, lse_d)
    for x, y in zip(g, g_d):
        assert torch.equal(x, y)
