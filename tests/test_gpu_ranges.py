"""Reads past the end of a tensor come back as zeros (gfx950 GPU required).

The kernels copy key/value, query and operand tiles through buffer resources
whose range is the tensor (one (batch, head) slice of it): a ragged or phantom
tile reads rows past the end, and those reads must return zeros rather than
whatever memory follows.  Here every tensor the kernels read is a view at the
start of a larger allocation whose remainder is NaN, with B * H = 1 so no other
head's data sits behind a slice.  The allocation covers everything a tile could
reach, so nothing can fault; if a read past the end were not zeroed, a NaN would
reach the output.  Shapes are ragged in both the query and the key axis.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

# past the end of every view: more than a 128-row q-tile and a 64-key tile of the
# widest row (192 bf16 values), and than a padded 128-key backward block
PAD = 1 << 20


def say(msg):
    print(f"[gpu-ranges] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _nan_tail(t: torch.Tensor, dev) -> torch.Tensor:
    """t copied to the start of a NaN-filled device buffer (integers: a huge value), as a
    contiguous view."""
    n = t.numel()
    fill = float("nan") if t.dtype.is_floating_point else (1 << 30)
    buf = torch.full((n + PAD,), fill, dtype=t.dtype, device=dev)
    view = buf[:n].view(t.shape)
    view.copy_(t.to(dev))
    assert view.data_ptr() == buf.data_ptr() and view.is_contiguous()
    return view


def _case(seed, Lq, Lk, ctx, bs):
    wl = W.custom(seed=seed, B=1, H=1, ctx=ctx, A=Lq // bs, bs=bs, dtype="bf16", mask_dtype="bf16")
    assert wl.Lq == Lq and wl.Lk == Lk
    return wl


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_forward_reads_past_the_end_as_zero(dev, split, masked):
    wl = _case(81, Lq=165, Lk=165 + 1000, ctx=1000, bs=15)   # q-tile 2 ragged, last k-tile 13 wide
    say(f"forward Lq={wl.Lq} Lk={wl.Lk} split={split} masked={masked}")
    q, kn, kr, v = (_nan_tail(t, dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v))
    m = _nan_tail(wl.mask, dev) if masked else None
    lse = _nan_tail(torch.zeros((1, 1, wl.Lq), dtype=torch.float32), dev)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale, lse=lse, split_keys=split)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse.cpu()).all()
    ref = oracle.mla_attention(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask if masked else None, wl.scale)
    d = np.abs(o.double().numpy() - ref)
    say(f"  max|err|={d.max():.3e} mean|err|={d.mean():.3e}")
    assert d.max() <= 1.5e-2 and d.mean() <= 1e-3


def test_block_forward_reads_past_the_end_as_zero(dev):
    wl = _case(82, Lq=160, Lk=160 + 777, ctx=777, bs=16)
    q, kn, kr, v = (_nan_tail(t, dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v))
    anchors = _nan_tail(torch.from_numpy(wl.anchors.astype(np.int32)), dev)
    out = mla.mla_attn_blocks(q, kn, kr, v, anchors, wl.block_size, wl.ctx, None, wl.scale)
    torch.cuda.synchronize()
    ref = oracle.mla_attention(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, wl.scale)
    d = np.abs(out.cpu().double().numpy() - ref)
    say(f"block forward Lq={wl.Lq} Lk={wl.Lk}: max|err|={d.max():.3e} mean|err|={d.mean():.3e}")
    assert np.isfinite(d).all() and d.max() <= 1.5e-2 and d.mean() <= 1e-3


def test_backward_reads_past_the_end_as_zero(dev):
    wl = _case(83, Lq=165, Lk=165 + 1000, ctx=1000, bs=15)
    dout = W.normal(np.random.default_rng(84), (1, 1, wl.Lq, 128), 1.0, "bf16")
    q, kn, kr, v, m, do = (_nan_tail(t, dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, dout))
    lse = torch.empty((1, 1, wl.Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale, lse=lse)
    out_v, lse_v = _nan_tail(out, dev), _nan_tail(lse, dev)
    grads = mla.mla_attn_bwd(q, kn, kr, v, m, out_v, do, lse_v, wl.scale)
    torch.cuda.synchronize()
    ref = oracle.mla_attention_backward(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, dout, wl.scale)
    for nm, g, r in zip(("dq", "dk_nope", "dk_rope", "dv"), grads, ref):
        gg = g.cpu().double().numpy()
        assert np.isfinite(gg).all(), nm
        rel = np.linalg.norm(gg - r) / np.linalg.norm(r)
        say(f"backward {nm}: rel_fro={rel:.2e}")
        assert rel <= 1e-2, nm


def test_expand_reads_past_the_end_as_zero(dev):
    rng = np.random.default_rng(85)
    B, Lk, R, H = 1, 77, 512, 2
    lat = W.normal(rng, (B, Lk, R), 1.0, "bf16")
    w = W.normal(rng, (H * 256, R), 0.05, "bf16")
    kn, v = mla.latent_expand(_nan_tail(lat, dev), _nan_tail(w, dev), H)
    torch.cuda.synchronize()
    ref_kn, ref_v = oracle.latent_expand(lat, w, H, 128, 128)
    for nm, got, ref in (("k_nope", kn, ref_kn), ("v", v, ref_v)):
        g = got.cpu().double().numpy()
        assert np.isfinite(g).all(), nm
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6), nm
