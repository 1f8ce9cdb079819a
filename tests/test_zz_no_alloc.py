"""dflash_mla_attn_no_alloc (the workspace-free attention for callers that cannot
allocate) against dflash_mla_attn with a workspace, through the C ABI: two calls
in a row on one GPU, the second on a smaller shape, so it runs on the scratch the
first one left behind (gfx950 GPU required)."""
import sys

import pytest
import torch

from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _pair(dev, wl):
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    out = torch.empty((wl.B, wl.H, wl.Lq, wl.Dv), dtype=q.dtype, device=dev)
    mla.mla_attn_no_alloc(q, kn, kr, v, m, wl.scale, out=out)
    want = mla.mla_attn(q, kn, kr, v, m, wl.scale, split_keys=False)
    torch.cuda.synchronize()
    return out, want


def test_no_alloc_matches_workspace_call_twice(dev):
    big = W.custom(seed=91, B=2, H=4, ctx=1500, A=20, bs=16, dtype="bf16", mask_dtype="bf16")   # Lq 320, Lk 1820
    small = W.custom(seed=92, B=1, H=2, ctx=300, A=5, bs=16, dtype="bf16", mask_dtype="f32")    # Lq 80, Lk 380
    for wl in (big, small):
        say(f"{wl.name}: B={wl.B} H={wl.H} Lq={wl.Lq} Lk={wl.Lk} mask={wl.mask_dtype}")
        out, want = _pair(dev, wl)
        d = (out.float() - want.float()).abs().max().item()
        say(f"  max|no_alloc - workspace call| = {d:.3e}")
        assert torch.equal(out, want)


def test_no_alloc_without_mask_and_too_large(dev):
    q, kn, kr, v = (t.to(dev) for t in W.random_attention_inputs(93, 1, 2, 64, 200, dtype="bf16"))
    out = torch.empty((1, 2, 64, 128), dtype=q.dtype, device=dev)
    mla.mla_attn_no_alloc(q, kn, kr, v, None, out=out)
    want = mla.mla_attn(q, kn, kr, v, None, split_keys=False)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    # a tile map past the scratch: rejected before anything is launched (tensors are
    # views of one small buffer; the call fails validation without touching them)
    B, Lq, Lk = 1, 128 * 64, 64 * 600
    assert mla.attn_workspace_bytes(B, Lq, Lk) > (32 << 20)
    lib = mla.load_library()
    st = lib.dflash_mla_attn_no_alloc(q.data_ptr(), kn.data_ptr(), kr.data_ptr(), v.data_ptr(), q.data_ptr() + 64,
                                      out.data_ptr(), B, 1, Lq, Lk, 128, 64, 128, 0.07, 1, 1, 0x4, None)
    assert st == 2, lib.dflash_last_error()
    say(f"  oversize: {lib.dflash_last_error().decode()}")
