"""The seeded input generator: shapes, anchors, mask structure (CPU only)."""
import numpy as np
import pytest
import torch

from dflash_block_draft_amd import workloads as W


def _check_mask_rule(wl):
    m = wl.mask.float().numpy()[:, 0]
    assert m.shape == (wl.B, wl.Lq, wl.Lk)
    assert set(np.unique(m).tolist()) <= {0.0, -np.inf}
    for b in range(wl.B):
        anc = wl.anchors[b]
        assert np.all(np.diff(anc) > 0), "anchors sorted and distinct"
        assert anc.min() >= 1 and anc.max() <= wl.ctx_valid - 1
        for i in range(0, wl.Lq, max(1, wl.Lq // 37)):
            j = i // wl.block_size
            vis = np.isfinite(m[b, i])
            want_ctx = (np.arange(wl.ctx) <= anc[j]) & (np.arange(wl.ctx) < wl.ctx_valid)
            assert np.array_equal(vis[:wl.ctx], want_ctx)
            noise = np.zeros(wl.Lq, bool)
            noise[j * wl.block_size:(j + 1) * wl.block_size] = True
            assert np.array_equal(vis[wl.ctx:], noise), "a block sees exactly its own keys"


def test_config0_shapes_and_rule():
    wl = W.config(0)
    assert (wl.B, wl.H, wl.Lq, wl.Lk) == (1, 4, 32, 96)
    assert wl.q.dtype == torch.float32 and wl.mask.dtype == torch.float32
    assert wl.q.shape == (1, 4, 32, 192) and wl.k_nope.shape == (1, 4, 96, 128)
    assert wl.k_rope.shape == (1, 96, 64) and wl.v.shape == (1, 4, 96, 128)
    _check_mask_rule(wl)


def test_config1_expand_inputs():
    wl = W.config(1)
    assert (wl.B, wl.H, wl.Lq, wl.Lk) == (2, 16, 256, 2304)
    assert wl.latent.shape == (2, 2304, 512) and wl.w_kv_b.shape == (16 * 256, 512)
    assert wl.k_nope is None and wl.v is None
    assert wl.latent.dtype == torch.bfloat16 and wl.mask.dtype == torch.float32
    assert abs(wl.w_kv_b.float().std().item() - 0.02) < 1e-3
    _check_mask_rule(wl)


@pytest.mark.parametrize("bs", [8, 32])
def test_config3_padding_and_rows(bs):
    wl = W.config(3, block_size=bs)
    assert wl.ctx_valid == 4096 - 204 and wl.Lq == 32 * bs
    m = wl.mask.float().numpy()[:, 0]
    assert np.all(m[:, :, wl.ctx_valid:wl.ctx] == -np.inf), "padding masked for every query"
    assert np.all(np.isfinite(m).any(-1)), "no row fully masked"
    _check_mask_rule(wl)


def test_workload_is_deterministic():
    a, b = W.config(0), W.config(0)
    assert torch.equal(a.q, b.q) and torch.equal(a.mask, b.mask)
    assert np.array_equal(a.anchors, b.anchors)


def test_visible_flops_definition():
    wl = W.config(0)
    pairs = int(np.isfinite(wl.mask.float().numpy()).sum())
    assert W.visible_flops(wl.mask, wl.B, wl.H, wl.Lq, wl.Lk) == pairs * 4 * 640


def test_bench_keys():
    import bench
    assert bench.split_key("3b") == ("3b", "")
    assert bench.split_key("3a") == ("3a", "")
    assert bench.split_key("4b") == ("4", "b")
    assert bench.split_key("2s") == ("2", "s")
    assert bench.split_key("3bs") == ("3b", "s")
