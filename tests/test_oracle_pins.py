"""The fp64 oracle against closed forms, invariants, brute force and a library routine."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_scale_is_q_head_dim_inverse_sqrt():
    # dspark page, KimiK3DSparkAttention attributes: scaling = q_head_dim ** -0.5,
    # q_head_dim = qk_nope_head_dim + qk_rope_head_dim
    from dflash_block_draft_amd import workloads as W
    wl = W.config(0)
    assert wl.scale == pytest.approx((128 + 64) ** -0.5, rel=0, abs=0)


def test_oracle_on_workload0_rows_sum_and_bounds():
    """Config-0 sanity: outputs are convex combinations of visible v rows."""
    from dflash_block_draft_amd import workloads as W
    wl = W.config(0)
    out = oracle.mla_attention(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, wl.scale)
    v = wl.v.double().numpy()
    vis = np.isfinite(wl.mask.double().numpy()[:, 0])
    for b in range(wl.B):
        for h in range(wl.H):
            for i in range(wl.Lq):
                sel = v[b, h, vis[b, i]]
                assert np.all(out[b, h, i] <= sel.max(0) + 1e-12)
                assert np.all(out[b, h, i] >= sel.min(0) - 1e-12)
