"""The MHA/GQA draft (materialise the context into the bf16 cache, then a block
over cache + itself) on the GPU against the fp64 oracle (oracle.materialize /
forward_block / rope / yarn_inv_freq).

Tolerance, from the arithmetic: bf16 inputs, fp32 accumulation; the chain rounds
to bf16 at the projection, the normalised value, its product with the weight and
the rotated value (K), and the probabilities and output (attention) -- each a
relative 2^-9.  Bound: 1e-2 on ||got - ref|| / ||ref|| per tensor, 5e-2 * max|ref|
per element.  The rotation angles are formed in fp64 on the GPU, so positions up
to the cache length add no error of their own.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import gqa as ogqa
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2
REL_MAX = 5e-2


def say(msg):
    print(f"[gpu-gqa] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _check(name, got, ref):
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else got
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  {name}: rel_fro={rel:.2e} max_err/max_ref={mx:.2e}")
    assert np.all(np.isfinite(g)), name
    assert rel <= REL_FRO and mx <= REL_MAX, name


def _run(dev, p, ctx_len):
    B, Hkv, Lmax, Hq = p["B"], p["Hkv"], p["Lmax"], p["Hq"]
    kc, vc = mla.gqa_new_cache(B, Hkv, Lmax, dev)
    kc.fill_(float("nan"))                        # rows the kernels must never read
    vc.fill_(float("nan"))
    mla.gqa_materialize(p["ctx_hidden"].to(dev), p["w_k"].to(dev), p["w_v"].to(dev), p["g_k"].to(dev), p["eps"],
                        p["rope"], kc, vc)
    torch.cuda.synchronize()
    k_mat, v_mat = kc.clone(), vc.clone()
    out = mla.gqa_forward_block(p["blk_hidden"].to(dev), p["w_q"].to(dev), p["w_k"].to(dev), p["w_v"].to(dev),
                                p["g_q"].to(dev), p["g_k"].to(dev), p["eps"], p["rope"], kc, vc,
                                torch.as_tensor(ctx_len, dtype=torch.int32).to(dev), Hq)
    torch.cuda.synchronize()
    return k_mat, v_mat, kc, vc, out


def _oracle_inv(p):
    th, fac, orig, bf, bsl, ms, msa = p["rope"]
    return oracle.yarn_inv_freq(p["d"], th, fac, int(orig), bf, bsl), oracle.yarn_mscale(fac, ms) / oracle.yarn_mscale(fac, msa)


CASES = [
    # B, Lc, bs, hidden, Hq, Hkv, ctx_len (None: drawn), Lmax extra
    ("gqa4_ragged", 2, 150, 8, 256, 8, 2, [150, 70], 0),
    ("mha_bs16", 1, 300, 16, 128, 4, 4, [300], 8),
    ("gqa4_bs16_no_ctx", 2, 64, 16, 192, 8, 2, [0, 64], 0),
    ("gqa8_bs8_clamped", 2, 200, 8, 160, 16, 2, [200, 5000], 0),
    ("long", 1, 4100, 16, 256, 8, 2, [4100], 0),
    ("split_k_projections", 2, 300, 16, 2048, 8, 2, [300, 111], 0),   # hidden 2048: K split across workgroups
    ("large_tile_materialize", 1, 16384, 16, 1024, 32, 8, [16384], 0),  # 16384 x 1024 cache projection: 256-wide tiles
]


@pytest.mark.parametrize("case", list(range(len(CASES))))
def test_gqa_materialize_and_block(dev, case):
    name, B, Lc, bs, hidden, Hq, Hkv, ctx_len, extra = CASES[case]
    p = W.gqa_inputs(90 + case, B, Lc, bs, hidden, Hq, Hkv, ctx_len=ctx_len)
    p["Lmax"] += extra
    Lmax = p["Lmax"]
    say(f"{name}: B={B} Lc={Lc} bs={bs} hidden={hidden} Hq={Hq} Hkv={Hkv} ctx_len={ctx_len} Lmax={Lmax}")
    k_mat, v_mat, kc, vc, out = _run(dev, p, ctx_len)
    inv, ms = _oracle_inv(p)
    rk, rv = oracle.materialize(p["ctx_hidden"], p["w_k"], p["w_v"], p["g_k"], p["eps"], Hkv, inv, ms)
    _check("k cache", k_mat[:, :, :Lc], rk)
    _check("v cache", v_mat[:, :, :, :Lc], rv.transpose(0, 1, 3, 2))
    clamped = np.minimum(np.maximum(np.asarray(ctx_len), 0), Lmax - bs)
    # the oracle reads the context it materialised itself, truncated to each row's length
    ref = oracle.forward_block(p["blk_hidden"], p["w_q"], p["w_k"], p["w_v"], p["g_q"], p["g_k"], p["eps"], Hq, Hkv,
                               rk, rv, np.minimum(clamped, Lc), inv, ms) if np.all(clamped <= Lc) else None
    if ref is not None:
        _check("block out", out, ref)
    # the block's own k / v were appended at the (clamped) context length
    from oracle.projection import linear, rms_norm
    x = oracle.gqa._heads(linear(p["blk_hidden"], p["w_k"]), Hkv)
    for b in range(B):
        c = int(clamped[b])
        pos = c + np.arange(bs)
        kb = ogqa.rope(rms_norm(x[b], p["g_k"], p["eps"]), pos, inv, ms)
        vb = oracle.gqa._heads(linear(p["blk_hidden"], p["w_v"]), Hkv)[b]
        _check(f"appended k row {b}", kc[b, :, c:c + bs], kb)
        _check(f"appended v row {b}", vc[b, :, :, c:c + bs], vb.transpose(0, 2, 1))


def test_gqa_clamped_context_matches_oracle(dev):
    """A ctx_len past the cache is clamped to Lmax - bs: the block then attends to
    the cache rows the materialise call wrote beyond the shorter context."""
    B, Lc, bs, hidden, Hq, Hkv = 1, 120, 8, 128, 4, 2
    p = W.gqa_inputs(99, B, Lc, bs, hidden, Hq, Hkv, ctx_len=[10 ** 6])
    p["Lmax"] = 128                                  # Lmax - bs = 120 = Lc
    k_mat, v_mat, kc, vc, out = _run(dev, p, [10 ** 6])
    inv, ms = _oracle_inv(p)
    rk, rv = oracle.materialize(p["ctx_hidden"], p["w_k"], p["w_v"], p["g_k"], p["eps"], Hkv, inv, ms)
    ref = oracle.forward_block(p["blk_hidden"], p["w_q"], p["w_k"], p["w_v"], p["g_q"], p["g_k"], p["eps"], Hq, Hkv,
                               rk, rv, [120], inv, ms)
    _check("block out (clamped)", out, ref)
