"""The projections around the attention on the GPU against the fp64 oracle
(oracle.context_project / q_project / kv_project).

Tolerance, from the arithmetic: inputs are exact bf16; products accumulate in
fp32; each chain rounds to bf16 at most four times (the Linear output, the
normalised value, its product with the norm weight, the final Linear output),
each a relative 2^-9, and the row statistics come from the rounded outputs.
Bound: 1e-2 on ||got - ref|| / ||ref|| per tensor and 5e-2 * max|ref| per
element; a wrong row source, split, head layout or missing norm is off by O(1).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2
REL_MAX = 5e-2


def say(msg):
    print(f"[gpu-proj] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _check(name, got, ref):
    g = got.detach().to("cpu", torch.float64).numpy()
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  {name}: rel_fro={rel:.2e} max_err/max_ref={mx:.2e}")
    assert np.all(np.isfinite(g)), name
    assert rel <= REL_FRO and mx <= REL_MAX, name


def _small(seed, B, ctx, Lq, H, hidden, q_lora_rank, n_layers=3):
    return W.projection_inputs(seed, B, ctx, Lq, H, hidden=hidden, q_lora_rank=q_lora_rank,
                               n_target_layers=n_layers)


@pytest.mark.parametrize("shape", [(2, 100, 40, 2, 256, 256), (1, 257, 33, 3, 384, 384)])
def test_context_project(dev, shape):
    B, ctx, Lq, H, hidden, rq = shape
    p = _small(80, B, ctx, Lq, H, hidden, rq)
    say(f"context_project B={B} ctx={ctx} K_in={p['target_hidden'].shape[2]} hidden={hidden}")
    out = mla.context_project(p["target_hidden"].to(dev), p["w_fc"].to(dev), p["g_hidden"].to(dev), p["eps"])
    torch.cuda.synchronize()
    _check("context", out, oracle.context_project(p["target_hidden"], p["w_fc"], p["g_hidden"], p["eps"]))


@pytest.mark.parametrize("shape", [(2, 100, 70, 3, 160, 256), (1, 64, 129, 2, 256, 384),
                                   (2, 16, 70, 2, 2048, 256)])   # few output tiles, long K: split-K
def test_q_project(dev, shape):
    B, ctx, Lq, H, hidden, rq = shape
    p = _small(81, B, ctx, Lq, H, hidden, rq)
    say(f"q_project B={B} Lq={Lq} hidden={hidden} q_lora_rank={rq} H={H}")
    q = mla.q_project(p["noise_hidden"].to(dev), p["w_q_a"].to(dev), p["g_q"].to(dev), p["eps"],
                      p["w_q_b"].to(dev), H)
    torch.cuda.synchronize()
    assert tuple(q.shape) == (B, H, Lq, 192)
    _check("q", q, oracle.q_project(p["noise_hidden"], p["w_q_a"], p["g_q"], p["eps"], p["w_q_b"], H))


@pytest.mark.parametrize("shape", [(2, 150, 40, 2, 128), (1, 0, 37, 3, 96), (1, 300, 100, 2, 224)])
def test_kv_project(dev, shape):
    B, ctx, Lq, H, hidden = shape
    p = _small(82, B, ctx, Lq, H, hidden, 128)
    say(f"kv_project B={B} ctx={ctx} Lq={Lq} hidden={hidden} H={H}")
    ch = p["ctx_hidden"].to(dev) if ctx > 0 else None
    kn, kr, v = mla.kv_project(ch, p["noise_hidden"].to(dev), p["w_kv_a"].to(dev), p["g_kv"].to(dev), p["eps"],
                               p["w_kv_b"].to(dev), H, p["R"])
    torch.cuda.synchronize()
    rkn, rkr, rv = oracle.kv_project(p["ctx_hidden"] if ctx > 0 else None, p["noise_hidden"], p["w_kv_a"],
                                     p["g_kv"], p["eps"], p["w_kv_b"], H, p["R"])
    _check("k_nope", kn, rkn)
    _check("k_rope", kr, rkr)
    _check("v", v, rv)


def test_projections_full_size_then_attention(dev):
    """The training-shaped workload's sizes (B 1, ctx 8192, 64 anchors x 16, 64
    heads) with hidden 7168 and q_lora_rank 1536: all three chains against the
    oracle (context on a 1024-token slice), then the attention on their outputs
    equals the attention on the oracle's outputs rounded to bf16 within the
    attention tolerance."""
    wl = W.config(2)
    p = W.projection_inputs(83, 1, wl.ctx, wl.Lq, wl.H)
    say("full-size projections: hidden 7168, q_lora_rank 1536, R 512, H 64")
    th = p["target_hidden"][:, :1024]
    ctxo = mla.context_project(th.to(dev), p["w_fc"].to(dev), p["g_hidden"].to(dev), p["eps"])
    q = mla.q_project(p["noise_hidden"].to(dev), p["w_q_a"].to(dev), p["g_q"].to(dev), p["eps"],
                      p["w_q_b"].to(dev), wl.H)
    kn, kr, v = mla.kv_project(p["ctx_hidden"].to(dev), p["noise_hidden"].to(dev), p["w_kv_a"].to(dev),
                               p["g_kv"].to(dev), p["eps"], p["w_kv_b"].to(dev), wl.H, p["R"])
    torch.cuda.synchronize()
    _check("context[:1024]", ctxo, oracle.context_project(th, p["w_fc"], p["g_hidden"], p["eps"]))
    rq = oracle.q_project(p["noise_hidden"], p["w_q_a"], p["g_q"], p["eps"], p["w_q_b"], wl.H)
    _check("q", q, rq)
    rkn, rkr, rv = oracle.kv_project(p["ctx_hidden"], p["noise_hidden"], p["w_kv_a"], p["g_kv"], p["eps"],
                                     p["w_kv_b"], wl.H, p["R"])
    _check("k_nope", kn, rkn)
    _check("k_rope", kr, rkr)
    _check("v", v, rv)
    m = wl.mask.to(dev)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev)  # noqa: E731
    ref = mla.mla_attn(bf(rq), bf(rkn), bf(rkr), bf(rv), m, wl.scale)
    torch.cuda.synchronize()
    d = (out.float() - ref.float()).abs()
    say(f"  attention on projected vs oracle-projected inputs: max={d.max().item():.3e} mean={d.mean().item():.3e}")
    assert d.mean().item() <= 1e-2


def test_context_project_large_tile(dev):
    """Enough output tiles for the 256 x 256 tile with its three-stage copy pipeline
    (4096 rows x 4096 outputs, K 4096)."""
    p = W.projection_inputs(84, 1, 4096, 16, 2, hidden=4096, q_lora_rank=128, n_target_layers=1)
    say("context_project 4096 x 4096, K 4096 (large tile)")
    out = mla.context_project(p["target_hidden"].to(dev), p["w_fc"].to(dev), p["g_hidden"].to(dev), p["eps"])
    torch.cuda.synchronize()
    _check("context (large tile)", out, oracle.context_project(p["target_hidden"], p["w_fc"], p["g_hidden"], p["eps"]))
