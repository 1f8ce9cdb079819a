#!/usr/bin/env python3
"""Benchmark of the DFlash/DSpark draft MLA attention hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the mask-occupancy pass, then the fused bf16 MFMA
attention (and, for the workload that has one, the kv_b_proj latent
expansion before them).  The headline workload is the training-shaped one
(batch 1, context 8192, 64 anchors x block 16, 64 heads, bf16 q/k/v, bf16
mask); the long-context and block-size-sweep workloads and the expand
workload are timed the same way and reported under "secondary".

Metric: visible TFLOP/s = (finite-mask query-key pairs) x heads x (2*192 + 2*128)
divided by the step time, and its fraction of MI355X's published dense bf16
MFMA peak (2.5 PFLOP/s).  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "draft-attn visible TFLOP/s + % of MI355X bf16 MFMA peak (1 GPU)"
ATTN_SRC = os.path.join(ROOT, "dflash_block_draft_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--warm-seconds", type=float, default=0.5,
                   help="untimed busy time before each timed region, after the warmup steps (0 under a profiler)")
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="2", help="headline workload: 0,1,2,3a,3b,4")
    p.add_argument("--secondary", default="4,1,3a,3b,2s,4s,2b,4b,2p,gqa",
                   help="comma list, or 'none'; a trailing 's' takes the mask from the block "
                        "structure (anchors) instead of the dense tensor, a trailing 'b' times "
                        "the backward, a trailing 'p' the projections around the attention; 'gqa' "
                        "the MHA/GQA draft of the MAX page")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="run one plain device copy of this size (for HBM counter calibration)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="offline: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE run, "
                        "WRITE_SIZE run, both with --copy-calibration-mb) into HBM bytes per attention "
                        "launch for --workload, stored in profiles/attn_traffic.json; no GPU needed")
    return p.parse_args()


def split_key(key: str):
    """'3b' -> ('3b', ''), '4s' -> ('4', 's'), '3bb' -> ('3b', 'b'): workload, then mode suffix."""
    base = key[:2] if key.startswith("3") else key[:1]
    return base, key[len(base):]


def make_workload(key: str):
    from dflash_block_draft_amd import workloads as W
    if key == "gqa":
        return None
    key = split_key(key)[0]
    if key == "3a":
        return W.config(3, block_size=8)
    if key == "3b":
        return W.config(3, block_size=32)
    return W.config(int(key))


def describe(wl) -> str:
    return (f"{wl.name}: B={wl.B} H={wl.H} ctx={wl.ctx} anchors={wl.num_anchors} "
            f"block={wl.block_size} Lq={wl.Lq} Lk={wl.Lk} q/k/v={wl.dtype} mask={wl.mask_dtype}"
            + (" +kv_b_proj expand R=512" if wl.latent is not None else ""))


def kernel_sha() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


_SMI = {"handle": None, "tried": 0}


def _smi_handle():
    """amdsmi's handle of the first GPU, initialised once per process; an
    initialisation that fails (seen on the first attempt in a process) is tried
    again, a few times, on later calls."""
    while _SMI["handle"] is None and _SMI["tried"] < 5:
        _SMI["tried"] += 1
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            _SMI["handle"] = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            time.sleep(0.1)
    return _SMI["handle"]


class SclkSampler:
    """Samples the shader clock the driver reports from a thread while the GPU
    runs the warm-up and the timed steps: amdsmi's GPU metrics (the SMU's average
    GFX clock, else the mean of the current per-XCC clocks), else sysfs
    pp_dpm_sclk.  Readings below 500 MHz are idle or deep-sleep values, not the
    clock of a busy GPU, and are dropped; None where nothing usable is read."""

    def __init__(self, period_s: float = 0.005):
        import glob
        import threading
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.smi = _smi_handle()               # the ROCm SMI library, when present
        self.source = ("amdsmi GFX clock during the timed steps" if self.smi is not None
                       else "sysfs pp_dpm_sclk during the timed steps")
        self.period = period_s
        self.smi_failures = 0
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        if self.smi is not None:
            try:
                import amdsmi
                m = amdsmi.amdsmi_get_gpu_metrics_info(self.smi)
                v = m.get("average_gfxclk_frequency")
                if not isinstance(v, (int, float)) or v <= 0 or v >= 0xFFFF:
                    cur = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 0xFFFF]
                    v = sum(cur) / len(cur) if cur else None
                if v is not None:
                    self.source = "amdsmi GPU metrics GFX clock during warm-up and timed steps"
                    self.smi_failures = 0
                    return float(v)
            except Exception:
                pass
            try:
                import amdsmi
                info = amdsmi.amdsmi_get_clock_info(self.smi, amdsmi.AmdSmiClkType.GFX)
                self.smi_failures = 0
                return float(info["clk"])
            except Exception:
                # a failed read (seen for a while after initialisation) is retried
                # on the next sample, for as long as the sampler runs
                self.smi_failures += 1
                return None
        for path in self.files:
            try:
                for line in open(path):
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self.stop.is_set():
            v = self._read()
            if v is not None and v >= 500:
                self.samples.append(v)
            self.stop.wait(self.period)

    def __enter__(self):
        if self.files or self.smi is not None:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.thread.is_alive():
            self.thread.join()

    def summary(self):
        if not self.samples:
            if self.smi is None and not self.files:
                return None
            return {"samples": 0, "failed_reads": self.smi_failures, "source": self.source}
        s = self.samples
        return {"mean_MHz": round(sum(s) / len(s)), "min_MHz": round(min(s)), "max_MHz": round(max(s)),
                "samples": len(s), "source": self.source}


WARM = {"seconds": 0.5}     # set from --warm-seconds


def host_info() -> dict:
    try:
        aff = sorted(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = []
    runs, start = [], None
    for c in aff:                      # compress the affinity set into ranges
        if start is None:
            start = prev = c
        elif c == prev + 1:
            prev = c
        else:
            runs.append(f"{start}-{prev}" if prev > start else f"{start}")
            start = prev = c
    if start is not None:
        runs.append(f"{start}-{prev}" if prev > start else f"{start}")
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(aff), "affinity": ",".join(runs)}


def measure(wl, steps: int, warmup: int, structured: bool = False) -> dict:
    import torch
    from dflash_block_draft_amd import mla
    from dflash_block_draft_amd import workloads as W

    dev = torch.device("cuda:0")
    q, kr, m = (t.to(dev) for t in (wl.q, wl.k_rope, wl.mask))
    expand = wl.latent is not None
    if expand:
        lat, w = wl.latent.to(dev), wl.w_kv_b.to(dev)
        kn = torch.empty((wl.B, wl.H, wl.Lk, wl.Dn), dtype=q.dtype, device=dev)
        v = torch.empty((wl.B, wl.H, wl.Lk, wl.Dv), dtype=q.dtype, device=dev)
    else:
        kn, v = wl.k_nope.to(dev), wl.v.to(dev)
    ws = mla.new_workspace(wl.B, wl.Lq, wl.Lk, dev, H=wl.H)   # room for key-split partials on small grids
    extra = mla.attn_split_workspace_bytes(wl.B, wl.H, wl.Lq, wl.Lk) - mla.attn_workspace_bytes(wl.B, wl.Lq, wl.Lk)
    key_runs = 1 if wl.dtype != "bf16" or extra <= 0 else round(extra / (wl.B * wl.H * wl.Lq * (wl.Dv * 2 + 4)))
    anchors = torch.as_tensor(wl.anchors.astype("int32")).to(dev)
    ctx_valid = torch.full((wl.B,), wl.ctx_valid, dtype=torch.int32, device=dev)
    out = torch.empty((wl.B, wl.H, wl.Lq, wl.Dv), dtype=q.dtype, device=dev)
    vis_flops = W.visible_flops(wl.mask, wl.B, wl.H, wl.Lq, wl.Lk)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks):
        if expand:
            marks[0].record()
            mla.latent_expand(lat, w, wl.H, k_nope=kn, v=v)
        marks[1].record()
        if structured:
            mla.block_occupancy(anchors, wl.block_size, wl.ctx, ctx_valid, ws)
            marks[2].record()
            mla.mla_attn_blocks(q, kn, kr, v, anchors, wl.block_size, wl.ctx, ctx_valid, wl.scale,
                                out=out, workspace=ws, reuse_tile_map=True)
        else:
            mla.mask_occupancy(m, ws)
            marks[2].record()
            mla.mla_attn(q, kn, kr, v, m, wl.scale, out=out, workspace=ws, reuse_tile_map=True)
        marks[3].record()

    scratch = [ev() for _ in range(4)]
    for _ in range(warmup):
        step(scratch)
    torch.cuda.synchronize()
    # then keep the GPU busy for at least --warm-seconds so its clocks settle at
    # their sustained level before the timed steps (untimed)
    marks = [[ev() for _ in range(4)] for _ in range(steps)]
    start, end = ev(), ev()
    with SclkSampler() as sclk:
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < WARM["seconds"]:
            for _ in range(8):
                step(scratch)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for k in range(steps):
            step(marks[k])
        end.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = start.elapsed_time(end) / steps
    occ = sum(mk[1].elapsed_time(mk[2]) for mk in marks) / steps
    att = sum(mk[2].elapsed_time(mk[3]) for mk in marks) / steps
    att_min = min(mk[2].elapsed_time(mk[3]) for mk in marks)
    exp_ms = sum(mk[0].elapsed_time(mk[1]) for mk in marks) / steps if expand else None

    # Cold caches: a 512 MB write (more than the 256 MB Infinity Cache and the L2s)
    # before every call, outside the events; reported next to the warm figures.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = max(3, steps // 4)
    cmarks = [[ev() for _ in range(4)] for _ in range(n_cold)]
    for k in range(n_cold):
        flush.zero_()
        step(cmarks[k])
    torch.cuda.synchronize()
    first = 0 if expand else 1
    cold_ms = sum(mk[first].elapsed_time(mk[3]) for mk in cmarks) / n_cold
    cold_att = sum(mk[2].elapsed_time(mk[3]) for mk in cmarks) / n_cold
    del flush

    # tile statistics from the occupancy map of this mask
    tm = mla.tile_map_view(ws, wl.B, wl.Lq, wl.Lk)
    cls = tm["classes"].cpu()
    n = cls.numel()
    frac = {name: round(float((cls == c).sum()) / n, 4)
            for c, name in ((0, "empty"), (1, "zero"), (2, "binary"), (3, "general"))}
    esz = 2 if wl.dtype == "bf16" else 4
    mask_bytes = wl.mask.numel() * wl.mask.element_size()
    attn_bytes = (wl.q.numel() + wl.B * wl.H * wl.Lk * (wl.Dn + wl.Dv) + wl.k_rope.numel()
                  + wl.B * wl.H * wl.Lq * wl.Dv) * esz
    res = {
        "workload": wl.name,
        "mask_from": "block structure (anchors, ctx_valid)" if structured else "dense tensor",
        "shape": {"B": wl.B, "H": wl.H, "Lq": wl.Lq, "Lk": wl.Lk, "ctx": wl.ctx,
                  "anchors": wl.num_anchors, "block_size": wl.block_size},
        "visible_gflop": round(vis_flops / 1e9, 3),
        "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "tflops": round(vis_flops / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100.0 * vis_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "attn_kernel_ms": round(att, 4),
        "attn_kernel_ms_min": round(att_min, 4),
        "attn_kernel_tflops": round(vis_flops / (att * 1e-3) / 1e12, 2),
        "cold_ms_per_step": round(cold_ms, 4),
        "cold_attn_kernel_ms": round(cold_att, 4),
        "cold_tflops": round(vis_flops / (cold_ms * 1e-3) / 1e12, 2),
        "occupancy_ms": round(occ, 4),
        "occupancy_mask_GBs": None if structured else round(mask_bytes / (occ * 1e-3) / 1e9, 1),
        "key_runs": key_runs,
        "tile_fractions_128x64": frac,
        "attn_algorithmic_bytes": attn_bytes,
        "attn_GBs": round(attn_bytes / (att * 1e-3) / 1e9, 1),
        "attn_pct_hbm_peak": round(100.0 * attn_bytes / (att * 1e-3) / 8e12, 2),
        "mask_bytes": mask_bytes,
        "sclk": sclk.summary(),
    }
    if expand:
        xf = 2 * wl.B * wl.Lk * 512 * wl.H * (wl.Dn + wl.Dv)
        res["expand_ms"] = round(exp_ms, 4)
        res["expand_tflops"] = round(xf / (exp_ms * 1e-3) / 1e12, 2)
    del q, kr, m, kn, v, ws, out, anchors, ctx_valid
    if expand:
        del lat, w
    torch.cuda.empty_cache()
    return res


def measure_bwd(wl, steps: int, warmup: int) -> dict:
    """One step = the attention backward (prep, dK/dV, dQ, dk_rope reduction) given
    out and lse from a forward on the same workspace (its tile map is reused)."""
    import numpy as np
    import torch
    from dflash_block_draft_amd import mla
    from dflash_block_draft_amd import workloads as W

    dev = torch.device("cuda:0")
    q, kn, kr, v, m = (t.to(dev) for t in (wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask))
    dout = W.normal(np.random.default_rng(1000 + wl.seed), (wl.B, wl.H, wl.Lq, wl.Dv), 1.0, wl.dtype).to(dev)
    ws = mla.new_bwd_workspace(wl.B, wl.H, wl.Lq, wl.Lk, dev)
    lse = torch.empty((wl.B, wl.H, wl.Lq), dtype=torch.float32, device=dev)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale, workspace=ws, lse=lse)
    grads = (torch.empty_like(q), torch.empty_like(kn), torch.empty_like(kr), torch.empty_like(v))

    def step():
        mla.mla_attn_bwd(q, kn, kr, v, m, out, dout, lse, wl.scale, workspace=ws, reuse_tile_map=True,
                         grads=grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = sum(times) / steps
    pairs = W.visible_pairs(wl.mask)
    flops = pairs * wl.H * (2 * (wl.Dn + wl.Dr) * 3 + 2 * wl.Dv * 2)   # QK^T, dQ, dK (192) + dP, dV (128)
    res = {
        "workload": wl.name,
        "pass": "backward (dq, dk_nope, dk_rope, dv)",
        "visible_gflop": round(flops / 1e9, 3),
        "flop_basis": "visible pairs x heads x 1664 (QK^T, dP, dV, dK, dQ once each)",
        "ms_per_step": round(ms, 4),
        "ms_min": round(min(times), 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
    }
    del q, kn, kr, v, m, dout, ws, lse, out, grads
    torch.cuda.empty_cache()
    return res


def measure_proj(wl, steps: int, warmup: int) -> dict:
    """The projections around the attention at the workload's B, ctx, Lq and H
    with hidden 7168, q_lora_rank 1536, R 512 and four target layers into fc:
    context_project (fc + hidden_norm), q_project (Q-LoRA), kv_project
    (kv_a_proj + kv_a_layernorm + kv_b_proj).  Each is timed on its own."""
    import torch
    from dflash_block_draft_amd import mla
    from dflash_block_draft_amd import workloads as W

    dev = torch.device("cuda:0")
    p = W.projection_inputs(2000 + wl.seed, wl.B, wl.ctx, wl.Lq, wl.H)
    t = {k: (v.to(dev) if hasattr(v, "to") else v) for k, v in p.items()}
    B, ctx, Lq, H, hid, rq, R, Dr = wl.B, wl.ctx, wl.Lq, wl.H, p["hidden"], p["q_lora_rank"], p["R"], p["Dr"]
    Kin = t["target_hidden"].shape[2]
    Lk = ctx + Lq
    ctx_out = torch.empty((B, ctx, hid), dtype=torch.bfloat16, device=dev)
    q_out = torch.empty((B, H, Lq, 192), dtype=torch.bfloat16, device=dev)
    ws_c = torch.empty(mla.load_library().dflash_mla_projection_workspace_bytes(B * ctx, hid), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(mla.load_library().dflash_mla_projection_workspace_bytes(B * Lq, rq), dtype=torch.uint8, device=dev)
    ws_kv = torch.empty(mla.load_library().dflash_mla_projection_workspace_bytes(B * Lk, R), dtype=torch.uint8, device=dev)
    calls = {
        "context_project": (lambda: mla.context_project(t["target_hidden"], t["w_fc"], t["g_hidden"], p["eps"],
                                                        out=ctx_out, workspace=ws_c),
                            2.0 * B * ctx * Kin * hid),
        "q_project": (lambda: mla.q_project(t["noise_hidden"], t["w_q_a"], t["g_q"], p["eps"], t["w_q_b"], H,
                                            out=q_out, workspace=ws_q),
                      2.0 * B * Lq * (hid * rq + rq * H * 192)),
        "kv_project": (lambda: mla.kv_project(t["ctx_hidden"], t["noise_hidden"], t["w_kv_a"], t["g_kv"], p["eps"],
                                              t["w_kv_b"], H, R, workspace=ws_kv),
                       2.0 * B * Lk * (hid * (R + Dr) + R * H * 256)),
    }
    res = {"workload": wl.name, "pass": "projections (hidden 7168, q_lora_rank 1536, R 512, fc from 4 layers)",
           "parts": {}}
    tot_ms = tot_f = 0.0
    for name, (fn, flops) in calls.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        tot_ms += ms
        tot_f += flops
        res["parts"][name] = {"ms": round(ms, 4), "gflop": round(flops / 1e9, 2),
                              "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                              "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    res.update({"ms_per_step": round(tot_ms, 4), "visible_gflop": round(tot_f / 1e9, 2),
                "tflops": round(tot_f / (tot_ms * 1e-3) / 1e12, 2),
                "pct_bf16_peak": round(100 * tot_f / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)})
    del t, ctx_out, q_out, ws_c, ws_q, ws_kv
    torch.cuda.empty_cache()
    return res


def measure_gqa(steps: int, warmup: int) -> dict:
    """The MHA/GQA draft: 8 requests with contexts of 8K-32K tokens (hidden 7168,
    32 query heads over 8 KV heads of 128, block 16).  Times the context
    materialisation (a GEMM into the cache) and forward_block; the block's
    attention reads every cached key and value once per KV head, so it is
    reported in HBM bytes per second against 8 TB/s."""
    import numpy as np
    import torch
    from dflash_block_draft_amd import mla
    from dflash_block_draft_amd import workloads as W

    dev = torch.device("cuda:0")
    B, Lc, bs, hidden, Hq, Hkv = 8, 32768, 16, 7168, 32, 8
    ctx = np.random.default_rng(3000).integers(8192, Lc + 1, size=B)
    # weights and the block from the seeded host recipe; the 8 x 32768 x 7168 context
    # hidden states N(0,1) from a seeded device generator (the host one would take minutes)
    p = W.gqa_inputs(3001, B, 16, bs, hidden, Hq, Hkv, ctx_len=ctx, Lmax=-(-(Lc + bs) // 8) * 8)
    t = {k: (v.to(dev) if hasattr(v, "to") else v) for k, v in p.items()}
    gen = torch.Generator(device=dev)
    gen.manual_seed(3002)
    t["ctx_hidden"] = torch.randn((B, Lc, hidden), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    kc, vc = mla.gqa_new_cache(B, Hkv, p["Lmax"], dev)
    ws = torch.empty(mla.load_library().dflash_gqa_workspace_bytes(B, bs, Hq, Hkv, p["Lmax"]), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, Hq, bs, 128), dtype=torch.bfloat16, device=dev)

    def mat():
        mla.gqa_materialize(t["ctx_hidden"], t["w_k"], t["w_v"], t["g_k"], p["eps"], p["rope"], kc, vc)

    def blk():
        mla.gqa_forward_block(t["blk_hidden"], t["w_q"], t["w_k"], t["w_v"], t["g_q"], t["g_k"], p["eps"], p["rope"],
                              kc, vc, t["ctx_len"], Hq, out=out, workspace=ws)

    res = {"workload": "gqa_draft_b8_ctx8k-32k_h32kv8_bs16", "pass": "MAX-page GQA draft (materialize, forward_block)"}
    for name, fn, n in (("materialize", mat, max(2, steps // 4)), ("forward_block", blk, steps)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(a.elapsed_time(b) / n, 4)
    mat_flops = 2.0 * B * Lc * hidden * 2 * Hkv * 128
    kv_bytes = float(sum(int(c) + bs for c in ctx)) * Hkv * 128 * 2 * 2
    res["materialize_tflops"] = round(mat_flops / (res["materialize_ms"] * 1e-3) / 1e12, 2)
    res["forward_block_kv_bytes"] = int(kv_bytes)
    res["forward_block_GBs"] = round(kv_bytes / (res["forward_block_ms"] * 1e-3) / 1e9, 1)
    res["forward_block_pct_hbm_peak"] = round(100 * kv_bytes / (res["forward_block_ms"] * 1e-3) / 8e12, 2)
    res["ms_per_step"] = res["forward_block_ms"]
    res["tflops"] = None
    res["pct_bf16_peak"] = None
    del t, kc, vc, ws, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, budget_s: float) -> dict:
    """The fp64 oracle as it stands, timed on the host on a bounded sample:
    batch row 0, heads 0, 1, ... (all query rows each) until the budget is used."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    import torch
    q, kn, kr, v, m = wl.q[:1], wl.k_nope[:1], wl.k_rope[:1], wl.v[:1], wl.mask[:1]
    pairs = int(torch.isfinite(m.float()).sum().item())
    done = 0
    t0 = time.perf_counter()
    while done < wl.H and (time.perf_counter() - t0) < budget_s:
        oracle.mla_attention(q[:, done:done + 1], kn[:, done:done + 1], kr, v[:, done:done + 1], m, wl.scale)
        done += 1
    dt = time.perf_counter() - t0
    flops = pairs * done * 640
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{wl.name}: batch row 0, heads 0..{done - 1} ({done} of {wl.H}), all {wl.Lq} query rows; "
                      f"{flops / 1e9:.1f} visible GFLOP in {dt:.1f} s (fp64 numpy)"}


def traffic_for(wl_name: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, if the
    kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(wl_name)
    if not rec or rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(path: str, counter: str):
    import csv
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                yield row.get("Kernel_Name", ""), float(row["Counter_Value"])


def traffic_from(args) -> None:
    """HBM bytes per launch of the attention kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled so that the calibration copy of known size
    reads and writes exactly its own bytes."""
    nb = args.copy_calibration_mb << 20
    if nb <= 0:
        raise SystemExit("--traffic-from needs --copy-calibration-mb (the size used in the counter runs)")
    out = {}
    for path, counter in zip(args.traffic_from, ("FETCH_SIZE", "WRITE_SIZE")):
        rows = list(_counter_rows(path, counter))
        copies = [v for k, v in rows if "copy" in k.lower()]
        attn = [v for k, v in rows if "attn_fwd_bf16" in k]
        if not copies or not attn:
            raise SystemExit(f"{path}: no calibration copy or attention dispatch with {counter}")
        factor = nb / (max(copies) * 1024.0)
        out[counter] = {"kib_per_launch_raw": sum(attn) / len(attn), "calibration_factor": factor,
                        "bytes_per_launch": sum(attn) / len(attn) * 1024.0 * factor, "launches": len(attn)}
    wl = make_workload(args.workload)
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[wl.name] = {"kernel_sha": kernel_sha(),
                     "bytes_per_launch": round(out["FETCH_SIZE"]["bytes_per_launch"]
                                               + out["WRITE_SIZE"]["bytes_per_launch"]),
                     "read_bytes": round(out["FETCH_SIZE"]["bytes_per_launch"]),
                     "write_bytes": round(out["WRITE_SIZE"]["bytes_per_launch"]),
                     "calibration": {k: round(v["calibration_factor"], 4) for k, v in out.items()},
                     "calibration_copy_bytes": nb}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(data[wl.name]))


def main():
    args = parse()
    WARM["seconds"] = max(0.0, args.warm_seconds)
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the draft attention "
              "shards over heads/batch rows with no exchange, but only the one-GPU path is implemented.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    from dflash_block_draft_amd import mla
    mla.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration_mb > 0:
        nb = args.copy_calibration_mb << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {nb} bytes read, {nb} bytes written")
        del src, dst

    log(f"building workload {args.workload}")
    wl = make_workload(args.workload)
    log(describe(wl))
    head = measure(wl, args.steps, args.warmup)
    log(f"headline: {head['ms_per_step']} ms/step, {head['tflops']} TFLOP/s "
        f"({head['pct_bf16_peak']}% of bf16 peak); attention kernel {head['attn_kernel_ms']} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        log(f"oracle: {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    secondary = []
    if args.secondary.strip().lower() != "none":
        for key in [k.strip() for k in args.secondary.split(",") if k.strip()]:
            if key == args.workload:
                continue
            if key == "gqa":
                log("GQA draft: materialize + forward_block")
                r = measure_gqa(max(3, args.steps // 2), max(1, args.warmup // 2))
                log(f"gqa: forward_block {r['forward_block_ms']} ms ({r['forward_block_GBs']} GB/s), "
                    f"materialize {r['materialize_ms']} ms ({r['materialize_tflops']} TFLOP/s)")
                secondary.append(r)
                continue
            log(f"building workload {key}")
            w2 = make_workload(key)
            log(describe(w2))
            mode = split_key(key)[1]
            if mode == "b":
                r = measure_bwd(w2, max(3, args.steps // 2), max(1, args.warmup // 2))
            elif mode == "p":
                r = measure_proj(w2, max(3, args.steps // 2), max(1, args.warmup // 2))
            else:
                r = measure(w2, max(3, args.steps // 2), max(1, args.warmup // 2), structured=mode == "s")
            log(f"{key}: {r['ms_per_step']} ms/step, {r['tflops']} TFLOP/s ({r['pct_bf16_peak']}%)")
            secondary.append(r)
            del w2

    att_s = head["attn_kernel_ms"] * 1e-3
    achieved = head["visible_gflop"] * 1e9 / att_s / 1e12
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors, DFlash block mask from sorted random anchors)",
        "config": {"workload": wl.name, "batch": wl.B, "heads": wl.H, "context": wl.ctx,
                   "anchors": wl.num_anchors, "block_size": wl.block_size, "Lq": wl.Lq, "Lk": wl.Lk,
                   "qk_nope": wl.Dn, "qk_rope_shared": wl.Dr, "v_head_dim": wl.Dv,
                   "mask_dtype": wl.mask_dtype, "parallelism": "none (1 GPU)"},
        "pct_bf16_peak": head["pct_bf16_peak"],
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(wl.name),
                     "basis": "visible FLOPs (finite-mask pairs x heads x 640) / mean time of the attention call (HIP events on its stream: the attention kernel plus, where the key list is split into runs, the merge of the runs)"},
        "cpu_baseline": cpu,
        "host": host_info(),
        "sclk": head.get("sclk"),
        "headline": head,
        "secondary": secondary,
        "attn_kernel_sha": kernel_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
