"""Seeded synthetic inputs for the DFlash/DSpark draft MLA attention.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the bench)
and the fp64 oracle consume what it returns, so the two sides always see the
same bf16/f32 values.

Tensor contract (NeMo AutoModel "draft_kimi_k3" pages, KimiK3DFlashAttention.forward
and KimiK3DSparkAttention.forward): queries come from the noise block only,
num_anchors * block_size of them; keys and values span
[context | noise block], the context placed before the noise block; the
additive mask has shape [batch, 1, Lq, ctx + Lq].

The fill rule of the mask is not printed on the pages (they say only that a
DFlash mask builder produces it).  The reading used here: query i belongs to
block j = i // block_size; context key k is visible iff k <= anchor_j and k is
not padding; noise key ctx + m is visible iff m // block_size == j, i.e. a
block sees all of its own keys, non-causally.  Every other entry is -inf.

Layouts (all contiguous):
  q         [B, H, Lq, Dn + Dr]   (q_nope then q_rope)
  k_nope    [B, H, Lk, Dn]
  k_rope    [B, Lk, Dr]           (one per token, shared by every head)
  v         [B, H, Lk, Dv]
  mask      [B, 1, Lq, Lk]
  latent    [B, Lk, R]            (kv_b_proj input; only for the expand workload)
  w_kv_b    [H * (Dn + Dv), R]    (Linear out x in; per head the slice is [k_nope | v])
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

DN = 128   # qk_nope_head_dim
DR = 64    # qk_rope_head_dim (head-shared, no rotary)
DV = 128   # v_head_dim
R_LATENT = 512  # kv_lora_rank for the expand workload

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    H: int
    ctx: int
    ctx_valid: int
    num_anchors: int
    block_size: int
    dtype: str        # "f32" | "bf16" for q / k / v / out
    mask_dtype: str   # "f32" | "bf16"
    anchors: np.ndarray          # [B, A] int64, sorted, distinct
    q: torch.Tensor
    k_rope: torch.Tensor
    mask: torch.Tensor
    k_nope: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    latent: Optional[torch.Tensor] = None
    w_kv_b: Optional[torch.Tensor] = None
    Dn: int = DN
    Dr: int = DR
    Dv: int = DV

    @property
    def Lq(self) -> int:
        return self.num_anchors * self.block_size

    @property
    def Lk(self) -> int:
        return self.ctx + self.Lq

    @property
    def scale(self) -> float:
        # softmax scale q_head_dim ** -0.5 with q_head_dim = qk_nope + qk_rope
        return float(self.Dn + self.Dr) ** -0.5


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def draw_anchors(rng: np.random.Generator, B: int, A: int, ctx_valid: int) -> np.ndarray:
    """Per batch row: A sorted, distinct anchors, uniform on [1, ctx_valid - 1]."""
    out = np.empty((B, A), dtype=np.int64)
    for b in range(B):
        out[b] = np.sort(rng.choice(np.arange(1, ctx_valid), size=A, replace=False))
    return out


def visibility(anchors: np.ndarray, ctx: int, ctx_valid, block_size: int) -> np.ndarray:
    """Boolean [B, Lq, Lk]: True where query i may see key k (reading stated above).
    ctx_valid is one int or one per batch row."""
    B, A = anchors.shape
    cv = np.broadcast_to(np.asarray(ctx_valid, dtype=np.int64), (B,))
    Lq = A * block_size
    Lk = ctx + Lq
    blk = np.arange(Lq) // block_size                        # block of each query
    k = np.arange(Lk)
    vis = np.zeros((B, Lq, Lk), dtype=bool)
    ctx_k = k[:ctx]
    for b in range(B):
        anc = anchors[b][blk]                                 # anchor of each query's block
        vis[b, :, :ctx] = (ctx_k[None, :] <= anc[:, None]) & (ctx_k[None, :] < cv[b])
    noise_blk = (k[ctx:] - ctx) // block_size
    vis[:, :, ctx:] = (noise_blk[None, :] == blk[:, None])[None]
    return vis


def additive_mask(vis: np.ndarray, mask_dtype: str) -> torch.Tensor:
    """0 where visible, -inf elsewhere; shape [B, 1, Lq, Lk]."""
    m = torch.zeros(vis.shape, dtype=_TORCH_DT[mask_dtype])
    m.masked_fill_(torch.from_numpy(~vis), float("-inf"))
    return m.unsqueeze(1).contiguous()


def normal(rng: np.random.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    """N(0, std^2) drawn in float32, then rounded (RNE) to the target dtype."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(_TORCH_DT[dtype]).contiguous()


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def _make(name, seed, B, H, ctx, A, bs, dtype, mask_dtype, pad=0, std=1.0,
          expand=False, make_kv=True) -> Workload:
    rng = np.random.default_rng(seed)
    ctx_valid = ctx - pad
    anchors = draw_anchors(rng, B, A, ctx_valid)
    Lq = A * bs
    Lk = ctx + Lq
    q = normal(rng, (B, H, Lq, DN + DR), std, dtype)
    wl = Workload(name=name, seed=seed, B=B, H=H, ctx=ctx, ctx_valid=ctx_valid,
                  num_anchors=A, block_size=bs, dtype=dtype, mask_dtype=mask_dtype,
                  anchors=anchors, q=q, k_rope=None, mask=None)
    if expand:
        wl.latent = normal(rng, (B, Lk, R_LATENT), 1.0, dtype)
        wl.w_kv_b = normal(rng, (H * (DN + DV), R_LATENT), 0.02, dtype)
        wl.k_rope = normal(rng, (B, Lk, DR), 1.0, dtype)
    else:
        if make_kv:
            wl.k_nope = normal(rng, (B, H, Lk, DN), std, dtype)
        wl.k_rope = normal(rng, (B, Lk, DR), std, dtype)
        if make_kv:
            wl.v = normal(rng, (B, H, Lk, DV), std, dtype)
    wl.mask = additive_mask(visibility(anchors, ctx, ctx_valid, bs), mask_dtype)
    return wl


def config(idx: int, block_size: Optional[int] = None) -> Workload:
    """Workload `idx` (0..4) with seed = idx; the block-size sweep (3) takes block_size 8 or 32."""
    if idx == 0:
        return _make("tiny_f32_ctx64_h4", 0, B=1, H=4, ctx=64, A=2, bs=16,
                     dtype="f32", mask_dtype="f32")
    if idx == 1:
        return _make("expand_bf16_b2_ctx2048_h16", 1, B=2, H=16, ctx=2048, A=16, bs=16,
                     dtype="bf16", mask_dtype="f32", expand=True)
    if idx == 2:
        return _make("train_bf16_ctx8192_h64", 2, B=1, H=64, ctx=8192, A=64, bs=16,
                     dtype="bf16", mask_dtype="bf16", std=2.0 ** -0.5)
    if idx == 3:
        bs = 8 if block_size is None else block_size
        if bs not in (8, 32):
            raise ValueError("the block-size sweep uses block_size 8 or 32")
        return _make(f"sweep_bf16_b4_ctx4096_h32_bs{bs}", 3, B=4, H=32, ctx=4096, A=32, bs=bs,
                     dtype="bf16", mask_dtype="bf16", pad=4096 // 20)
    if idx == 4:
        return _make("longctx_bf16_ctx32768_h32", 4, B=1, H=32, ctx=32768, A=256, bs=16,
                     dtype="bf16", mask_dtype="f32")
    raise ValueError(f"unknown workload {idx}")


def custom(seed: int, B: int, H: int, ctx: int, A: int, bs: int, dtype: str = "bf16",
           mask_dtype: str = "f32", pad: int = 0, std: float = 1.0) -> Workload:
    """Same recipe at an arbitrary (small) shape, for ragged-tile tests."""
    return _make(f"custom_s{seed}_b{B}_h{H}_ctx{ctx}_a{A}_bs{bs}", seed, B=B, H=H, ctx=ctx,
                 A=A, bs=bs, dtype=dtype, mask_dtype=mask_dtype, pad=pad, std=std)


def random_attention_inputs(seed: int, B: int, H: int, Lq: int, Lk: int, dtype: str = "f32",
                            std: float = 1.0):
    """Plain N(0, std^2) q / k_nope / k_rope / v at any (Lq, Lk); no mask."""
    rng = np.random.default_rng(seed)
    q = normal(rng, (B, H, Lq, DN + DR), std, dtype)
    kn = normal(rng, (B, H, Lk, DN), std, dtype)
    kr = normal(rng, (B, Lk, DR), std, dtype)
    v = normal(rng, (B, H, Lk, DV), std, dtype)
    return q, kn, kr, v


def visible_pairs(mask: torch.Tensor) -> int:
    """Number of (batch, query, key) entries whose mask value is finite."""
    return int(torch.isfinite(mask.float()).sum().item())


def visible_flops(mask: Optional[torch.Tensor], B: int, H: int, Lq: int, Lk: int,
                  Dqk: int = DN + DR, Dv: int = DV) -> int:
    """Visible FLOPs: finite-mask (query, key) pairs x heads x (2*Dqk + 2*Dv)."""
    pairs = B * Lq * Lk if mask is None else visible_pairs(mask)
    return pairs * H * (2 * Dqk + 2 * Dv)


# --------------------------------------------------------------------------
# projections around the attention (fc + hidden_norm, Q-LoRA, kv_a + kv_b)
# --------------------------------------------------------------------------

# Sizes for the full-size projection workload.  The pages give kv_lora_rank 512
# (the expand workload), qk_rope 64, qk_nope 128, v 128; the hidden size, the
# Q-LoRA rank and the number of target layers feeding fc are not stated, so
# they take the values of the Kimi/DeepSeek-V3 MLA family the draft inherits
# (hidden 7168, q_lora_rank 1536) and four target layers.
PROJ_HIDDEN = 7168
PROJ_Q_LORA = 1536
PROJ_TARGET_LAYERS = 4
RMS_EPS = 1e-6


def projection_inputs(seed: int, B: int, ctx: int, Lq: int, H: int, hidden: int = PROJ_HIDDEN,
                      q_lora_rank: int = PROJ_Q_LORA, R: int = R_LATENT, Dr: int = DR,
                      n_target_layers: int = PROJ_TARGET_LAYERS) -> dict:
    """Hidden states N(0,1); Linear weights N(0, 0.02^2); RMSNorm weights 1 + N(0, 0.1^2); all bf16."""
    rng = np.random.default_rng(seed)
    return {
        "target_hidden": normal(rng, (B, ctx, n_target_layers * hidden), 1.0, "bf16"),
        "w_fc": normal(rng, (hidden, n_target_layers * hidden), 0.02, "bf16"),
        "g_hidden": (1.0 + normal(rng, (hidden,), 0.1, "f32")).to(torch.bfloat16),
        "ctx_hidden": normal(rng, (B, ctx, hidden), 1.0, "bf16"),
        "noise_hidden": normal(rng, (B, Lq, hidden), 1.0, "bf16"),
        "w_q_a": normal(rng, (q_lora_rank, hidden), 0.02, "bf16"),
        "g_q": (1.0 + normal(rng, (q_lora_rank,), 0.1, "f32")).to(torch.bfloat16),
        "w_q_b": normal(rng, (H * (DN + DR), q_lora_rank), 0.02, "bf16"),
        "w_kv_a": normal(rng, (R + Dr, hidden), 0.02, "bf16"),
        "g_kv": (1.0 + normal(rng, (R,), 0.1, "f32")).to(torch.bfloat16),
        "w_kv_b": normal(rng, (H * (DN + DV), R), 0.02, "bf16"),
        "B": B, "ctx": ctx, "Lq": Lq, "H": H, "hidden": hidden, "q_lora_rank": q_lora_rank, "R": R, "Dr": Dr,
        "eps": RMS_EPS,
    }


# --------------------------------------------------------------------------
# the MHA/GQA draft (Modular MAX page) -- materialised context + block attention
# --------------------------------------------------------------------------

# The page gives the config fields, not their values.  Readings: the target's
# hidden 7168; 32 query heads over 8 KV heads of 128; block size 16; yarn RoPE
# with theta 50000, factor 32 over an original 4096 positions, beta_fast 32,
# beta_slow 1, mscale = mscale_all_dim = 1 (the Kimi K2 family's values).
GQA_ROPE = (50000.0, 32.0, 4096.0, 32.0, 1.0, 1.0, 1.0)


def gqa_inputs(seed: int, B: int, Lc: int, bs: int, hidden: int, Hq: int, Hkv: int, ctx_len=None,
               Lmax: Optional[int] = None, d: int = 128) -> dict:
    """Hidden states N(0,1), projections N(0, 0.02^2), qk-norm weights 1 + N(0, 0.1^2),
    all bf16; ctx_len[b] (default: uniform in [Lc/2, Lc]) int32."""
    rng = np.random.default_rng(seed)
    if ctx_len is None:
        ctx_len = rng.integers(Lc // 2, Lc + 1, size=B)
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    if Lmax is None:
        Lmax = -(-(Lc + bs) // 8) * 8
    return {
        "ctx_hidden": normal(rng, (B, Lc, hidden), 1.0, "bf16"),
        "blk_hidden": normal(rng, (B, bs, hidden), 1.0, "bf16"),
        "w_q": normal(rng, (Hq * d, hidden), 0.02, "bf16"),
        "w_k": normal(rng, (Hkv * d, hidden), 0.02, "bf16"),
        "w_v": normal(rng, (Hkv * d, hidden), 0.02, "bf16"),
        "g_q": (1.0 + normal(rng, (d,), 0.1, "f32")).to(torch.bfloat16),
        "g_k": (1.0 + normal(rng, (d,), 0.1, "f32")).to(torch.bfloat16),
        "ctx_len": torch.from_numpy(ctx_len),
        "B": B, "Lc": Lc, "bs": bs, "hidden": hidden, "Hq": Hq, "Hkv": Hkv, "Lmax": Lmax, "d": d,
        "eps": RMS_EPS, "rope": GQA_ROPE,
    }
