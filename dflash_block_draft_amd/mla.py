"""Thin Python binding of the C ABI in include/dflash_mla.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are passed
to the library.  Every step of the computation runs in the HIP kernels; there
is no fallback of any kind, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; DFLASH_MLA_LIB selects another build of the same library
# (e.g. the host-sanitized one the ABI tests run under)
LIB_PATH = os.environ.get("DFLASH_MLA_LIB") or os.path.join(_HERE, "libdflash_mla.so")

TILE_M = 128
TILE_N = 64
DN, DR, DV = 128, 64, 128

_F32, _BF16 = 0, 1
_DT = {torch.float32: _F32, torch.bfloat16: _BF16}
FLAG_REUSE_TILE_MAP = 0x1
FLAG_NO_TILE_SKIP = 0x2
FLAG_CHECK_ONLY = 0x4
FLAG_SPLIT_KEYS = 0x8

EXPORTED = (
    "dflash_status_string", "dflash_last_error", "dflash_mla_latent_expand",
    "dflash_mla_attn_workspace_bytes", "dflash_mla_tile_map_layout",
    "dflash_mla_mask_occupancy", "dflash_mla_attn", "dflash_mla_block_occupancy",
    "dflash_mla_attn_blocks", "dflash_mla_attn_lse", "dflash_mla_attn_bwd_workspace_bytes",
    "dflash_mla_attn_bwd", "dflash_mla_projection_workspace_bytes", "dflash_mla_context_project",
    "dflash_mla_q_project", "dflash_mla_kv_project", "dflash_gqa_materialize", "dflash_gqa_workspace_bytes",
    "dflash_gqa_forward_block", "dflash_mla_attn_split_workspace_bytes", "dflash_mla_attn_no_alloc",
)


class DflashError(ValueError):
    """A non-OK status from the library (bad configuration raises ValueError,
    as the pages' config builders do)."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libdflash_mla.so (built by dflash_block_draft_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m dflash_block_draft_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, u32, f32, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t,
                                  ctypes.c_uint32, ctypes.c_float, ctypes.c_int)
    lib.dflash_status_string.argtypes = [i32]
    lib.dflash_status_string.restype = ctypes.c_char_p
    lib.dflash_last_error.argtypes = []
    lib.dflash_last_error.restype = ctypes.c_char_p
    lib.dflash_mla_latent_expand.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.dflash_mla_latent_expand.restype = i32
    lib.dflash_mla_attn_workspace_bytes.argtypes = [i64, i64, i64]
    lib.dflash_mla_attn_workspace_bytes.restype = sz
    lib.dflash_mla_attn_split_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.dflash_mla_attn_split_workspace_bytes.restype = sz
    p64, psz = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)
    lib.dflash_mla_tile_map_layout.argtypes = [i64, i64, i64, p64, p64, psz, psz, psz, psz, psz]
    lib.dflash_mla_tile_map_layout.restype = i32
    lib.dflash_mla_mask_occupancy.argtypes = [vp, i32, i64, i64, i64, vp, sz, vp]
    lib.dflash_mla_mask_occupancy.restype = i32
    lib.dflash_mla_attn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32,
                                    i32, i32, vp, sz, u32, vp]
    lib.dflash_mla_attn.restype = i32
    lib.dflash_mla_attn_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32,
                                        i32, i32, vp, sz, u32, vp]
    lib.dflash_mla_attn_lse.restype = i32
    lib.dflash_mla_attn_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f32,
                                             i32, i32, u32, vp]
    lib.dflash_mla_attn_no_alloc.restype = i32
    lib.dflash_mla_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.dflash_mla_attn_bwd_workspace_bytes.restype = sz
    lib.dflash_mla_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                        i64, i64, i64, f32, i32, i32, vp, sz, u32, vp]
    lib.dflash_mla_attn_bwd.restype = i32
    lib.dflash_mla_projection_workspace_bytes.argtypes = [i64, i64]
    lib.dflash_mla_projection_workspace_bytes.restype = sz
    lib.dflash_mla_context_project.argtypes = [vp, vp, vp, f32, vp, i64, i64, i64, i64, vp, sz, vp]
    lib.dflash_mla_context_project.restype = i32
    lib.dflash_mla_q_project.argtypes = [vp, vp, vp, f32, vp, vp, i64, i64, i64, i64, i64, i64, vp, sz, vp]
    lib.dflash_mla_q_project.restype = i32
    lib.dflash_mla_kv_project.argtypes = [vp, vp, vp, vp, f32, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                          i64, i64, vp, sz, vp]
    lib.dflash_mla_kv_project.restype = i32
    lib.dflash_gqa_materialize.argtypes = [vp, vp, vp, vp, f32, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    lib.dflash_gqa_materialize.restype = i32
    lib.dflash_gqa_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.dflash_gqa_workspace_bytes.restype = sz
    lib.dflash_gqa_forward_block.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                             i64, i64, i64, f32, vp, sz, vp]
    lib.dflash_gqa_forward_block.restype = i32
    lib.dflash_mla_block_occupancy.argtypes = [vp, vp, i64, i64, i64, i64, vp, sz, vp]
    lib.dflash_mla_block_occupancy.restype = i32
    lib.dflash_mla_attn_blocks.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                           f32, i32, vp, sz, u32, vp]
    lib.dflash_mla_attn_blocks.restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise DflashError(status, lib.dflash_status_string(status).decode(),
                          lib.dflash_last_error().decode())


def _stream(t: torch.Tensor) -> Optional[int]:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if dtype is None and t.dtype not in _DT:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def latent_expand(latent: torch.Tensor, w_kv_b: torch.Tensor, num_heads: int,
                  qk_nope_head_dim: int = DN, v_head_dim: int = DV,
                  k_nope: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None):
    """kv_b_proj: latent [B, Lk, R] x w_kv_b [H*(Dn+Dv), R] -> (k_nope [B,H,Lk,Dn], v [B,H,Lk,Dv])."""
    lib = load_library()
    _dev(latent, "latent", ndim=3)
    _dev(w_kv_b, "w_kv_b", dtype=latent.dtype, ndim=2)
    B, Lk, R = latent.shape
    H = int(num_heads)
    if k_nope is None:
        k_nope = torch.empty((B, H, Lk, qk_nope_head_dim), dtype=latent.dtype, device=latent.device)
    if v is None:
        v = torch.empty((B, H, Lk, v_head_dim), dtype=latent.dtype, device=latent.device)
    _dev(k_nope, "k_nope", dtype=latent.dtype, ndim=4)
    _dev(v, "v", dtype=latent.dtype, ndim=4)
    if tuple(w_kv_b.shape) != (H * (qk_nope_head_dim + v_head_dim), R):
        raise ValueError(f"w_kv_b must be [{H * (qk_nope_head_dim + v_head_dim)}, {R}], got {tuple(w_kv_b.shape)}")
    if tuple(k_nope.shape) != (B, H, Lk, qk_nope_head_dim) or tuple(v.shape) != (B, H, Lk, v_head_dim):
        raise ValueError("output shapes do not match [B, H, Lk, D]")
    _check(lib.dflash_mla_latent_expand(_ptr(latent), _ptr(w_kv_b), _ptr(k_nope), _ptr(v),
                                        B, Lk, R, H, qk_nope_head_dim, v_head_dim,
                                        _DT[latent.dtype], _stream(latent)))
    return k_nope, v


def attn_workspace_bytes(B: int, Lq: int, Lk: int) -> int:
    return int(load_library().dflash_mla_attn_workspace_bytes(B, Lq, Lk))


def attn_split_workspace_bytes(B: int, H: int, Lq: int, Lk: int) -> int:
    return int(load_library().dflash_mla_attn_split_workspace_bytes(B, H, Lq, Lk))


def new_workspace(B: int, Lq: int, Lk: int, device, H: Optional[int] = None) -> torch.Tensor:
    """Attention workspace: the tile map; with H also room for the key-split partials."""
    n = attn_workspace_bytes(B, Lq, Lk)
    if H is not None:
        n = max(n, attn_split_workspace_bytes(B, H, Lq, Lk))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _split_flag(B: int, H: int, Lq: int, Lk: int, workspace: Optional[torch.Tensor]) -> int:
    """FLAG_SPLIT_KEYS when this shape splits and the workspace holds the partials."""
    sb = attn_split_workspace_bytes(B, H, Lq, Lk)
    if workspace is None or sb <= attn_workspace_bytes(B, Lq, Lk) or workspace.numel() < sb:
        return 0
    return FLAG_SPLIT_KEYS


def mask_occupancy(mask: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run the occupancy pass alone; returns the workspace holding the tile map."""
    lib = load_library()
    _dev(mask, "mask", ndim=4)
    B, one, Lq, Lk = mask.shape
    if one != 1:
        raise ValueError("mask must be [B, 1, Lq, Lk]")
    if workspace is None:
        workspace = new_workspace(B, Lq, Lk, mask.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    _check(lib.dflash_mla_mask_occupancy(_ptr(mask), _DT[mask.dtype], B, Lq, Lk, _ptr(workspace),
                                         workspace.numel(), _stream(mask)))
    return workspace


def tile_map_view(workspace: torch.Tensor, B: int, Lq: int, Lk: int) -> dict:
    """Views of the occupancy results inside a workspace (see dflash_mla_tile_map_layout)."""
    lib = load_library()
    nq, nk = ctypes.c_int64(), ctypes.c_int64()
    offs = [ctypes.c_size_t() for _ in range(5)]
    _check(lib.dflash_mla_tile_map_layout(B, Lq, Lk, ctypes.byref(nq), ctypes.byref(nk),
                                          *[ctypes.byref(o) for o in offs]))
    nq, nk = nq.value, nk.value
    c_off, n_off, l_off, o_off, b_off = (o.value for o in offs)
    ws = workspace
    return {
        "n_q_tiles": nq, "n_k_tiles": nk,
        "classes": ws[c_off:c_off + B * nq * nk].view(B, nq, nk),
        "counts": ws[n_off:n_off + 4 * B * nq].view(torch.int32).view(B, nq),
        "lists": ws[l_off:l_off + 4 * B * nq * nk].view(torch.int32).view(B, nq, nk),
        "order": ws[o_off:o_off + 4 * B * nq].view(torch.int32),
        "bits": ws[b_off:b_off + 8 * B * nq * nk * TILE_M].view(torch.int64).view(B, nq, nk, TILE_M),
    }


def mla_attn(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
             mask: Optional[torch.Tensor] = None, scale: Optional[float] = None, *,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             reuse_tile_map: bool = False, tile_skip: bool = True, lse: Optional[torch.Tensor] = None,
             split_keys: bool = True):
    """Draft MLA attention: q [B,H,Lq,Dn+Dr], k_nope [B,H,Lk,Dn], k_rope [B,Lk,Dr] (head-shared),
    v [B,H,Lk,Dv], mask [B,1,Lq,Lk] or None -> out [B,H,Lq,Dv].  scale defaults to
    q_head_dim ** -0.5.  With `lse` (a float32 [B,H,Lq] device tensor) the row
    log-normalisers are written there too (dflash_mla_attn_lse).  bf16 with
    `split_keys`: a small grid is split over key ranges when the workspace (allocated
    here when not given) holds the partials."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    dt = q.dtype
    _dev(k_nope, "k_nope", dtype=dt, ndim=4)
    _dev(k_rope, "k_rope", dtype=dt, ndim=3)
    _dev(v, "v", dtype=dt, ndim=4)
    B, H, Lq, Dqk = q.shape
    Lk, Dn = k_nope.shape[2], k_nope.shape[3]
    Dr, Dv = k_rope.shape[2], v.shape[3]
    if Dqk != Dn + Dr:
        raise ValueError(f"q last dim {Dqk} != Dn + Dr = {Dn + Dr}")
    if tuple(k_nope.shape[:2]) != (B, H) or tuple(v.shape[:3]) != (B, H, Lk) or tuple(k_rope.shape[:2]) != (B, Lk):
        raise ValueError("q / k_nope / k_rope / v shapes are inconsistent")
    if scale is None:
        scale = float(Dn + Dr) ** -0.5
    mask_dt = _F32
    if mask is not None:
        _dev(mask, "mask", ndim=4)
        if tuple(mask.shape) != (B, 1, Lq, Lk):
            raise ValueError(f"mask must be [{B}, 1, {Lq}, {Lk}], got {tuple(mask.shape)}")
        mask_dt = _DT[mask.dtype]
    split = split_keys and dt == torch.bfloat16 and tile_skip
    if mask is not None:
        if workspace is None:
            if reuse_tile_map:
                raise ValueError("reuse_tile_map needs the workspace that holds the map")
            workspace = new_workspace(B, Lq, Lk, q.device, H=H if split else None)
    elif reuse_tile_map and workspace is None:
        raise ValueError("reuse_tile_map without a mask needs the workspace that holds the map")
    elif workspace is None and split and attn_split_workspace_bytes(B, H, Lq, Lk) > attn_workspace_bytes(B, Lq, Lk):
        workspace = new_workspace(B, Lq, Lk, q.device, H=H)
    if out is None:
        out = torch.empty((B, H, Lq, Dv), dtype=dt, device=q.device)
    _dev(out, "out", dtype=dt, ndim=4)
    if workspace is not None:
        _dev(workspace, "workspace", dtype=torch.uint8)
    flags = (FLAG_REUSE_TILE_MAP if reuse_tile_map else 0) | (0 if tile_skip else FLAG_NO_TILE_SKIP)
    if split:
        flags |= _split_flag(B, H, Lq, Lk, workspace)
    wsb = 0 if workspace is None else workspace.numel()
    if lse is None:
        _check(lib.dflash_mla_attn(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(mask), _ptr(out),
                                   B, H, Lq, Lk, Dn, Dr, Dv, float(scale), _DT[dt], mask_dt,
                                   _ptr(workspace), wsb, flags, _stream(q)))
    else:
        _dev(lse, "lse", dtype=torch.float32, ndim=3)
        if tuple(lse.shape) != (B, H, Lq):
            raise ValueError(f"lse must be [{B}, {H}, {Lq}]")
        _check(lib.dflash_mla_attn_lse(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(mask), _ptr(out),
                                       _ptr(lse), B, H, Lq, Lk, Dn, Dr, Dv, float(scale), _DT[dt], mask_dt,
                                       _ptr(workspace), wsb, flags, _stream(q)))
    return out


def mla_attn_no_alloc(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                      mask: Optional[torch.Tensor] = None, scale: Optional[float] = None, *,
                      out: torch.Tensor, tile_skip: bool = True) -> torch.Tensor:
    """dflash_mla_attn_no_alloc: mla_attn without a workspace (the tile map goes to the
    library's static per-GPU scratch).  `out` must be given: nothing is allocated here
    either."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    dt = q.dtype
    _dev(k_nope, "k_nope", dtype=dt, ndim=4)
    _dev(k_rope, "k_rope", dtype=dt, ndim=3)
    _dev(v, "v", dtype=dt, ndim=4)
    _dev(out, "out", dtype=dt, ndim=4)
    B, H, Lq, _ = q.shape
    Lk, Dn = k_nope.shape[2], k_nope.shape[3]
    Dr, Dv = k_rope.shape[2], v.shape[3]
    if scale is None:
        scale = float(Dn + Dr) ** -0.5
    mask_dt = _F32
    if mask is not None:
        _dev(mask, "mask", ndim=4)
        mask_dt = _DT[mask.dtype]
    flags = 0 if tile_skip else FLAG_NO_TILE_SKIP
    _check(lib.dflash_mla_attn_no_alloc(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(mask), _ptr(out),
                                        B, H, Lq, Lk, Dn, Dr, Dv, float(scale), _DT[dt], mask_dt, flags,
                                        _stream(q)))
    return out


def attn_bwd_workspace_bytes(B: int, H: int, Lq: int, Lk: int) -> int:
    return int(load_library().dflash_mla_attn_bwd_workspace_bytes(B, H, Lq, Lk))


def new_bwd_workspace(B: int, H: int, Lq: int, Lk: int, device) -> torch.Tensor:
    """A workspace for the backward; it also serves the forward (the tile map comes first)."""
    n = attn_bwd_workspace_bytes(B, H, Lq, Lk)
    if n == 0:
        raise ValueError("invalid sizes for the backward workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mla_attn_bwd(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                 mask: Optional[torch.Tensor], out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                 scale: Optional[float] = None, *, workspace: Optional[torch.Tensor] = None,
                 reuse_tile_map: bool = False, grads=None):
    """Gradients (dq, dk_nope, dk_rope, dv) of mla_attn (bf16); out and lse from the
    forward with lse.  `grads` may supply the four output tensors."""
    lib = load_library()
    for t, n, nd in ((q, "q", 4), (k_nope, "k_nope", 4), (k_rope, "k_rope", 3), (v, "v", 4), (out, "out", 4),
                     (dout, "dout", 4)):
        _dev(t, n, dtype=torch.bfloat16, ndim=nd)
    _dev(lse, "lse", dtype=torch.float32, ndim=3)
    B, H, Lq, _ = q.shape
    Lk, Dn, Dr, Dv = k_nope.shape[2], k_nope.shape[3], k_rope.shape[2], v.shape[3]
    if tuple(out.shape) != (B, H, Lq, Dv) or tuple(dout.shape) != (B, H, Lq, Dv) or tuple(lse.shape) != (B, H, Lq):
        raise ValueError("out / dout / lse shapes are inconsistent with q and v")
    if scale is None:
        scale = float(Dn + Dr) ** -0.5
    mask_dt = _F32
    if mask is not None:
        _dev(mask, "mask", ndim=4)
        mask_dt = _DT[mask.dtype]
    if workspace is None:
        if reuse_tile_map:
            raise ValueError("reuse_tile_map needs the workspace that holds the map")
        workspace = new_bwd_workspace(B, H, Lq, Lk, q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k_nope), torch.empty_like(k_rope), torch.empty_like(v))
    dq, dkn, dkr, dv = grads
    for t, ref, n in ((dq, q, "dq"), (dkn, k_nope, "dk_nope"), (dkr, k_rope, "dk_rope"), (dv, v, "dv")):
        _dev(t, n, dtype=torch.bfloat16)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have shape {tuple(ref.shape)}")
    _check(lib.dflash_mla_attn_bwd(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(mask), _ptr(out),
                                   _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dkn), _ptr(dkr), _ptr(dv),
                                   B, H, Lq, Lk, Dn, Dr, Dv, float(scale), _BF16, mask_dt,
                                   _ptr(workspace), workspace.numel(),
                                   FLAG_REUSE_TILE_MAP if reuse_tile_map else 0, _stream(q)))
    return dq, dkn, dkr, dv


def _block_tensors(anchors: torch.Tensor, ctx_valid: Optional[torch.Tensor]):
    _dev(anchors, "anchors", dtype=torch.int32, ndim=2)
    if ctx_valid is not None:
        _dev(ctx_valid, "ctx_valid", dtype=torch.int32, ndim=1)
        if ctx_valid.shape[0] != anchors.shape[0]:
            raise ValueError("ctx_valid must be [B]")
    return anchors.shape


def block_occupancy(anchors: torch.Tensor, block_size: int, ctx: int, ctx_valid: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tile map of the DFlash block mask from anchors [B, A] (int32) and ctx_valid [B]
    (int32, or None = ctx); returns the workspace holding it."""
    lib = load_library()
    B, A = _block_tensors(anchors, ctx_valid)
    Lq = A * int(block_size)
    if workspace is None:
        workspace = new_workspace(B, Lq, int(ctx) + Lq, anchors.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    _check(lib.dflash_mla_block_occupancy(_ptr(anchors), _ptr(ctx_valid), B, A, int(block_size), int(ctx),
                                          _ptr(workspace), workspace.numel(), _stream(anchors)))
    return workspace


def mla_attn_blocks(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                    anchors: torch.Tensor, block_size: int, ctx: int, ctx_valid: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, *, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, reuse_tile_map: bool = False,
                    split_keys: bool = True) -> torch.Tensor:
    """mla_attn with the DFlash block mask given by anchors [B, A] (int32), block_size,
    ctx and ctx_valid [B] (int32, or None = ctx) instead of a dense mask (key split
    as for mla_attn)."""
    lib = load_library()
    _dev(q, "q", dtype=torch.bfloat16, ndim=4)
    _dev(k_nope, "k_nope", dtype=torch.bfloat16, ndim=4)
    _dev(k_rope, "k_rope", dtype=torch.bfloat16, ndim=3)
    _dev(v, "v", dtype=torch.bfloat16, ndim=4)
    B, A = _block_tensors(anchors, ctx_valid)
    Bq, H, Lq, Dqk = q.shape
    Dn, Dr, Dv = k_nope.shape[3], k_rope.shape[2], v.shape[3]
    if Bq != B or Lq != A * int(block_size):
        raise ValueError(f"q must be [{B}, H, {A * int(block_size)}, D], got {tuple(q.shape)}")
    Lk = int(ctx) + Lq
    if tuple(k_nope.shape[:3]) != (B, H, Lk) or tuple(v.shape[:3]) != (B, H, Lk) or tuple(k_rope.shape[:2]) != (B, Lk):
        raise ValueError("k_nope / k_rope / v shapes must use Lk = ctx + A * block_size")
    if scale is None:
        scale = float(Dn + Dr) ** -0.5
    if workspace is None:
        if reuse_tile_map:
            raise ValueError("reuse_tile_map needs the workspace that holds the map")
        workspace = new_workspace(B, Lq, Lk, q.device, H=H if split_keys else None)
    _dev(workspace, "workspace", dtype=torch.uint8)
    if out is None:
        out = torch.empty((B, H, Lq, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out", dtype=q.dtype, ndim=4)
    flags = (FLAG_REUSE_TILE_MAP if reuse_tile_map else 0) | (_split_flag(B, H, Lq, Lk, workspace) if split_keys else 0)
    _check(lib.dflash_mla_attn_blocks(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(anchors), _ptr(ctx_valid),
                                      _ptr(out), B, H, A, int(block_size), int(ctx), Dn, Dr, Dv, float(scale),
                                      _BF16, _ptr(workspace), workspace.numel(), flags, _stream(q)))
    return out


def _proj_ws(rows: int, width: int, device, workspace):
    n = int(load_library().dflash_mla_projection_workspace_bytes(rows, width))
    if n == 0:
        raise ValueError("invalid projection sizes")
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    return workspace


def context_project(target_hidden: torch.Tensor, w_fc: torch.Tensor, gamma: torch.Tensor, eps: float, *,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rmsnorm(target_hidden @ w_fc^T) * gamma: [B, ctx, K_in] -> [B, ctx, hidden] (bf16)."""
    lib = load_library()
    _dev(target_hidden, "target_hidden", dtype=torch.bfloat16, ndim=3)
    _dev(w_fc, "w_fc", dtype=torch.bfloat16, ndim=2)
    _dev(gamma, "gamma", dtype=torch.bfloat16, ndim=1)
    B, ctx, K_in = target_hidden.shape
    hidden = w_fc.shape[0]
    if w_fc.shape[1] != K_in or gamma.shape[0] != hidden:
        raise ValueError("w_fc must be [hidden, K_in] and gamma [hidden]")
    if out is None:
        out = torch.empty((B, ctx, hidden), dtype=torch.bfloat16, device=target_hidden.device)
    _dev(out, "out", dtype=torch.bfloat16, ndim=3)
    workspace = _proj_ws(B * ctx, hidden, target_hidden.device, workspace)
    _check(lib.dflash_mla_context_project(_ptr(target_hidden), _ptr(w_fc), _ptr(gamma), float(eps), _ptr(out),
                                          B, ctx, K_in, hidden, _ptr(workspace), workspace.numel(),
                                          _stream(target_hidden)))
    return out


def q_project(x: torch.Tensor, w_q_a: torch.Tensor, gamma_q: torch.Tensor, eps: float, w_q_b: torch.Tensor,
              H: int, *, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Q-LoRA: (rmsnorm(x @ w_q_a^T) * gamma_q) @ w_q_b^T, as [B, H, Lq, Dqk] (bf16)."""
    lib = load_library()
    _dev(x, "x", dtype=torch.bfloat16, ndim=3)
    for t, n in ((w_q_a, "w_q_a"), (w_q_b, "w_q_b")):
        _dev(t, n, dtype=torch.bfloat16, ndim=2)
    _dev(gamma_q, "gamma_q", dtype=torch.bfloat16, ndim=1)
    B, Lq, hidden = x.shape
    Rq = w_q_a.shape[0]
    if w_q_a.shape[1] != hidden or gamma_q.shape[0] != Rq or w_q_b.shape[1] != Rq or w_q_b.shape[0] % H:
        raise ValueError("inconsistent Q-LoRA shapes")
    Dqk = w_q_b.shape[0] // H
    if out is None:
        out = torch.empty((B, H, Lq, Dqk), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", dtype=torch.bfloat16, ndim=4)
    workspace = _proj_ws(B * Lq, Rq, x.device, workspace)
    _check(lib.dflash_mla_q_project(_ptr(x), _ptr(w_q_a), _ptr(gamma_q), float(eps), _ptr(w_q_b), _ptr(out),
                                    B, Lq, hidden, Rq, H, Dqk, _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def kv_project(ctx_hidden: Optional[torch.Tensor], noise_hidden: torch.Tensor, w_kv_a: torch.Tensor,
               gamma_kv: torch.Tensor, eps: float, w_kv_b: torch.Tensor, H: int, R: int, *,
               workspace: Optional[torch.Tensor] = None):
    """Keys and values over [context | noise]: returns (k_nope [B,H,Lk,128],
    k_rope_shared [B,Lk,Dr], v [B,H,Lk,128]) with Lk = ctx + Lq (bf16)."""
    lib = load_library()
    _dev(noise_hidden, "noise_hidden", dtype=torch.bfloat16, ndim=3)
    B, Lq, hidden = noise_hidden.shape
    ctx = 0
    if ctx_hidden is not None:
        _dev(ctx_hidden, "ctx_hidden", dtype=torch.bfloat16, ndim=3)
        if ctx_hidden.shape[0] != B or ctx_hidden.shape[2] != hidden:
            raise ValueError("ctx_hidden must be [B, ctx, hidden]")
        ctx = ctx_hidden.shape[1]
    for t, n in ((w_kv_a, "w_kv_a"), (w_kv_b, "w_kv_b")):
        _dev(t, n, dtype=torch.bfloat16, ndim=2)
    _dev(gamma_kv, "gamma_kv", dtype=torch.bfloat16, ndim=1)
    Dr = w_kv_a.shape[0] - R
    if w_kv_a.shape[1] != hidden or Dr <= 0 or gamma_kv.shape[0] != R or tuple(w_kv_b.shape) != (H * 256, R):
        raise ValueError("inconsistent kv projection shapes")
    Lk = ctx + Lq
    dev = noise_hidden.device
    kn = torch.empty((B, H, Lk, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, H, Lk, 128), dtype=torch.bfloat16, device=dev)
    kr = torch.empty((B, Lk, Dr), dtype=torch.bfloat16, device=dev)
    workspace = _proj_ws(B * Lk, R, dev, workspace)
    _check(lib.dflash_mla_kv_project(_ptr(ctx_hidden), _ptr(noise_hidden), _ptr(w_kv_a), _ptr(gamma_kv), float(eps),
                                     _ptr(w_kv_b), _ptr(kn), _ptr(kr), _ptr(v), B, ctx, Lq, hidden, R, Dr, H, 128, 128,
                                     _ptr(workspace), workspace.numel(), _stream(noise_hidden)))
    return kn, kr, v


def _rope_array(rope):
    """(theta, factor, original_max_position, beta_fast, beta_slow, mscale, mscale_all_dim)."""
    vals = [float(x) for x in rope]
    if len(vals) != 7:
        raise ValueError("rope takes 7 values")
    return (ctypes.c_float * 7)(*vals)


def gqa_new_cache(B: int, Hkv: int, Lmax: int, device):
    """(k_cache [B, Hkv, Lmax, 128], v_cache_t [B, Hkv, 128, Lmax]) bf16, uninitialised."""
    return (torch.empty((B, Hkv, Lmax, 128), dtype=torch.bfloat16, device=device),
            torch.empty((B, Hkv, 128, Lmax), dtype=torch.bfloat16, device=device))


def gqa_materialize(ctx_hidden: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, gamma_k: torch.Tensor,
                    eps: float, rope, k_cache: torch.Tensor, v_cache_t: torch.Tensor) -> None:
    """Write the context's qk-normed, yarn-RoPE'd keys and its values into the caches."""
    lib = load_library()
    _dev(ctx_hidden, "ctx_hidden", dtype=torch.bfloat16, ndim=3)
    for t, n in ((w_k, "w_k"), (w_v, "w_v")):
        _dev(t, n, dtype=torch.bfloat16, ndim=2)
    _dev(gamma_k, "gamma_k", dtype=torch.bfloat16, ndim=1)
    _dev(k_cache, "k_cache", dtype=torch.bfloat16, ndim=4)
    _dev(v_cache_t, "v_cache_t", dtype=torch.bfloat16, ndim=4)
    B, Lc, hidden = ctx_hidden.shape
    _, Hkv, Lmax, hd = k_cache.shape
    if tuple(v_cache_t.shape) != (B, Hkv, hd, Lmax) or tuple(w_k.shape) != (Hkv * hd, hidden) or w_v.shape != w_k.shape:
        raise ValueError("inconsistent cache / weight shapes")
    _check(lib.dflash_gqa_materialize(_ptr(ctx_hidden), _ptr(w_k), _ptr(w_v), _ptr(gamma_k), float(eps),
                                      ctypes.cast(_rope_array(rope), ctypes.c_void_p), _ptr(k_cache), _ptr(v_cache_t),
                                      B, Lc, Lmax, hidden, Hkv, hd, _stream(ctx_hidden)))


def gqa_forward_block(blk_hidden: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                      gamma_q: torch.Tensor, gamma_k: torch.Tensor, eps: float, rope, k_cache: torch.Tensor,
                      v_cache_t: torch.Tensor, ctx_len: torch.Tensor, Hq: int, scale: Optional[float] = None, *,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A block over [cached context | itself]: appends the block's k / v to the caches
    at ctx_len (int32 [B], device) and returns the attention output [B, Hq, bs, 128]."""
    lib = load_library()
    _dev(blk_hidden, "blk_hidden", dtype=torch.bfloat16, ndim=3)
    _dev(ctx_len, "ctx_len", dtype=torch.int32, ndim=1)
    B, bs, hidden = blk_hidden.shape
    _, Hkv, Lmax, hd = k_cache.shape
    if scale is None:
        scale = hd ** -0.5
    if out is None:
        out = torch.empty((B, Hq, bs, hd), dtype=torch.bfloat16, device=blk_hidden.device)
    _dev(out, "out", dtype=torch.bfloat16, ndim=4)
    if workspace is None:
        n = int(lib.dflash_gqa_workspace_bytes(B, bs, Hq, Hkv, Lmax))
        if n == 0:
            raise ValueError("invalid sizes for the block attention")
        workspace = torch.empty(n, dtype=torch.uint8, device=blk_hidden.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    _check(lib.dflash_gqa_forward_block(_ptr(blk_hidden), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(gamma_q), _ptr(gamma_k),
                                        float(eps), ctypes.cast(_rope_array(rope), ctypes.c_void_p), _ptr(k_cache),
                                        _ptr(v_cache_t), _ptr(ctx_len), _ptr(out), B, bs, Lmax, hidden, Hq, Hkv, hd,
                                        float(scale), _ptr(workspace), workspace.numel(), _stream(blk_hidden)))
    return out
