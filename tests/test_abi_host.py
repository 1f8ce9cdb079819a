"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/dflash_mla.h declares, and argument validation returns the
documented status before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash_mla.h")


@pytest.fixture(scope="module")
def lib():
    from dflash_block_draft_amd import mla
    if not os.path.exists(mla.LIB_PATH):
        from dflash_block_draft_amd import build
        build.build(verbose=False)
    return mla.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ("dflash_mla_latent_expand", "dflash_mla_attn", "dflash_mla_attn_workspace_bytes",
              "dflash_mla_block_occupancy", "dflash_mla_attn_blocks",
              "dflash_mla_mask_occupancy", "dflash_mla_tile_map_layout", "dflash_status_string",
              "dflash_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from dflash_block_draft_amd import mla
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, f"{name} declared in the header but not exported"
        assert getattr(lib, name) is not None
    assert set(mla.EXPORTED) <= exported


def test_status_strings(lib):
    assert lib.dflash_status_string(0) == b"DFLASH_OK"
    assert lib.dflash_status_string(3) == b"DFLASH_ERR_WORKSPACE"
    assert lib.dflash_status_string(99) == b"DFLASH_ERR_UNKNOWN"


def test_workspace_and_layout(lib):
    assert lib.dflash_mla_attn_workspace_bytes(0, 1, 1) == 0
    assert lib.dflash_mla_attn_workspace_bytes(1, -5, 1) == 0
    n = lib.dflash_mla_attn_workspace_bytes(1, 4096, 36864)
    nq, nk = ctypes.c_int64(), ctypes.c_int64()
    offs = [ctypes.c_size_t() for _ in range(5)]
    st = lib.dflash_mla_tile_map_layout(1, 4096, 36864, ctypes.byref(nq), ctypes.byref(nk),
                                        *[ctypes.byref(o) for o in offs])
    assert st == 0
    assert (nq.value, nk.value) == (32, 576)
    c, cnt, lst, order, bits = (o.value for o in offs)
    assert c == 0 and cnt >= 32 * 576 and lst >= cnt + 32 * 4 and order >= lst + 32 * 576 * 4
    assert bits >= order + 32 * 4
    assert all(x % 256 == 0 for x in (c, cnt, lst, order, bits))
    assert n >= bits + 32 * 576 * 128 * 8
    assert lib.dflash_mla_tile_map_layout(1, 0, 5, None, None, None, None, None, None, None) == 1


FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced (validation fails first)


def _attn(lib, **kw):
    args = dict(q=FAKE, kn=FAKE * 2, kr=FAKE * 3, v=FAKE * 4, mask=None, out=FAKE * 5,
                B=1, H=2, Lq=32, Lk=96, Dn=128, Dr=64, Dv=128, scale=192 ** -0.5, dt=1, mdt=0,
                ws=None, wsb=0, flags=0)
    args.update(kw)
    return lib.dflash_mla_attn(args["q"], args["kn"], args["kr"], args["v"], args["mask"], args["out"],
                               args["B"], args["H"], args["Lq"], args["Lk"], args["Dn"], args["Dr"],
                               args["Dv"], args["scale"], args["dt"], args["mdt"], args["ws"],
                               args["wsb"], args["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),                      # null tensor
    (dict(v=FAKE * 4 + 2), 1),              # misaligned
    (dict(Lq=0), 1),                        # empty query axis (no zero-row drafts)
    (dict(B=-1), 1),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(dt=7), 1),
    (dict(flags=0x80), 1),
    (dict(Dn=64), 2),                       # head dims the library does not implement
    (dict(Dr=32), 2),
    (dict(Dv=64), 2),
    (dict(dt=0, mdt=1, mask=FAKE * 8), 2),  # f32 attention with a bf16 mask
    (dict(out=FAKE * 4), 1),                # out aliases v
    (dict(mask=FAKE * 100), 3),             # masked bf16 call without a workspace
    (dict(mask=FAKE * 100, ws=FAKE * 400, wsb=16), 3),   # workspace too small
    (dict(mask=FAKE * 100, ws=FAKE * 400 + 16, wsb=1 << 20), 3),  # workspace misaligned
    (dict(q=1 << 44, kn=2 << 44, kr=3 << 44, v=4 << 44, out=5 << 44, mask=6 << 44, Lk=1 << 30,
          ws=7 << 44, wsb=1 << 40), 2),     # masked bf16 call with 2^24 key tiles
    (dict(q=1 << 44, kn=2 << 44, kr=3 << 44, v=4 << 44, out=5 << 44, Lk=1 << 30), 2),   # unmasked, same limit
    (dict(q=1 << 44, kn=2 << 44, kr=3 << 44, v=4 << 44, out=5 << 44, Lk=1 << 23), 2),   # k_nope slice of 2^31 bytes
])
def test_attn_validation(lib, kw, status):
    assert _attn(lib, **kw) == status
    assert lib.dflash_last_error() != b""


def test_attn_largest_bf16_key_count_passes_validation(lib):
    # 2^23 - 1 keys: the (batch, head) slice of k_nope is just under 2^31 bytes (CHECK_ONLY launches nothing)
    kw = dict(q=1 << 44, kn=2 << 44, kr=3 << 44, v=4 << 44, out=5 << 44, Lk=(1 << 23) - 1, flags=0x4)
    assert _attn(lib, **kw) == 0


def test_expand_validation(lib):
    f = lib.dflash_mla_latent_expand
    assert f(None, FAKE, FAKE * 2, FAKE * 3, 1, 4, 512, 2, 128, 128, 1, None) == 1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, 4, 500, 2, 128, 128, 1, None) == 2   # R % 32
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, 4, 512, 2, 64, 128, 1, None) == 2    # Dn
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 3, 1, 4, 512, 2, 128, 128, 1, None) == 1   # k_nope aliases v
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 0, 4, 512, 2, 128, 128, 1, None) == 1


def test_occupancy_validation(lib):
    f = lib.dflash_mla_mask_occupancy
    assert f(None, 0, 1, 32, 96, FAKE * 256, 1 << 20, None) == 1
    assert f(FAKE, 0, 1, 32, 96, None, 0, None) == 3
    assert f(FAKE, 5, 1, 32, 96, FAKE * 256, 1 << 20, None) == 1


def test_python_binding_rejects_host_tensors():
    import torch
    from dflash_block_draft_amd import mla
    x = torch.zeros(1, 1, 4, 192)
    with pytest.raises((ValueError, RuntimeError)):
        mla.mla_attn(x, x, x, x)


def _blocks(lib, **kw):
    args = dict(q=FAKE, kn=FAKE * 2, kr=FAKE * 3, v=FAKE * 4, anchors=FAKE * 6, cv=None, out=FAKE * 5,
                B=1, H=2, A=2, bs=16, ctx=64, Dn=128, Dr=64, Dv=128, scale=192 ** -0.5, dt=1,
                ws=FAKE * 256, wsb=1 << 20, flags=0)
    args.update(kw)
    return lib.dflash_mla_attn_blocks(args["q"], args["kn"], args["kr"], args["v"], args["anchors"], args["cv"],
                                      args["out"], args["B"], args["H"], args["A"], args["bs"], args["ctx"],
                                      args["Dn"], args["Dr"], args["Dv"], args["scale"], args["dt"], args["ws"],
                                      args["wsb"], args["flags"], None)


# every case fails validation, so nothing is launched
@pytest.mark.parametrize("kw,status", [
    (dict(anchors=None), 1),
    (dict(anchors=FAKE * 6 + 2), 1),        # misaligned anchors
    (dict(cv=FAKE * 7 + 1), 1),             # misaligned ctx_valid
    (dict(A=0), 1),
    (dict(bs=0), 1),
    (dict(ctx=-1), 1),
    (dict(flags=0x2), 1),                   # tile-skip switch is not offered here
    (dict(flags=0x4), 1),
    (dict(dt=0), 2),                        # f32: the block path is bf16 only
    (dict(ws=None, wsb=0), 3),
    (dict(wsb=16), 3),
    (dict(ws=FAKE * 256 + 16), 3),
    (dict(ws=FAKE * 6), 1),                 # workspace overlaps anchors
    (dict(ws=FAKE * 4), 1),                 # workspace overlaps v
    (dict(out=FAKE * 6), 1),                # out overlaps anchors
    (dict(out=FAKE * 4), 1),                # out aliases v
    (dict(Dv=64), 2),
    (dict(scale=0.0), 1),
    (dict(A=1 << 20, bs=1 << 12), 2),       # Lq beyond int32
    (dict(q=1 << 44, kn=2 << 44, kr=3 << 44, v=4 << 44, out=5 << 44, anchors=6 << 44, ws=7 << 44,
          wsb=1 << 40, ctx=1 << 30), 2),    # 2^24 key tiles
])
def test_attn_blocks_validation(lib, kw, status):
    assert _blocks(lib, **kw) == status
    assert lib.dflash_last_error() != b""


def test_block_occupancy_validation(lib):
    f = lib.dflash_mla_block_occupancy
    assert f(None, None, 1, 2, 16, 64, FAKE * 256, 1 << 20, None) == 1
    assert f(FAKE + 1, None, 1, 2, 16, 64, FAKE * 256, 1 << 20, None) == 1
    assert f(FAKE, None, 0, 2, 16, 64, FAKE * 256, 1 << 20, None) == 1
    assert f(FAKE, None, 1, 2, 16, -3, FAKE * 256, 1 << 20, None) == 1
    assert f(FAKE, None, 1, 2, 16, 64, None, 0, None) == 3
    assert f(FAKE, None, 1, 2, 16, 64, FAKE * 256, 64, None) == 3
    assert f(FAKE * 256, None, 1, 2, 16, 64, FAKE * 256, 1 << 20, None) == 1   # overlap


def test_block_binding_rejects_bad_tensors():
    import torch
    from dflash_block_draft_amd import mla
    with pytest.raises(ValueError):
        mla.block_occupancy(torch.zeros(1, 2, dtype=torch.int32), 16, 64)        # host tensor


def _bwd(lib, **kw):
    args = dict(q=FAKE, kn=FAKE * 2, kr=FAKE * 3, v=FAKE * 4, mask=None, out=FAKE * 5, dout=FAKE * 6,
                lse=FAKE * 7, dq=FAKE * 8, dkn=FAKE * 9, dkr=FAKE * 10, dv=FAKE * 11, B=1, H=2, Lq=32, Lk=96,
                Dn=128, Dr=64, Dv=128, scale=192 ** -0.5, dt=1, mdt=0, ws=FAKE * 256, wsb=1 << 24, flags=0)
    args.update(kw)
    k = ["q", "kn", "kr", "v", "mask", "out", "dout", "lse", "dq", "dkn", "dkr", "dv", "B", "H", "Lq", "Lk",
         "Dn", "Dr", "Dv", "scale", "dt", "mdt", "ws", "wsb", "flags"]
    return lib.dflash_mla_attn_bwd(*[args[n] for n in k], None)


def test_bwd_workspace_bytes(lib):
    assert lib.dflash_mla_attn_bwd_workspace_bytes(1, 2, 0, 96) == 0
    assert lib.dflash_mla_attn_bwd_workspace_bytes(1, 0, 32, 96) == 0
    n = lib.dflash_mla_attn_bwd_workspace_bytes(1, 64, 1024, 9216)
    # tile map + lse2/D + q^T + dout^T (padded queries) + k_nope^T + k_rope^T + per-head rope parts
    assert n >= lib.dflash_mla_attn_workspace_bytes(1, 1024, 9216) + 64 * 1024 * (8 + 2 * 320) \
        + 64 * 9216 * 2 * 128 + 9216 * 2 * 64 + 64 * 9216 * 64 * 4


# every case fails validation, so nothing is launched
@pytest.mark.parametrize("kw,status", [
    (dict(dout=None), 1),
    (dict(lse=FAKE * 7 + 2), 1),              # lse misaligned
    (dict(dq=FAKE * 8 + 8), 1),
    (dict(Lq=0), 1),
    (dict(scale=-1.0), 1),
    (dict(flags=0x2), 1),                     # only REUSE_TILE_MAP is accepted
    (dict(dt=0), 2),                          # f32 backward is not built
    (dict(Dr=32), 2),
    (dict(B=300, H=300), 2),                  # B * H beyond one grid dimension
    (dict(ws=None, wsb=0), 3),
    (dict(wsb=64), 3),
    (dict(ws=FAKE * 256 + 16), 3),
    (dict(dq=FAKE), 1),                       # dq aliases q
    (dict(dv=FAKE * 10), 1),                  # dv aliases dk_rope
    (dict(ws=FAKE * 2), 1),                   # workspace overlaps k_nope
])
def test_attn_bwd_validation(lib, kw, status):
    assert _bwd(lib, **kw) == status
    assert lib.dflash_last_error() != b""


def test_attn_lse_validation(lib):
    f = lib.dflash_mla_attn_lse
    base = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, FAKE * 5]
    tail = [1, 2, 32, 96, 128, 64, 128, 192 ** -0.5, 1, 0, None, 0, 0, None]
    assert f(*base, None, *tail) == 1                       # lse NULL
    assert f(*base, FAKE * 5, *tail) == 1                   # lse overlaps out
    assert f(*base, FAKE * 6 + 1, *tail) == 1               # misaligned


def test_projection_workspace_bytes(lib):
    assert lib.dflash_mla_projection_workspace_bytes(0, 128) == 0
    assert lib.dflash_mla_projection_workspace_bytes(1000, 512) >= 1000 * 512 * 2 + 1000 * 4 * 4


def test_projection_validation(lib):
    cp, qp, kvp = lib.dflash_mla_context_project, lib.dflash_mla_q_project, lib.dflash_mla_kv_project
    ws, wsb = FAKE * 256, 1 << 26
    # context: (th, w_fc, gamma, eps, out, B, ctx, K_in, hidden, ws, wsb, stream)
    assert cp(None, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, 1, 64, 256, 128, ws, wsb, None) == 1
    assert cp(FAKE, FAKE * 2, FAKE * 3, -1.0, FAKE * 4, 1, 64, 256, 128, ws, wsb, None) == 1   # eps < 0
    assert cp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, 1, 64, 250, 128, ws, wsb, None) == 2   # K_in % 32
    assert cp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, 1, 64, 256, 100, ws, wsb, None) == 2   # hidden % 128
    assert cp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, 1, 64, 256, 128, None, 0, None) == 3
    assert cp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE, 1, 64, 256, 128, ws, wsb, None) == 1       # out aliases input
    # q: (x, wqa, gq, eps, wqb, q, B, Lq, hidden, Rq, H, Dqk, ws, wsb, stream)
    assert qp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, FAKE * 5, 1, 32, 256, 100, 2, 192, ws, wsb, None) == 2  # Rq % 128
    assert qp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, FAKE * 5, 1, 32, 256, 128, 2, 190, ws, wsb, None) == 2  # Dqk % 4
    assert qp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, FAKE * 5, 1, 0, 256, 128, 2, 192, ws, wsb, None) == 1
    assert qp(FAKE, FAKE * 2, FAKE * 3, 1e-6, FAKE * 4, FAKE * 5, 1, 32, 256, 128, 2, 192, ws, 64, None) == 3
    # kv: (ctx_h, noise_h, wkva, gkv, eps, wkvb, kn, kr, v, B, ctx, Lq, hidden, R, Dr, H, Dn, Dv, ws, wsb, stream)
    args = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1e-6, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8,
            1, 64, 32, 256, 512, 64, 2, 128, 128, ws, wsb, None]
    bad = list(args); bad[0] = None
    assert kvp(*bad) == 1                                   # ctx > 0 needs ctx_hidden
    bad = list(args); bad[13] = 500
    assert kvp(*bad) == 2                                   # R % 128
    bad = list(args); bad[16] = 64
    assert kvp(*bad) == 2                                   # Dn
    bad = list(args); bad[6] = FAKE * 8
    assert kvp(*bad) == 1                                   # k_nope overlaps v


def test_gqa_validation(lib):
    import ctypes as C
    rope = (C.c_float * 7)(50000.0, 32.0, 4096.0, 32.0, 1.0, 1.0, 1.0)
    bad_rope = (C.c_float * 7)(0.5, 32.0, 4096.0, 32.0, 1.0, 1.0, 1.0)
    mat = lib.dflash_gqa_materialize
    # (ctx, wk, wv, gk, eps, rope, kc, vc, B, Lc, Lmax, hidden, Hkv, hd, stream)
    good = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1e-6, C.cast(rope, C.c_void_p), FAKE * 64, FAKE * 128,
            1, 64, 128, 256, 2, 128, None]
    for idx, val, status in ((0, None, 1), (5, None, 1), (5, C.cast(bad_rope, C.c_void_p), 1), (9, 200, 1),
                             (13, 64, 2), (10, 130, 2), (11, 250, 2), (7, FAKE * 64, 1)):
        args = list(good)
        args[idx] = val
        assert mat(*args) == status, (idx, val)
    fb = lib.dflash_gqa_forward_block
    # (blk, wq, wk, wv, gq, gk, eps, rope, kc, vc, ctx_len, out, B, bs, Lmax, hidden, Hq, Hkv, hd, scale, ws, wsb, stream)
    good = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6, 1e-6, C.cast(rope, C.c_void_p), FAKE * 64,
            FAKE * 128, FAKE * 7, FAKE * 8, 1, 16, 128, 256, 8, 2, 128, 0.088, FAKE * 256, 1 << 26, None]
    for idx, val, status in ((10, None, 1), (10, FAKE * 7 + 2, 1), (16, 7, 2), (13, 32, 2), (13, 200, 1),
                             (19, 0.0, 1), (20, None, 3), (21, 64, 3), (11, FAKE * 64, 1),
                             (14, 1 << 23, 2)):                 # a cache slice beyond a 32-bit buffer range
        args = list(good)
        args[idx] = val
        assert fb(*args) == status, (idx, val)
    assert lib.dflash_gqa_workspace_bytes(1, 16, 8, 2, 128) > 0
    assert lib.dflash_gqa_workspace_bytes(0, 16, 8, 2, 128) == 0


def test_map_only_reuse_validation(lib):
    # mask NULL + REUSE_TILE_MAP: bf16 needs the workspace; f32 and NO_TILE_SKIP are rejected
    assert _attn(lib, flags=0x1) == 3
    assert _attn(lib, flags=0x1, dt=0) == 1
    assert _attn(lib, flags=0x3, ws=FAKE * 256, wsb=1 << 20) == 1


def test_split_keys_workspace_bytes(lib):
    mb, sb = lib.dflash_mla_attn_workspace_bytes, lib.dflash_mla_attn_split_workspace_bytes
    # 512 items fit one round of two workgroups per CU: 2 runs each
    rows2, m2 = 64 * 1024, mb(1, 1024, 9216)
    assert m2 + 2 * rows2 * (128 * 2 + 4) <= sb(1, 64, 1024, 9216) <= m2 + 2 * rows2 * (128 * 2 + 4) + 3 * 256
    assert sb(1, 32, 4096, 36864) == mb(1, 4096, 36864)    # 1024 items: no split, the map alone
    assert sb(1, 2, 32, 96) == mb(1, 32, 96)               # 2 k-tiles: too short to split
    # 2 batches x 2 q-tiles x 16 heads = 64 items over 36 k-tiles: 8 runs (a run
    # of the whole key range keeps 36 / 8 = 4.5 >= 4 k-tiles)
    rows, m = 2 * 16 * 256, mb(2, 256, 2304)
    n = sb(2, 16, 256, 2304)
    assert m + 8 * rows * (128 * 2 + 4) <= n <= m + 8 * rows * (128 * 2 + 4) + 3 * 256
    # 64 items over 28 k-tiles: 4 runs (8 would leave 28 / 8 = 3.5 < 4 k-tiles per run)
    n4 = sb(2, 16, 256, 1792)
    assert mb(2, 256, 1792) + 4 * rows * (128 * 2 + 4) <= n4 <= mb(2, 256, 1792) + 4 * rows * (128 * 2 + 4) + 3 * 256
    # 1 x 1 q-tile x 8 heads over 129 k-tiles: 8 runs (the cap)
    n8 = sb(1, 8, 16, 8208)
    assert n8 >= mb(1, 16, 8208) + 8 * 8 * 16 * (128 * 2 + 4)
    assert sb(0, 1, 32, 96) == 0 and sb(1, 0, 32, 96) == 0 and sb(1, 1, 0, 96) == 0


def test_split_keys_validation(lib):
    big = dict(q=1 << 40, kn=2 << 40, kr=3 << 40, v=4 << 40, out=5 << 40, B=2, H=16, Lq=256, Lk=2304)
    need = lib.dflash_mla_attn_split_workspace_bytes(2, 16, 256, 2304)
    ws = 6 << 40
    assert _attn(lib, flags=0x8, **big) == 3                               # a split shape needs the workspace
    assert _attn(lib, flags=0x8, ws=ws, wsb=need - 256, **big) == 3        # too small for the partials
    assert _attn(lib, flags=0x8, ws=ws + 16, wsb=need, **big) == 1         # misaligned
    assert _attn(lib, flags=0x8, ws=(4 << 40) + 256, wsb=need, **big) == 1  # overlaps v
    assert _attn(lib, flags=0xC, ws=ws, wsb=need, **big) == 0              # valid (check only)
    assert _attn(lib, flags=0xC, dt=0, **big) == 0                         # f32 ignores the split
    assert _attn(lib, flags=0xE, **big) == 0                               # ignored with NO_TILE_SKIP (no mask)
    assert _attn(lib, flags=0xC, ws=None, wsb=0) == 0                      # a shape that does not split


def test_no_alloc_validation(lib):
    f = lib.dflash_mla_attn_no_alloc
    base = (FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 100, FAKE * 5, 1, 2, 32, 96, 128, 64, 128, 192 ** -0.5, 1, 1)
    assert f(*base, 0x4, None) == 0                         # valid (check only: nothing launched)
    assert f(*base, 0x1, None) == 1                         # REUSE_TILE_MAP: the scratch holds no map to reuse
    assert f(*base, 0x8, None) == 1                         # SPLIT_KEYS: no room for partials
    assert f(*base[:6], 0, 2, 32, 96, *base[10:], 0x4, None) == 1     # B = 0
    big = (1 << 44, 2 << 44, 3 << 44, 4 << 44, 5 << 44, 6 << 44)
    # a tile map past the static scratch: UNSUPPORTED
    assert mla_ws(lib, 1, 128 * 64, 64 * 600) > 32 << 20
    assert f(*big, 1, 1, 128 * 64, 64 * 600, 128, 64, 128, 0.07, 1, 1, 0x4, None) == 2
    assert b"scratch" in lib.dflash_last_error()
    # the largest map that fits is accepted
    assert f(*big, 1, 1, 128 * 32, 64 * 576, 128, 64, 128, 0.07, 1, 1, 0x4, None) == 0


def mla_ws(lib, B, Lq, Lk):
    return lib.dflash_mla_attn_workspace_bytes(B, Lq, Lk)
