"""HIP path vs the fp64 oracle, through the C ABI (gfx950 GPU required).

Tolerances (absolute, on the output): fp32 inputs max|err| <= 1e-5; bf16
inputs max|err| <= 1.5e-2 and mean|err| <= 1e-3.  The oracle always runs on
exactly the values the GPU consumed (bf16/f32 upcast to fp64).  Every
workload is compared over its whole output (all of B*H*Lq*Dv); the longest
one in four groups of heads, so each oracle call takes seconds.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dflash_block_draft_amd import mla
from dflash_block_draft_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16_MAX = 1.5e-2
TOL_BF16_MEAN = 1e-3


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    mla.load_library()
    return torch.device("cuda:0")


def _to(dev, *ts):
    return [None if t is None else t.to(dev) for t in ts]


def _err(out_gpu, ref):
    d = np.abs(out_gpu.detach().to("cpu", torch.float64).numpy() - ref)
    return float(d.max()), float(d.mean())


def _check(out_gpu, ref, dtype, what):
    mx, mean = _err(out_gpu, ref)
    say(f"{what}: max|err|={mx:.3e} mean|err|={mean:.3e}")
    if dtype == "f32":
        assert mx <= TOL_F32, what
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, what


def _attn_case(dev, wl, rows=None, **kw):
    say(f"{wl.name}: B={wl.B} H={wl.H} Lq={wl.Lq} Lk={wl.Lk} dtype={wl.dtype} mask={wl.mask_dtype}")
    q, kn, kr, v, m = _to(dev, wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale, **kw)
    torch.cuda.synchronize()
    ref = oracle.mla_attention(wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask, wl.scale, q_rows=rows)
    got = out if rows is None else out[:, :, torch.as_tensor(rows, device=dev)]
    _check(got, ref, wl.dtype, wl.name)
    return out


# ------------------------------------------------------------- the five workloads

def test_config0_f32(dev):
    _attn_case(dev, W.config(0))


def test_config1_expand_then_attention(dev):
    wl = W.config(1)
    lat, w, q, kr, m = _to(dev, wl.latent, wl.w_kv_b, wl.q, wl.k_rope, wl.mask)
    say("config1 expand")
    kn, v = mla.latent_expand(lat, w, wl.H)
    torch.cuda.synchronize()
    ref_kn, ref_v = oracle.latent_expand(wl.latent, wl.w_kv_b, wl.H, wl.Dn, wl.Dv)
    for name, got, ref in (("k_nope", kn, ref_kn), ("v", v, ref_v)):
        g = got.to("cpu", torch.float64).numpy()
        # within one bf16 rounding of the fp64 value: |g - ref| <= 2^-8 |ref| (+ tiny abs)
        bound = np.abs(ref) * 2.0 ** -8 + 1e-6
        assert np.all(np.abs(g - ref) <= bound), name
        say(f"expand {name}: max|err|={np.abs(g - ref).max():.3e}")
    say("config1 attention on the expanded k/v")
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale)
    torch.cuda.synchronize()
    # end to end: the oracle's attention on the oracle's own fp64 expansion (the GPU
    # path rounded its k/v to bf16 first, which the bf16 tolerance covers)
    ref_e2e = oracle.mla_attention(wl.q, ref_kn, wl.k_rope, ref_v, wl.mask, wl.scale)
    _check(out, ref_e2e, "bf16", "config1 end-to-end (fp64 expand)")


def test_config2_whole(dev):
    _attn_case(dev, W.config(2))


@pytest.mark.parametrize("bs", [8, 32])
def test_config3_whole(dev, bs):
    _attn_case(dev, W.config(3, block_size=bs))


@pytest.fixture(scope="module")
def config4_out(dev):
    wl = W.config(4)
    say(f"{wl.name}: B={wl.B} H={wl.H} Lq={wl.Lq} Lk={wl.Lk}")
    q, kn, kr, v, m = _to(dev, wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask)
    out = mla.mla_attn(q, kn, kr, v, m, wl.scale)
    torch.cuda.synchronize()
    return wl, out.cpu()


@pytest.mark.parametrize("group", range(4))
def test_config4_whole(config4_out, group):
    """All rows of heads 8g .. 8g+7; the four groups together are the whole output
    (each group's mean bound implies the bound on the mean of all four)."""
    wl, out = config4_out
    hs = slice(8 * group, 8 * group + 8)
    ref = oracle.mla_attention(wl.q[:, hs], wl.k_nope[:, hs], wl.k_rope, wl.v[:, hs], wl.mask, wl.scale)
    _check(out[:, hs], ref, wl.dtype, f"{wl.name} heads {hs.start}-{hs.stop - 1}")


# ------------------------------------------------------------- ragged and edge cases

@pytest.mark.parametrize("dtype,mdt", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
def test_ragged_tiles(dev, dtype, mdt):
    # Lq = 35 (one partial q-tile), Lk = 100 + 35 = 135 (three k-tiles, the last partial)
    wl = W.custom(seed=11, B=2, H=3, ctx=100, A=5, bs=7, dtype=dtype, mask_dtype=mdt)
    _attn_case(dev, wl)


def test_several_tiles_and_ragged_tail(dev):
    # Lq = 300 (3 q-tiles), Lk = 700 + 300 = 1000 (16 k-tiles, last one 40 wide)
    wl = W.custom(seed=12, B=1, H=4, ctx=700, A=20, bs=15, dtype="bf16", mask_dtype="f32")
    _attn_case(dev, wl)


def test_odd_lk_scalar_mask_path(dev):
    # Lk odd: mask rows are not 16-byte aligned -> scalar classification and loads
    wl = W.custom(seed=13, B=2, H=2, ctx=101, A=4, bs=8, dtype="bf16", mask_dtype="bf16")
    assert wl.Lk % 2 == 1
    _attn_case(dev, wl)


def test_no_mask_equals_zero_mask_and_oracle(dev):
    q, kn, kr, v = W.random_attention_inputs(14, 2, 3, 200, 333, dtype="bf16")
    zero = torch.zeros(2, 1, 200, 333, dtype=torch.float32)
    qd, knd, krd, vd, zd = _to(dev, q, kn, kr, v, zero)
    a = mla.mla_attn(qd, knd, krd, vd, None)
    b = mla.mla_attn(qd, knd, krd, vd, zd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.mla_attention(q, kn, kr, v, None, 192 ** -0.5)
    _check(a, ref, "bf16", "no-mask")


def test_general_additive_mask(dev):
    """Finite non-zero mask values (general tiles everywhere) plus -inf holes.
    Mask values ~ N(0, 3^2) make the softmax far peakier than the DFlash
    workloads; the bf16 bounds still hold."""
    B, H, Lq, Lk = 2, 2, 160, 300
    q, kn, kr, v = W.random_attention_inputs(15, B, H, Lq, Lk, dtype="bf16")
    rng = np.random.default_rng(15)
    m = rng.standard_normal((B, 1, Lq, Lk)).astype(np.float32) * 3.0
    m[rng.random(m.shape) < 0.3] = -np.inf
    m[..., 0] = 0.0
    for mdt in (torch.float32, torch.bfloat16):
        mask = torch.from_numpy(m).to(mdt)
        qd, knd, krd, vd, md = _to(dev, q, kn, kr, v, mask)
        out = mla.mla_attn(qd, knd, krd, vd, md)
        torch.cuda.synchronize()
        ref = oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5)
        _check(out, ref, "bf16", f"general mask {mdt}")


def test_fully_masked_rows_and_huge_negatives(dev):
    B, H, Lq, Lk = 1, 2, 140, 200
    q, kn, kr, v = W.random_attention_inputs(16, B, H, Lq, Lk, dtype="bf16")
    m = np.zeros((B, 1, Lq, Lk), dtype=np.float32)
    m[0, 0, 3, :] = -np.inf                          # fully masked row -> 0
    m[0, 0, 130:140, :] = -np.inf                    # rows in the partial q-tile, fully masked
    fmin = np.finfo(np.float32).min
    m[0, 0, 5, :] = fmin                             # every entry a huge finite negative
    m[0, 0, 7, 100:] = fmin                          # half visible, half huge negative
    mask = torch.from_numpy(m)
    qd, knd, krd, vd, md = _to(dev, q, kn, kr, v, mask)
    out = mla.mla_attn(qd, knd, krd, vd, md)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.all(o[0, :, 3] == 0) and torch.all(o[0, :, 130:140] == 0)
    ref = oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5)
    _check(out, ref, "bf16", "dead rows / finfo.min rows")


def test_huge_negative_tile_then_binary_tiles(dev):
    """A first key tile of huge finite negatives (a general tile: the stabiliser
    becomes about -3.4e38), then binary 0 / -inf tiles.  There the fast path's
    exponent offset overflows, and the tile must be redone on the exact path; rows
    whose binary tiles hide every key keep the softmax over the huge negatives,
    which in fp32 and fp64 alike is the plain mean of their values."""
    B, H, Lq, Lk = 1, 2, 128, 384
    q, kn, kr, v = W.random_attention_inputs(19, B, H, Lq, Lk, dtype="bf16")
    rng = np.random.default_rng(19)
    m = np.where(rng.random((B, 1, Lq, Lk)) < 0.5, 0.0, -np.inf).astype(np.float32)
    m[..., :64] = float(torch.finfo(torch.bfloat16).min)   # representable in both mask dtypes
    m[0, 0, 10:20, 64:] = -np.inf
    for mdt in (torch.float32, torch.bfloat16):
        mask = torch.from_numpy(m).to(mdt)
        qd, knd, krd, vd, md = _to(dev, q, kn, kr, v, mask)
        out = mla.mla_attn(qd, knd, krd, vd, md)
        torch.cuda.synchronize()
        ref = oracle.mla_attention(q, kn, kr, v, mask, 192 ** -0.5)
        _check(out, ref, "bf16", f"huge-negative tile then binary tiles, {mdt}")


def test_largest_key_count(dev):
    """The largest bf16 key count, 2^23 - 1: one (batch, head) slice of k_nope / v
    is just under 2^31 bytes, the limit of the kernel's 32-bit buffer ranges, and
    the last (ragged, binary) key tile sits at byte offsets just below it.  One DFlash
    block of 16 queries whose anchor is 1000 sees 1001 context keys and its own 16
    noise keys at the very end.  K / V are drawn on the device (seeded); the oracle
    gets the visible keys only -- exact, since every other key has weight 0."""
    Lk, bs, anchor = (1 << 23) - 1, 16, 1000
    ctx = Lk - bs
    gen = torch.Generator(device=dev)
    gen.manual_seed(23)
    say(f"largest key count: Lk={Lk}")
    q = torch.randn((1, 1, bs, 192), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((1, 1, Lk, 128), generator=gen, device=dev).to(torch.bfloat16)
    kr = torch.randn((1, Lk, 64), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((1, 1, Lk, 128), generator=gen, device=dev).to(torch.bfloat16)
    mask = torch.full((1, 1, bs, Lk), float("-inf"), dtype=torch.bfloat16, device=dev)
    mask[..., :anchor + 1] = 0
    mask[..., ctx:] = 0
    out = mla.mla_attn(q, kn, kr, v, mask)
    anchors = torch.tensor([[anchor]], dtype=torch.int32, device=dev)
    out_blocks = mla.mla_attn_blocks(q, kn, kr, v, anchors, bs, ctx)
    torch.cuda.synchronize()
    assert torch.equal(out, out_blocks)
    cols = torch.cat([torch.arange(anchor + 1), torch.arange(ctx, Lk)]).to(dev)
    ref = oracle.mla_attention(q.cpu(), kn[:, :, cols].cpu(), kr[:, cols].cpu(), v[:, :, cols].cpu(),
                               mask[..., cols].cpu(), 192 ** -0.5)
    _check(out, ref, "bf16", "largest key count")
    del q, kn, kr, v, mask, out, out_blocks
    torch.cuda.empty_cache()


def test_single_visible_key_returns_its_value(dev):
    B, H, Lq, Lk = 2, 3, 64, 130
    q, kn, kr, v = W.random_attention_inputs(17, B, H, Lq, Lk, dtype="bf16")
    rng = np.random.default_rng(17)
    js = rng.integers(0, Lk, size=(B, Lq))
    m = np.full((B, 1, Lq, Lk), -np.inf, dtype=np.float32)
    for b in range(B):
        m[b, 0, np.arange(Lq), js[b]] = 0.0
    qd, knd, krd, vd, md = _to(dev, q, kn, kr, v, torch.from_numpy(m))
    out = mla.mla_attn(qd, knd, krd, vd, md)
    torch.cuda.synchronize()
    o = out.cpu()
    for b in range(B):
        want = v[b][:, torch.as_tensor(js[b])]
        assert torch.equal(o[b], want)


# ------------------------------------------------------------- occupancy, skip, determinism

def _tile_map_masks():
    """Masks for the occupancy pass: 16-byte-aligned rows (Lk % 8 == 0 for bf16,
    % 4 == 0 for f32; the vectorised path) and unaligned rows (the per-entry path),
    with ragged last tiles, plus one with general values, NaN and +inf entries."""
    yield W.config(2).mask
    yield W.custom(seed=18, B=3, H=1, ctx=450, A=9, bs=16, mask_dtype="f32").mask      # Lk 594: per-entry f32
    yield W.custom(seed=21, B=2, H=1, ctx=452, A=9, bs=16, mask_dtype="f32").mask      # Lk 596: vector f32, ragged
    yield W.custom(seed=22, B=2, H=1, ctx=456, A=9, bs=16, mask_dtype="bf16").mask     # Lk 600: vector bf16, ragged
    yield W.custom(seed=23, B=1, H=1, ctx=455, A=9, bs=16, mask_dtype="bf16").mask     # Lk 599: per-entry bf16
    for dt in ("f32", "bf16"):
        m = W.custom(seed=24, B=1, H=1, ctx=504, A=8, bs=16, mask_dtype=dt).mask.clone()   # Lk 632
        m[0, 0, 3, 5] = 0.5           # general value inside an otherwise binary tile
        m[0, 0, 70, 200] = float("nan")
        m[0, 0, 100, 400] = float("inf")
        m[0, 0, 1, 600:632] = -2.0    # general values in the ragged last tile
        yield m


def test_tile_map_exact(dev):
    for mask in _tile_map_masks():
        B, _, Lq, Lk = mask.shape
        say(f"tile map {tuple(mask.shape)} {mask.dtype}")
        md = mask.to(dev)
        ws = mla.mask_occupancy(md)
        torch.cuda.synchronize()
        tm = mla.tile_map_view(ws, B, Lq, Lk)
        want = oracle.tile_classes(mask, mla.TILE_M, mla.TILE_N)
        got = tm["classes"].cpu().numpy()
        assert np.array_equal(got, want)
        counts = tm["counts"].cpu().numpy()
        lists = tm["lists"].cpu().numpy()
        for b, row in enumerate(oracle.tile_lists(want)):
            for qt, (idx, cls) in enumerate(row):
                assert counts[b, qt] == len(idx)
                ent = lists[b, qt, :len(idx)]
                assert np.array_equal(ent & 0xFFFFFF, idx) and np.array_equal(ent >> 24, cls)
        flat = counts.reshape(-1)
        order = tm["order"].cpu().numpy()
        want_order = sorted(range(flat.size), key=lambda i: (-flat[i], i))
        assert list(order) == want_order
        want_bits = oracle.tile_bits(mask, mla.TILE_M, mla.TILE_N, want)
        got_bits = tm["bits"].cpu().numpy().view(np.uint64)
        sel = want == 2
        assert sel.sum() > 0
        assert np.array_equal(got_bits[sel], want_bits[sel])


def test_tile_map_many_rows_order(dev):
    """More (b, q-tile) rows than the list pass ranks itself: the separate ranking
    kernel orders them (decreasing count, ties by index)."""
    rng = np.random.default_rng(25)
    B, Lq, Lk = 3, 128 * 200, 130                       # 600 rows, 3 k-tiles (one ragged)
    m = np.full((B, 1, Lq, Lk), -np.inf, dtype=np.float32)
    vis = rng.random((B, Lq // 128, 3)) < 0.5
    for b, qt, kt in zip(*np.nonzero(vis)):
        r = qt * 128 + rng.integers(0, 128)
        m[b, 0, r, kt * 64 + rng.integers(0, min(64, Lk - kt * 64))] = 0.0
    mask = torch.from_numpy(m).to(torch.bfloat16)
    ws = mla.mask_occupancy(mask.to(dev))
    torch.cuda.synchronize()
    tm = mla.tile_map_view(ws, B, Lq, Lk)
    want = oracle.tile_classes(mask, mla.TILE_M, mla.TILE_N)
    assert np.array_equal(tm["classes"].cpu().numpy(), want)
    flat = tm["counts"].cpu().numpy().reshape(-1)
    assert np.array_equal(flat, (want != 0).sum(-1).reshape(-1))
    want_order = sorted(range(flat.size), key=lambda i: (-flat[i], i))
    assert list(tm["order"].cpu().numpy()) == want_order


def test_skip_on_equals_skip_off_bitwise(dev):
    wl = W.custom(seed=19, B=2, H=4, ctx=900, A=12, bs=16, dtype="bf16", mask_dtype="bf16")
    q, kn, kr, v, m = _to(dev, wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask)
    a = mla.mla_attn(q, kn, kr, v, m, tile_skip=True, split_keys=False)   # (visiting every tile is unsplit)
    b = mla.mla_attn(q, kn, kr, v, m, tile_skip=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_deterministic_and_reuse_tile_map(dev):
    wl = W.custom(seed=20, B=1, H=8, ctx=1500, A=24, bs=16, dtype="bf16", mask_dtype="f32")
    q, kn, kr, v, m = _to(dev, wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask)
    ws = mla.new_workspace(wl.B, wl.Lq, wl.Lk, dev, H=wl.H)   # 24 work items: split over keys
    assert ws.numel() > mla.attn_workspace_bytes(wl.B, wl.Lq, wl.Lk)
    a = mla.mla_attn(q, kn, kr, v, m, workspace=ws)
    b = mla.mla_attn(q, kn, kr, v, m, workspace=ws)
    q2 = torch.flip(q, dims=[1]).contiguous()               # "next layer": new q, same mask
    c = mla.mla_attn(q2, kn, kr, v, m, workspace=ws, reuse_tile_map=True)
    d = mla.mla_attn(q2, kn, kr, v, m)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(c, d)


def test_non_default_stream(dev):
    wl = W.custom(seed=21, B=1, H=2, ctx=300, A=6, bs=16, dtype="bf16", mask_dtype="f32")
    q, kn, kr, v, m = _to(dev, wl.q, wl.k_nope, wl.k_rope, wl.v, wl.mask)
    ref = mla.mla_attn(q, kn, kr, v, m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = mla.mla_attn(q, kn, kr, v, m)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# ------------------------------------------------------------- expand
@pytest.mark.gpu
def test_expand_deep_tile_ragged(dev):
    """The expand's one-round tile path (288 rows x 256 outputs per workgroup,
    chosen when those tiles fill the chip once): 4600 rows (a ragged last row
    tile), R = 512, 16 heads, bf16, against the fp64 definition."""
    rng = np.random.default_rng(23)
    B, Lk, R, H = 2, 2300, 512, 16
    lat = W.normal(rng, (B, Lk, R), 1.0, "bf16")
    w = W.normal(rng, (H * 256, R), R ** -0.5, "bf16")
    ld, wd = _to(dev, lat, w)
    say(f"expand deep tile: B={B} Lk={Lk} R={R} H={H}")
    kn, v = mla.latent_expand(ld, wd, H)
    torch.cuda.synchronize()
    ref_kn, ref_v = oracle.latent_expand(lat, w, H, 128, 128)
    for got, ref in ((kn, ref_kn), (v, ref_v)):
        g = got.to("cpu", torch.float64).numpy()
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_expand_ragged(dev, dtype):
    rng = np.random.default_rng(22)
    B, Lk, R, H = 2, 77, 96, 3
    lat = W.normal(rng, (B, Lk, R), 1.0, dtype)
    w = W.normal(rng, (H * 256, R), 0.05, dtype)
    ld, wd = _to(dev, lat, w)
    kn, v = mla.latent_expand(ld, wd, H)
    torch.cuda.synchronize()
    ref_kn, ref_v = oracle.latent_expand(lat, w, H, 128, 128)
    for got, ref in ((kn, ref_kn), (v, ref_v)):
        g = got.to("cpu", torch.float64).numpy()
        if dtype == "f32":
            assert np.abs(g - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        else:
            assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
