// C ABI of the library (declared in include/dflash_mla.h): argument checks,
// workspace layout and kernel dispatch.  Nothing here allocates device memory;
// every launch goes on the caller's stream.  The only state is the static
// scratch array of dflash_mla_attn_no_alloc and its per-device addresses.
#include <cmath>
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/dflash_mla.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dflash_status fail(dflash_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dflash_status ok() {
  g_last_error.clear();
  return DFLASH_OK;
}

dflash_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DFLASH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t dt_size(dflash_dtype d) { return d == DFLASH_BF16 ? 2 : 4; }

bool valid_dtype(int d) { return d == DFLASH_F32 || d == DFLASH_BF16; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Multiply positive sizes, reporting overflow past 2^62.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a <= 0 || b <= 0) return false;
  if (a > (int64_t(1) << 62) / b) return false;
  *out = a * b;
  return true;
}

struct TileLayout {
  int64_t nqt, nkt;
  size_t classes, counts, lists, order, bits, sync, total;
};

bool tile_layout(int64_t B, int64_t Lq, int64_t Lk, TileLayout* t) {
  if (B <= 0 || Lq <= 0 || Lk <= 0) return false;
  t->nqt = (Lq + DFLASH_TILE_M - 1) / DFLASH_TILE_M;
  t->nkt = (Lk + DFLASH_TILE_N - 1) / DFLASH_TILE_N;
  int64_t rows, cells;
  if (!mul_ok(B, t->nqt, &rows) || !mul_ok(rows, t->nkt, &cells)) return false;
  t->classes = 0;
  t->counts = align_up(static_cast<size_t>(cells), 256);
  t->lists = t->counts + align_up(static_cast<size_t>(rows) * 4, 256);
  t->order = t->lists + align_up(static_cast<size_t>(cells) * 4, 256);
  t->bits = t->order + align_up(static_cast<size_t>(rows) * 4, 256);
  t->sync = align_up(t->bits + static_cast<size_t>(cells) * DFLASH_TILE_M * 8, 256);
  t->total = t->sync + 256;
  return true;
}

// Key-range splits of a bf16 forward.  Two workgroups run on each of the 256
// compute units, so up to 512 (batch, q-tile, head) items are all resident at
// once and the longest item sets the kernel time; with a block mask the items'
// tile counts differ widely (the last q-tile of a workload sees the whole
// context, the first only its start).  While the items fit in that one round,
// each item's tile list is cut into 2, 4 or 8 runs while a run of the whole key
// range keeps >= 4 k-tiles: the launch order (longest q-tiles first) then hands
// the short runs to the units that finished a long one.
int attn_splits(int64_t B, int64_t H, int64_t Lq, int64_t Lk) {
  const int64_t items = B * ((Lq + DFLASH_TILE_M - 1) / DFLASH_TILE_M) * H;
  const int64_t nkt = (Lk + DFLASH_TILE_N - 1) / DFLASH_TILE_N;
  int sp = 1;
  while (sp < 8 && items * sp <= 512 && nkt / (2 * sp) >= 4) sp *= 2;
  return sp;
}

// Workspace of a split forward: the tile map, then part_o [S,B,H,Lq,Dv] bf16 and
// part_lse [S,B,H,Lq] f32.  Returns false on overflow / invalid sizes.
struct SplitLayout {
  int nsplit;
  size_t part_o, part_lse, total;
};
bool split_layout(int64_t B, int64_t H, int64_t Lq, int64_t Lk, SplitLayout* L) {
  TileLayout t;
  if (H <= 0 || !tile_layout(B, Lq, Lk, &t)) return false;
  L->nsplit = attn_splits(B, H, Lq, Lk);
  int64_t rows, n;
  if (!mul_ok(B, H, &rows) || !mul_ok(rows, Lq, &rows) || !mul_ok(rows, L->nsplit, &n) ||
      !mul_ok(n, static_cast<int64_t>(dflash::kDv) * 2, &n))
    return false;
  if (L->nsplit == 1) {
    L->part_o = L->part_lse = L->total = t.total;
    return true;
  }
  L->part_o = align_up(t.total, 256);
  L->part_lse = align_up(L->part_o + static_cast<size_t>(n), 256);
  L->total = align_up(L->part_lse + static_cast<size_t>(rows) * L->nsplit * 4, 256);
  return true;
}


}  // namespace

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "DFLASH_OK";
    case DFLASH_ERR_INVALID_ARG: return "DFLASH_ERR_INVALID_ARG";
    case DFLASH_ERR_UNSUPPORTED: return "DFLASH_ERR_UNSUPPORTED";
    case DFLASH_ERR_WORKSPACE: return "DFLASH_ERR_WORKSPACE";
    case DFLASH_ERR_HIP: return "DFLASH_ERR_HIP";
  }
  return "DFLASH_ERR_UNKNOWN";
}

const char* dflash_last_error(void) { return g_last_error.c_str(); }

size_t dflash_mla_attn_workspace_bytes(int64_t B, int64_t Lq, int64_t Lk) {
  TileLayout t;
  if (!tile_layout(B, Lq, Lk, &t)) return 0;
  return t.total;
}

size_t dflash_mla_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk) {
  SplitLayout L;
  if (!split_layout(B, H, Lq, Lk, &L)) return 0;
  return L.total;
}

dflash_status dflash_mla_tile_map_layout(int64_t B, int64_t Lq, int64_t Lk, int64_t* n_q_tiles,
                                         int64_t* n_k_tiles, size_t* classes_offset,
                                         size_t* counts_offset, size_t* lists_offset,
                                         size_t* order_offset, size_t* bits_offset) {
  TileLayout t;
  if (!tile_layout(B, Lq, Lk, &t)) return fail(DFLASH_ERR_INVALID_ARG, "B, Lq, Lk must be positive (got %lld, %lld, %lld)", (long long)B, (long long)Lq, (long long)Lk);
  if (n_q_tiles) *n_q_tiles = t.nqt;
  if (n_k_tiles) *n_k_tiles = t.nkt;
  if (classes_offset) *classes_offset = t.classes;
  if (counts_offset) *counts_offset = t.counts;
  if (lists_offset) *lists_offset = t.lists;
  if (order_offset) *order_offset = t.order;
  if (bits_offset) *bits_offset = t.bits;
  return ok();
}

// need_mask = false: only the tile map in the workspace is used (a map computed
// earlier, e.g. from the block structure), no mask is read.
static dflash_status check_occupancy_args(const void* mask, int mask_dt, int64_t B, int64_t Lq,
                                          int64_t Lk, const void* ws, size_t ws_bytes,
                                          TileLayout* t, bool need_mask = true) {
  if (need_mask) {
    if (!mask) return fail(DFLASH_ERR_INVALID_ARG, "additive_mask is NULL");
    if (!valid_dtype(mask_dt)) return fail(DFLASH_ERR_INVALID_ARG, "mask_dt %d is not a dflash_dtype", mask_dt);
    if (!aligned16(mask)) return fail(DFLASH_ERR_INVALID_ARG, "additive_mask is not 16-byte aligned");
  }
  if (B <= 0 || Lq <= 0 || Lk <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "B, Lq, Lk must be positive (got %lld, %lld, %lld)", (long long)B, (long long)Lq, (long long)Lk);
  if (B > INT32_MAX || Lq > INT32_MAX || Lk > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "B, Lq, Lk must each fit in int32");
  if (!tile_layout(B, Lq, Lk, t)) return fail(DFLASH_ERR_INVALID_ARG, "tile map size overflows");
  if (t->nkt >= (int64_t(1) << 24)) return fail(DFLASH_ERR_UNSUPPORTED, "Lk too large for the tile lists");
  if (B * t->nqt * t->nkt > INT32_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "too many tiles");
  if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < t->total)
    return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, t->total);
  return ok();
}

static dflash::OccupancyArgs occupancy_args(const void* mask, int mask_dt, int64_t B, int64_t Lq,
                                            int64_t Lk, void* ws, const TileLayout& t) {
  dflash::OccupancyArgs o;
  char* w = static_cast<char*>(ws);
  o.mask = mask;
  o.mask_bf16 = mask_dt == DFLASH_BF16;
  o.B = static_cast<int>(B);
  o.Lq = static_cast<int>(Lq);
  o.Lk = static_cast<int>(Lk);
  o.nqt = static_cast<int>(t.nqt);
  o.nkt = static_cast<int>(t.nkt);
  o.classes = reinterpret_cast<uint8_t*>(w + t.classes);
  o.counts = reinterpret_cast<int32_t*>(w + t.counts);
  o.lists = reinterpret_cast<int32_t*>(w + t.lists);
  o.order = reinterpret_cast<int32_t*>(w + t.order);
  o.bits = reinterpret_cast<uint64_t*>(w + t.bits);
  o.sync = reinterpret_cast<uint32_t*>(w + t.sync);
  o.anchors = nullptr;
  o.ctx_valid = nullptr;
  o.A = o.bs = o.ctx = 0;
  return o;
}

// Validation shared by the block-structure entry points: Lq = A * block_size,
// Lk = ctx + Lq; returns the tile layout.
static dflash_status check_block_args(const int32_t* anchors, const int32_t* ctx_valid, int64_t B, int64_t A,
                                      int64_t block_size, int64_t ctx, const void* ws, size_t ws_bytes,
                                      TileLayout* t, int64_t* Lq, int64_t* Lk) {
  if (!anchors) return fail(DFLASH_ERR_INVALID_ARG, "anchors is NULL");
  if ((reinterpret_cast<uintptr_t>(anchors) & 3u) != 0 || (reinterpret_cast<uintptr_t>(ctx_valid) & 3u) != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "anchors / ctx_valid must be 4-byte aligned");
  if (B <= 0 || A <= 0 || block_size <= 0 || ctx < 0)
    return fail(DFLASH_ERR_INVALID_ARG, "B, A, block_size must be positive and ctx >= 0 (got %lld, %lld, %lld, %lld)",
                (long long)B, (long long)A, (long long)block_size, (long long)ctx);
  int64_t lq;
  if (!mul_ok(A, block_size, &lq) || lq > INT32_MAX || ctx > INT32_MAX - lq)
    return fail(DFLASH_ERR_UNSUPPORTED, "A * block_size + ctx must fit in int32");
  *Lq = lq;
  *Lk = ctx + lq;
  if (!tile_layout(B, *Lq, *Lk, t)) return fail(DFLASH_ERR_INVALID_ARG, "tile map size overflows");
  if (B > INT32_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "B must fit in int32");
  if (t->nkt >= (int64_t(1) << 24)) return fail(DFLASH_ERR_UNSUPPORTED, "Lk too large for the tile lists");
  if (B * t->nqt * t->nkt > INT32_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "too many tiles");
  if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < t->total)
    return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, t->total);
  const Range rw = range_of(ws, t->total);
  if (overlaps(rw, range_of(anchors, static_cast<size_t>(B) * A * 4)) ||
      (ctx_valid && overlaps(rw, range_of(ctx_valid, static_cast<size_t>(B) * 4))))
    return fail(DFLASH_ERR_INVALID_ARG, "the workspace overlaps anchors / ctx_valid");
  return ok();
}

static dflash::OccupancyArgs block_args(const int32_t* anchors, const int32_t* ctx_valid, int64_t B, int64_t A,
                                        int64_t block_size, int64_t ctx, int64_t Lq, int64_t Lk, void* ws,
                                        const TileLayout& t) {
  dflash::OccupancyArgs o = occupancy_args(nullptr, DFLASH_F32, B, Lq, Lk, ws, t);
  o.anchors = anchors;
  o.ctx_valid = ctx_valid;
  o.A = static_cast<int>(A);
  o.bs = static_cast<int>(block_size);
  o.ctx = static_cast<int>(ctx);
  return o;
}

dflash_status dflash_mla_mask_occupancy(const void* additive_mask, dflash_dtype mask_dt, int64_t B,
                                        int64_t Lq, int64_t Lk, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  TileLayout t;
  dflash_status st = check_occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, workspace_bytes, &t);
  if (st != DFLASH_OK) return st;
  const dflash::OccupancyArgs o = occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, t);
  return hip_status(dflash::launch_occupancy(o, static_cast<hipStream_t>(stream)), "mask occupancy launch");
}

}  // extern "C"

namespace {

// kv_b_proj as a linear layer: rows (b, token), outputs n = h * 256 + e scattered to
// k_nope (e < 128) and v (e >= 128) in [B, H, Lk, 128].
dflash::LinearArgs expand_linear(const void* latent, const void* w, void* kn, void* v, int64_t B, int64_t Lk,
                                 int64_t R, int64_t H) {
  dflash::LinearArgs l = {};
  l.a1 = static_cast<const uint16_t*>(latent);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(Lk);
  l.K = static_cast<int>(R);
  l.w = static_cast<const uint16_t*>(w);
  l.N = static_cast<int>(H * 256);
  l.mode = dflash::kLinearKV;
  l.y1 = static_cast<uint16_t*>(kn);
  l.y2 = static_cast<uint16_t*>(v);
  return l;
}

}  // namespace

extern "C" {

dflash_status dflash_mla_latent_expand(const void* latent, const void* w_kv_b, void* k_nope, void* v,
                                       int64_t B, int64_t Lk, int64_t R, int64_t H, int64_t Dn,
                                       int64_t Dv, dflash_dtype dt, void* stream) {
  if (!latent || !w_kv_b || !k_nope || !v) return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(latent) || !aligned16(w_kv_b) || !aligned16(k_nope) || !aligned16(v))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B <= 0 || Lk <= 0 || R <= 0 || H <= 0 || Dn <= 0 || Dv <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive");
  if (!valid_dtype(dt)) return fail(DFLASH_ERR_INVALID_ARG, "dt %d is not a dflash_dtype", (int)dt);
  if (Dn != dflash::kDn || Dv != dflash::kDv)
    return fail(DFLASH_ERR_UNSUPPORTED, "only Dn = 128 and Dv = 128 are built (got %lld, %lld)", (long long)Dn, (long long)Dv);
  if (R % 32 != 0) return fail(DFLASH_ERR_UNSUPPORTED, "R must be a multiple of 32 (got %lld)", (long long)R);
  int64_t M, tmp;
  if (!mul_ok(B, Lk, &M) || M > INT32_MAX || H > 16384 || R > INT32_MAX || !mul_ok(M, R, &tmp))
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t es = dt_size(dt);
  const Range rl = range_of(latent, static_cast<size_t>(M) * R * es);
  const Range rw = range_of(w_kv_b, static_cast<size_t>(H) * 256 * R * es);
  const Range rk = range_of(k_nope, static_cast<size_t>(M) * H * 128 * es);
  const Range rv = range_of(v, static_cast<size_t>(M) * H * 128 * es);
  if (overlaps(rk, rv) || overlaps(rk, rl) || overlaps(rk, rw) || overlaps(rv, rl) || overlaps(rv, rw))
    return fail(DFLASH_ERR_INVALID_ARG, "outputs overlap each other or an input");
  dflash::ExpandArgs a = {};
  a.latent = latent;
  a.w = w_kv_b;
  a.kn = k_nope;
  a.v = v;
  a.B = static_cast<int>(B);
  a.Lk = static_cast<int>(Lk);
  a.R = static_cast<int>(R);
  a.H = static_cast<int>(H);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == DFLASH_BF16) {
    const dflash::LinearArgs l = expand_linear(latent, w_kv_b, k_nope, v, B, Lk, R, H);
    return hip_status(dflash::launch_linear_bf16(l, s), "latent expand launch");
  }
  return hip_status(dflash::launch_expand_f32(a, s), "latent expand launch");
}

}  // extern "C"

namespace {

// The forward of dflash_mla_attn / dflash_mla_attn_lse (lse may be null).
dflash_status attn_impl(const void* q, const void* k_nope, const void* k_rope_shared, const void* v,
                        const void* additive_mask, void* out, float* lse, int64_t B, int64_t H, int64_t Lq,
                        int64_t Lk, int64_t Dn, int64_t Dr, int64_t Dv, float scale, dflash_dtype dt,
                        dflash_dtype mask_dt, void* workspace, size_t workspace_bytes, uint32_t flags,
                        void* stream) {
  if (!q || !k_nope || !k_rope_shared || !v || !out) return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_rope_shared) || !aligned16(v) || !aligned16(out) ||
      (additive_mask && !aligned16(additive_mask)))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || Dn <= 0 || Dr <= 0 || Dv <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive (B=%lld H=%lld Lq=%lld Lk=%lld)", (long long)B, (long long)H, (long long)Lq, (long long)Lk);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DFLASH_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!valid_dtype(dt) || !valid_dtype(mask_dt)) return fail(DFLASH_ERR_INVALID_ARG, "dtype is not a dflash_dtype");
  if (flags & ~(DFLASH_ATTN_REUSE_TILE_MAP | DFLASH_ATTN_NO_TILE_SKIP | DFLASH_ATTN_CHECK_ONLY |
                DFLASH_ATTN_SPLIT_KEYS))
    return fail(DFLASH_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (Dn != dflash::kDn || Dr != dflash::kDr || Dv != dflash::kDv)
    return fail(DFLASH_ERR_UNSUPPORTED, "only Dn=128, Dr=64, Dv=128 are built (got %lld, %lld, %lld)", (long long)Dn, (long long)Dr, (long long)Dv);
  if (additive_mask && dt == DFLASH_F32 && mask_dt != DFLASH_F32)
    return fail(DFLASH_ERR_UNSUPPORTED, "an f32 attention takes an f32 mask");
  if (B > INT32_MAX || H > INT32_MAX || Lq > INT32_MAX || Lk > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes must each fit in int32");
  int64_t bh, tmp;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, Lq, &tmp) || !mul_ok(tmp, Dn + Dr, &tmp) || !mul_ok(bh, Lk, &tmp) ||
      !mul_ok(tmp, Dn, &tmp) || !mul_ok(B * Lq, Lk, &tmp))
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t es = dt_size(dt);
  const Range ro = range_of(out, static_cast<size_t>(bh) * Lq * Dv * es);
  const Range ins[5] = {
      range_of(q, static_cast<size_t>(bh) * Lq * (Dn + Dr) * es),
      range_of(k_nope, static_cast<size_t>(bh) * Lk * Dn * es),
      range_of(k_rope_shared, static_cast<size_t>(B) * Lk * Dr * es),
      range_of(v, static_cast<size_t>(bh) * Lk * Dv * es),
      additive_mask ? range_of(additive_mask, static_cast<size_t>(B) * Lq * Lk * dt_size(mask_dt)) : Range{0, 0},
  };
  for (const Range& r : ins)
    if (overlaps(ro, r)) return fail(DFLASH_ERR_INVALID_ARG, "out overlaps an input");
  const Range rl = lse ? range_of(lse, static_cast<size_t>(bh) * Lq * 4) : Range{0, 0};
  if (lse) {
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(DFLASH_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (overlaps(rl, ro)) return fail(DFLASH_ERR_INVALID_ARG, "lse overlaps out");
    for (const Range& r : ins)
      if (overlaps(rl, r)) return fail(DFLASH_ERR_INVALID_ARG, "lse overlaps an input");
  }
  if (dt == DFLASH_BF16 && (Lk + DFLASH_TILE_N - 1) / DFLASH_TILE_N > dflash::kMaxKeyTiles)
    return fail(DFLASH_ERR_UNSUPPORTED, "a bf16 call supports at most %d key tiles, got Lk = %lld",
                dflash::kMaxKeyTiles, (long long)Lk);
  // the bf16 kernel copies K / V tiles through buffer resources whose range and
  // offsets are 32-bit: one (batch, head) slice of k_nope or v must fit in 2^31 bytes
  if (dt == DFLASH_BF16 && Lk * (Dn * 2) > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "a bf16 call takes at most %lld keys (one (batch, head) k_nope / v slice "
                "within 2^31 bytes), got Lk = %lld", (long long)(INT32_MAX / (Dn * 2)), (long long)Lk);
  const bool map_only = !additive_mask && (flags & DFLASH_ATTN_REUSE_TILE_MAP);   // the workspace's map alone
  if (map_only && dt == DFLASH_F32) return fail(DFLASH_ERR_INVALID_ARG, "the f32 path keeps no tile map to reuse");
  if (map_only && (flags & DFLASH_ATTN_NO_TILE_SKIP))
    return fail(DFLASH_ERR_INVALID_ARG, "NO_TILE_SKIP needs the mask (a reused map alone has no values for empty tiles)");
  SplitLayout sl = {1, 0, 0, 0};
  if (dt == DFLASH_BF16 && (flags & DFLASH_ATTN_SPLIT_KEYS) && !(flags & DFLASH_ATTN_NO_TILE_SKIP)) {
    if (!split_layout(B, H, Lq, Lk, &sl)) return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
    if (sl.nsplit > 1) {
      if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "SPLIT_KEYS needs a workspace");
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(DFLASH_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
      if (workspace_bytes < sl.total)
        return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, a split call of this shape needs %zu",
                    workspace_bytes, sl.total);
      const Range rw = range_of(workspace, sl.total);
      if (overlaps(ro, rw) || overlaps(rl, rw)) return fail(DFLASH_ERR_INVALID_ARG, "out / lse overlap the workspace");
      for (const Range& r : ins)
        if (overlaps(rw, r)) return fail(DFLASH_ERR_INVALID_ARG, "the workspace overlaps an input");
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (dt == DFLASH_F32) {
    if (flags & DFLASH_ATTN_CHECK_ONLY) return ok();
    if (static_cast<int64_t>(B) > 65535 || H > 65535) return fail(DFLASH_ERR_UNSUPPORTED, "B and H must be <= 65535 for f32");
    dflash::AttnF32Args a;
    a.q = static_cast<const float*>(q);
    a.kn = static_cast<const float*>(k_nope);
    a.kr = static_cast<const float*>(k_rope_shared);
    a.v = static_cast<const float*>(v);
    a.mask = static_cast<const float*>(additive_mask);
    a.out = static_cast<float*>(out);
    a.B = static_cast<int>(B);
    a.H = static_cast<int>(H);
    a.Lq = static_cast<int>(Lq);
    a.Lk = static_cast<int>(Lk);
    a.scale = scale;
    a.lse = lse;
    return hip_status(dflash::launch_attn_f32(a, s), "f32 attention launch");
  }

  dflash::AttnBf16Args a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kn = static_cast<const uint16_t*>(k_nope);
  a.kr = static_cast<const uint16_t*>(k_rope_shared);
  a.v = static_cast<const uint16_t*>(v);
  a.mask = additive_mask;
  a.out = static_cast<uint16_t*>(out);
  a.B = static_cast<int>(B);
  a.H = static_cast<int>(H);
  a.Lq = static_cast<int>(Lq);
  a.Lk = static_cast<int>(Lk);
  a.nqt = static_cast<int>((Lq + DFLASH_TILE_M - 1) / DFLASH_TILE_M);
  a.nkt = static_cast<int>((Lk + DFLASH_TILE_N - 1) / DFLASH_TILE_N);
  a.scale = scale;
  a.mask_bf16 = mask_dt == DFLASH_BF16;
  a.lse = lse;
  if (static_cast<int64_t>(B) * a.nqt * H > INT32_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "too many work items");
  if (a.nkt > dflash::kMaxKeyTiles)
    return fail(DFLASH_ERR_UNSUPPORTED, "a bf16 call supports at most %d key tiles, got Lk = %lld",
                dflash::kMaxKeyTiles, (long long)Lk);
  if (additive_mask || map_only) {
    TileLayout t;
    dflash_status st = check_occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, workspace_bytes, &t,
                                            !map_only);
    if (st != DFLASH_OK) return st;
    const Range rw = range_of(workspace, t.total);
    if (overlaps(ro, rw) || overlaps(rl, rw)) return fail(DFLASH_ERR_INVALID_ARG, "out / lse overlap the workspace");
    for (const Range& r : ins)
      if (overlaps(rw, r)) return fail(DFLASH_ERR_INVALID_ARG, "the workspace overlaps an input");
    if (flags & DFLASH_ATTN_CHECK_ONLY) return ok();
    const dflash::OccupancyArgs o = occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, t);
    if (!(flags & DFLASH_ATTN_REUSE_TILE_MAP)) {
      st = hip_status(dflash::launch_occupancy(o, s), "mask occupancy launch");
      if (st != DFLASH_OK) return st;
    }
    if (flags & DFLASH_ATTN_NO_TILE_SKIP) {
      st = hip_status(dflash::launch_lists_all_tiles(o, s), "tile list rewrite launch");
      if (st != DFLASH_OK) return st;
    }
    a.classes = o.classes;
    a.counts = o.counts;
    a.lists = o.lists;
    a.order = o.order;
    a.bits = o.bits;
  }
  if (flags & DFLASH_ATTN_CHECK_ONLY) return ok();
  a.nsplit = sl.nsplit;
  if (sl.nsplit > 1) {
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<uint16_t*>(ws + sl.part_o);
    a.part_lse = reinterpret_cast<float*>(ws + sl.part_lse);
    a.lse = nullptr;
  }
  dflash_status st = hip_status(dflash::launch_attn_bf16(a, s), "bf16 attention launch");
  if (st != DFLASH_OK || sl.nsplit == 1) return st;
  dflash::AttnCombineArgs c;
  c.part_o = a.part_o;
  c.part_lse = a.part_lse;
  c.out = a.out;
  c.lse = lse;
  c.rows = B * H * Lq;
  c.nsplit = sl.nsplit;
  return hip_status(dflash::launch_attn_combine(c, s), "split combine launch");
}

// Backward workspace: the forward's tile map, then the backward's own arrays.
struct BwdLayout {
  TileLayout t;
  int64_t Lqp, Lkp;
  size_t qT, doT, knT, krT, rope, ld, bitsT, total;
};

bool bwd_layout(int64_t B, int64_t H, int64_t Lq, int64_t Lk, BwdLayout* L) {
  if (H <= 0 || !tile_layout(B, Lq, Lk, &L->t)) return false;
  L->Lqp = L->t.nqt * DFLASH_TILE_M;
  L->Lkp = L->t.nkt * DFLASH_TILE_N;
  int64_t bh, a, c, d, e, f, g, bt;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, L->Lqp, &a) || !mul_ok(a, 4, &c) || !mul_ok(a, 2 * 192, &d) ||
      !mul_ok(bh, L->Lkp, &e) || !mul_ok(e, 2 * 128, &e) || !mul_ok(B, L->Lkp * 2 * 64, &f) ||
      !mul_ok(bh, Lk, &g) || !mul_ok(g, 64 * 4, &g) || !mul_ok(B * L->t.nqt, L->t.nkt, &bt) || !mul_ok(bt, 1024, &bt))
    return false;
  L->qT = align_up(L->t.total, 256);
  L->doT = L->qT + align_up(static_cast<size_t>(d), 256);
  L->knT = L->doT + align_up(static_cast<size_t>(a) * 2 * 128, 256);
  L->krT = L->knT + align_up(static_cast<size_t>(e), 256);
  L->rope = L->krT + align_up(static_cast<size_t>(f), 256);
  L->ld = L->rope + align_up(static_cast<size_t>(g), 256);
  L->bitsT = L->ld + align_up(static_cast<size_t>(c) * 2, 256);
  L->total = L->bitsT + align_up(static_cast<size_t>(bt), 256);
  return true;
}

}  // namespace

extern "C" {

dflash_status dflash_mla_attn(const void* q, const void* k_nope, const void* k_rope_shared,
                              const void* v, const void* additive_mask, void* out, int64_t B,
                              int64_t H, int64_t Lq, int64_t Lk, int64_t Dn, int64_t Dr,
                              int64_t Dv, float scale, dflash_dtype dt, dflash_dtype mask_dt,
                              void* workspace, size_t workspace_bytes, uint32_t flags,
                              void* stream) {
  return attn_impl(q, k_nope, k_rope_shared, v, additive_mask, out, nullptr, B, H, Lq, Lk, Dn, Dr, Dv, scale, dt,
                   mask_dt, workspace, workspace_bytes, flags, stream);
}

dflash_status dflash_mla_attn_lse(const void* q, const void* k_nope, const void* k_rope_shared,
                                  const void* v, const void* additive_mask, void* out, float* lse,
                                  int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t Dn, int64_t Dr,
                                  int64_t Dv, float scale, dflash_dtype dt, dflash_dtype mask_dt,
                                  void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  if (!lse) return fail(DFLASH_ERR_INVALID_ARG, "lse is NULL");
  return attn_impl(q, k_nope, k_rope_shared, v, additive_mask, out, lse, B, H, Lq, Lk, Dn, Dr, Dv, scale, dt,
                   mask_dt, workspace, workspace_bytes, flags, stream);
}

}  // extern "C"

// Scratch of dflash_mla_attn_no_alloc: the tile map of a masked bf16 call lives
// here instead of in a caller's workspace.  Every GPU the library runs on holds
// its own copy until the process ends; calls on one GPU share it.  In host code
// `scratch` is only a stand-in for the device array: its address on each device
// comes from hipGetSymbolAddress (once per device, with that device current), and
// only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DFLASH_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices] = {};

// the current device's address of `scratch`
dflash_status scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(DFLASH_ERR_UNSUPPORTED, "device %d: the no-alloc scratch serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the no-alloc scratch");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(DFLASH_ERR_HIP, "the no-alloc scratch has no 256-byte aligned device address");
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" {

dflash_status dflash_mla_attn_no_alloc(const void* q, const void* k_nope, const void* k_rope_shared,
                                       const void* v, const void* additive_mask, void* out, int64_t B,
                                       int64_t H, int64_t Lq, int64_t Lk, int64_t Dn, int64_t Dr,
                                       int64_t Dv, float scale, dflash_dtype dt, dflash_dtype mask_dt,
                                       uint32_t flags, void* stream) {
  if (flags & ~(DFLASH_ATTN_NO_TILE_SKIP | DFLASH_ATTN_CHECK_ONLY))
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_mla_attn_no_alloc takes only NO_TILE_SKIP and CHECK_ONLY "
                "(got flags 0x%x): its scratch holds no map to reuse and no room for split partials", flags);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (dt == DFLASH_BF16 && additive_mask) {
    const size_t need = dflash_mla_attn_workspace_bytes(B, Lq, Lk);
    if (need == 0)
      return fail(DFLASH_ERR_INVALID_ARG, "B, Lq, Lk must be positive (got %lld, %lld, %lld)", (long long)B,
                  (long long)Lq, (long long)Lk);
    if (need > DFLASH_NO_ALLOC_SCRATCH_BYTES)
      return fail(DFLASH_ERR_UNSUPPORTED, "the tile map of B=%lld, Lq=%lld, Lk=%lld needs %zu bytes; the no-alloc "
                  "scratch holds %zu (use dflash_mla_attn with a workspace)", (long long)B, (long long)Lq,
                  (long long)Lk, need, static_cast<size_t>(DFLASH_NO_ALLOC_SCRATCH_BYTES));
    ws_bytes = DFLASH_NO_ALLOC_SCRATCH_BYTES;
    if (flags & DFLASH_ATTN_CHECK_ONLY) {
      // validation only, nothing launched: a stand-in address above every allocation
      ws = reinterpret_cast<void*>(uintptr_t(1) << 62);
    } else {
      const dflash_status st = scratch_address(&ws);
      if (st != DFLASH_OK) return st;
    }
  }
  return attn_impl(q, k_nope, k_rope_shared, v, additive_mask, out, nullptr, B, H, Lq, Lk, Dn, Dr, Dv, scale, dt,
                   mask_dt, ws, ws_bytes, flags, stream);
}

size_t dflash_mla_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk) {
  BwdLayout L;
  return bwd_layout(B, H, Lq, Lk, &L) ? L.total : 0;
}

dflash_status dflash_mla_attn_bwd(const void* q, const void* k_nope, const void* k_rope_shared, const void* v,
                                  const void* additive_mask, const void* out, const void* dout, const float* lse,
                                  void* dq, void* dk_nope, void* dk_rope_shared, void* dv, int64_t B, int64_t H,
                                  int64_t Lq, int64_t Lk, int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                                  dflash_dtype dt, dflash_dtype mask_dt, void* workspace, size_t workspace_bytes,
                                  uint32_t flags, void* stream) {
  if (!q || !k_nope || !k_rope_shared || !v || !out || !dout || !lse || !dq || !dk_nope || !dk_rope_shared || !dv)
    return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_rope_shared) || !aligned16(v) || !aligned16(out) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk_nope) || !aligned16(dk_rope_shared) || !aligned16(dv) ||
      (additive_mask && !aligned16(additive_mask)) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned (lse: 4-byte)");
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || Dn <= 0 || Dr <= 0 || Dv <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive (B=%lld H=%lld Lq=%lld Lk=%lld)", (long long)B,
                (long long)H, (long long)Lq, (long long)Lk);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DFLASH_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!valid_dtype(dt) || !valid_dtype(mask_dt)) return fail(DFLASH_ERR_INVALID_ARG, "dtype is not a dflash_dtype");
  if (flags & ~DFLASH_ATTN_REUSE_TILE_MAP) return fail(DFLASH_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (Dn != dflash::kDn || Dr != dflash::kDr || Dv != dflash::kDv)
    return fail(DFLASH_ERR_UNSUPPORTED, "only Dn=128, Dr=64, Dv=128 are built (got %lld, %lld, %lld)", (long long)Dn,
                (long long)Dr, (long long)Dv);
  if (dt != DFLASH_BF16) return fail(DFLASH_ERR_UNSUPPORTED, "the backward is built for bf16 tensors only");
  if (Lq > INT32_MAX || Lk > INT32_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "Lq and Lk must each fit in int32");
  int64_t bh;
  if (!mul_ok(B, H, &bh) || bh > 65535) return fail(DFLASH_ERR_UNSUPPORTED, "B * H must be at most 65535");
  BwdLayout L;
  if (!bwd_layout(B, H, Lq, Lk, &L)) return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  if (L.t.nkt > dflash::kMaxKeyTiles || bh * L.t.nqt > INT32_MAX || L.Lqp > INT32_MAX || L.Lkp > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large for the backward launches");
  // the staging loads address one (b, h) slice of each operand through a 32-bit range
  if (L.Lkp * 2 * 192 > INT32_MAX || L.Lqp * 2 * 192 > INT32_MAX || B * L.t.nqt * L.t.nkt * 1024 > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "the backward takes at most 2^31 bytes per (batch, head) operand slice "
                "and per tile-map visibility array");
  if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  const size_t nq = static_cast<size_t>(bh) * Lq, nk = static_cast<size_t>(bh) * Lk;
  const Range ins[8] = {
      range_of(q, nq * 192 * 2), range_of(k_nope, nk * 128 * 2), range_of(k_rope_shared, static_cast<size_t>(B) * Lk * 64 * 2),
      range_of(v, nk * 128 * 2), range_of(out, nq * 128 * 2), range_of(dout, nq * 128 * 2), range_of(lse, nq * 4),
      additive_mask ? range_of(additive_mask, static_cast<size_t>(B) * Lq * Lk * dt_size(mask_dt)) : Range{0, 0}};
  const Range outs[5] = {range_of(dq, nq * 192 * 2), range_of(dk_nope, nk * 128 * 2),
                         range_of(dk_rope_shared, static_cast<size_t>(B) * Lk * 64 * 2), range_of(dv, nk * 128 * 2),
                         range_of(workspace, L.total)};
  for (int i = 0; i < 5; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return fail(DFLASH_ERR_INVALID_ARG, "an output or the workspace overlaps an input");
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], outs[j])) return fail(DFLASH_ERR_INVALID_ARG, "outputs / workspace overlap each other");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  dflash::AttnBwdArgs a = {};
  const bool map_only = !additive_mask && (flags & DFLASH_ATTN_REUSE_TILE_MAP);   // the workspace's map alone
  if (additive_mask || map_only) {
    dflash_status st = check_occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, workspace_bytes, &L.t,
                                            !map_only);
    if (st != DFLASH_OK) return st;
    const dflash::OccupancyArgs o = occupancy_args(additive_mask, mask_dt, B, Lq, Lk, workspace, L.t);
    if (!(flags & DFLASH_ATTN_REUSE_TILE_MAP)) {
      st = hip_status(dflash::launch_occupancy(o, s), "mask occupancy launch");
      if (st != DFLASH_OK) return st;
    }
    a.classes = o.classes;
    a.counts = o.counts;
    a.lists = o.lists;
    a.order = o.order;
    a.bits = o.bits;
  }
  a.q = static_cast<const uint16_t*>(q);
  a.kn = static_cast<const uint16_t*>(k_nope);
  a.kr = static_cast<const uint16_t*>(k_rope_shared);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.mask = additive_mask;
  a.mask_bf16 = mask_dt == DFLASH_BF16;
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dkn = static_cast<uint16_t*>(dk_nope);
  a.dkr = static_cast<uint16_t*>(dk_rope_shared);
  a.dv = static_cast<uint16_t*>(dv);
  a.qT = reinterpret_cast<uint16_t*>(ws + L.qT);
  a.doT = reinterpret_cast<uint16_t*>(ws + L.doT);
  a.knT = reinterpret_cast<uint16_t*>(ws + L.knT);
  a.krT = reinterpret_cast<uint16_t*>(ws + L.krT);
  a.rope_part = reinterpret_cast<float*>(ws + L.rope);
  a.ld = reinterpret_cast<float*>(ws + L.ld);
  a.bitsT = reinterpret_cast<uint32_t*>(ws + L.bitsT);
  a.B = static_cast<int>(B);
  a.H = static_cast<int>(H);
  a.Lq = static_cast<int>(Lq);
  a.Lk = static_cast<int>(Lk);
  a.nqt = static_cast<int>(L.t.nqt);
  a.nkt = static_cast<int>(L.t.nkt);
  a.Lqp = static_cast<int>(L.Lqp);
  a.Lkp = static_cast<int>(L.Lkp);
  a.scale = scale;
  return hip_status(dflash::launch_attn_bwd_bf16(a, s), "attention backward launch");
}

// ---------------------------------------------------------------- projections

// intermediate [rows, width] bf16, its row statistics, and split-K scratch for the
// product that makes the intermediate (capped at 64 MiB: larger products fill
// the chip without splitting)
static size_t proj_split_bytes(int64_t rows, int64_t width) {
  const size_t full = static_cast<size_t>(dflash::kLinearMaxSplits) * rows * width * 4;
  return std::min<size_t>(full, size_t(64) << 20);
}

size_t dflash_mla_projection_workspace_bytes(int64_t rows, int64_t width) {
  int64_t e, st;
  if (rows <= 0 || width <= 0 || !mul_ok(rows, width, &e) || !mul_ok(rows, (width + 127) / 128, &st) ||
      !mul_ok(e, 64, &st))
    return 0;
  return align_up(static_cast<size_t>(e) * 2, 256) + align_up(static_cast<size_t>(rows) * ((width + 127) / 128) * 4, 256) +
         align_up(proj_split_bytes(rows, width), 256);
}

}  // extern "C"

namespace {

dflash_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(DFLASH_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return ok();
}

bool any_overlap(const Range* r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlaps(r[i], r[j])) return true;
  return false;
}

dflash::LinearArgs linear_args() {
  dflash::LinearArgs l = {};
  l.mode = dflash::kLinearPlain;
  return l;
}

}  // namespace

extern "C" {

dflash_status dflash_mla_context_project(const void* target_hidden, const void* w_fc, const void* gamma, float eps,
                                         void* out, int64_t B, int64_t ctx, int64_t K_in, int64_t hidden,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_hidden || !w_fc || !gamma || !out) return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(target_hidden) || !aligned16(w_fc) || !aligned16(gamma) || !aligned16(out))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B <= 0 || ctx <= 0 || K_in <= 0 || hidden <= 0) return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DFLASH_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (K_in % 32 != 0 || hidden % 128 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "K_in must be a multiple of 32 and hidden of 128");
  int64_t M, tmp;
  if (!mul_ok(B, ctx, &M) || M > INT32_MAX || K_in > INT32_MAX || hidden > INT32_MAX || !mul_ok(M, K_in, &tmp) ||
      !mul_ok(hidden, K_in, &tmp) || (M + 127) / 128 > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t need = dflash_mla_projection_workspace_bytes(M, hidden);
  dflash_status st = check_ws(workspace, workspace_bytes, need);
  if (st != DFLASH_OK) return st;
  const Range r[4] = {range_of(out, static_cast<size_t>(M) * hidden * 2), range_of(target_hidden, static_cast<size_t>(M) * K_in * 2),
                      range_of(w_fc, static_cast<size_t>(hidden) * K_in * 2), range_of(workspace, need)};
  const Range g = range_of(gamma, static_cast<size_t>(hidden) * 2);
  if (any_overlap(r, 4) || overlaps(r[0], g) || overlaps(r[3], g))
    return fail(DFLASH_ERR_INVALID_ARG, "out / workspace overlap an input or each other");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* stats = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(M) * hidden * 2, 256));
  dflash::LinearArgs l = linear_args();
  l.a1 = static_cast<const uint16_t*>(target_hidden);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(ctx);
  l.K = static_cast<int>(K_in);
  l.w = static_cast<const uint16_t*>(w_fc);
  l.N = static_cast<int>(hidden);
  l.y1 = static_cast<uint16_t*>(out);
  l.stats_out = stats;
  l.Nstat = static_cast<int>(hidden);
  st = hip_status(dflash::launch_linear_bf16(l, s), "fc launch");
  if (st != DFLASH_OK) return st;
  dflash::RmsApplyArgs n = {};
  n.x = static_cast<const uint16_t*>(out);
  n.y = static_cast<uint16_t*>(out);
  n.M = M;
  n.N = static_cast<int>(hidden);
  n.stats = stats;
  n.parts = static_cast<int>(hidden / 128);
  n.gamma = static_cast<const uint16_t*>(gamma);
  n.eps = eps;
  return hip_status(dflash::launch_rms_apply_bf16(n, s), "hidden_norm launch");
}

dflash_status dflash_mla_q_project(const void* x, const void* w_q_a, const void* gamma_q, float eps, const void* w_q_b,
                                   void* q, int64_t B, int64_t Lq, int64_t hidden, int64_t q_lora_rank, int64_t H,
                                   int64_t Dqk, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_q_a || !gamma_q || !w_q_b || !q) return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(x) || !aligned16(w_q_a) || !aligned16(gamma_q) || !aligned16(w_q_b) || !aligned16(q))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B <= 0 || Lq <= 0 || hidden <= 0 || q_lora_rank <= 0 || H <= 0 || Dqk <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DFLASH_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (hidden % 32 != 0 || q_lora_rank % 128 != 0 || Dqk % 4 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a multiple of 32, q_lora_rank of 128, Dqk of 4");
  int64_t M, N, tmp;
  if (!mul_ok(B, Lq, &M) || M > INT32_MAX || !mul_ok(H, Dqk, &N) || N > INT32_MAX || hidden > INT32_MAX ||
      q_lora_rank > INT32_MAX || !mul_ok(M, hidden, &tmp) || !mul_ok(N, q_lora_rank, &tmp) || !mul_ok(M, N, &tmp) ||
      !mul_ok(q_lora_rank, hidden, &tmp))
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t need = dflash_mla_projection_workspace_bytes(M, q_lora_rank);
  dflash_status st = check_ws(workspace, workspace_bytes, need);
  if (st != DFLASH_OK) return st;
  const Range r[6] = {range_of(q, static_cast<size_t>(M) * N * 2), range_of(workspace, need),
                      range_of(x, static_cast<size_t>(M) * hidden * 2), range_of(w_q_a, static_cast<size_t>(q_lora_rank) * hidden * 2),
                      range_of(w_q_b, static_cast<size_t>(N) * q_lora_rank * 2), range_of(gamma_q, static_cast<size_t>(q_lora_rank) * 2)};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && overlaps(r[i], r[j])) return fail(DFLASH_ERR_INVALID_ARG, "q / workspace overlap another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* qa = static_cast<uint16_t*>(workspace);
  float* stats = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(M) * q_lora_rank * 2, 256));
  dflash::LinearArgs l = linear_args();
  l.a1 = static_cast<const uint16_t*>(x);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(Lq);
  l.K = static_cast<int>(hidden);
  l.w = static_cast<const uint16_t*>(w_q_a);
  l.N = static_cast<int>(q_lora_rank);
  l.y1 = qa;
  l.stats_out = stats;
  l.Nstat = static_cast<int>(q_lora_rank);
  float* split = reinterpret_cast<float*>(reinterpret_cast<char*>(stats) +
                                          align_up(static_cast<size_t>(M) * (q_lora_rank / 128) * 4, 256));
  st = hip_status(dflash::launch_linear_bf16(l, s, split, proj_split_bytes(M, q_lora_rank)), "q_a_proj launch");
  if (st != DFLASH_OK) return st;
  dflash::LinearArgs l2 = linear_args();
  l2.a1 = qa;
  l2.B = static_cast<int>(B);
  l2.T1 = static_cast<int>(Lq);
  l2.K = static_cast<int>(q_lora_rank);
  l2.w = static_cast<const uint16_t*>(w_q_b);
  l2.N = static_cast<int>(N);
  l2.stats_in = stats;
  l2.stats_parts = static_cast<int>(q_lora_rank / 128);
  l2.gamma = static_cast<const uint16_t*>(gamma_q);
  l2.eps = eps;
  l2.mode = dflash::kLinearHeads;
  l2.y1 = static_cast<uint16_t*>(q);
  l2.D = static_cast<int>(Dqk);
  return hip_status(dflash::launch_linear_bf16(l2, s), "q_b_proj launch");
}

dflash_status dflash_mla_kv_project(const void* ctx_hidden, const void* noise_hidden, const void* w_kv_a,
                                    const void* gamma_kv, float eps, const void* w_kv_b, void* k_nope,
                                    void* k_rope_shared, void* v, int64_t B, int64_t ctx, int64_t Lq, int64_t hidden,
                                    int64_t R, int64_t Dr, int64_t H, int64_t Dn, int64_t Dv, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if ((ctx > 0 && !ctx_hidden) || !noise_hidden || !w_kv_a || !gamma_kv || !w_kv_b || !k_nope || !k_rope_shared || !v)
    return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if ((ctx > 0 && !aligned16(ctx_hidden)) || !aligned16(noise_hidden) || !aligned16(w_kv_a) || !aligned16(gamma_kv) ||
      !aligned16(w_kv_b) || !aligned16(k_nope) || !aligned16(k_rope_shared) || !aligned16(v))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B <= 0 || ctx < 0 || Lq <= 0 || hidden <= 0 || R <= 0 || Dr <= 0 || H <= 0 || Dn <= 0 || Dv <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive (ctx >= 0)");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DFLASH_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (Dn != dflash::kDn || Dv != dflash::kDv) return fail(DFLASH_ERR_UNSUPPORTED, "only Dn = Dv = 128 are built");
  if (hidden % 32 != 0 || R % 128 != 0 || Dr % 4 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a multiple of 32, R of 128, Dr of 4");
  int64_t M, tmp;
  const int64_t Lk = ctx + Lq;
  if (!mul_ok(B, Lk, &M) || M > INT32_MAX || hidden > INT32_MAX || R + Dr > INT32_MAX || H > 16384 ||
      !mul_ok(M, hidden, &tmp) || !mul_ok(M, R + Dr, &tmp) || !mul_ok(M * H, 256, &tmp) || !mul_ok(R + Dr, hidden, &tmp))
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t need = dflash_mla_projection_workspace_bytes(M, R);
  dflash_status st = check_ws(workspace, workspace_bytes, need);
  if (st != DFLASH_OK) return st;
  const Range r[10] = {range_of(k_nope, static_cast<size_t>(M) * H * Dn * 2), range_of(v, static_cast<size_t>(M) * H * Dv * 2),
                       range_of(k_rope_shared, static_cast<size_t>(M) * Dr * 2), range_of(workspace, need),
                       ctx > 0 ? range_of(ctx_hidden, static_cast<size_t>(B) * ctx * hidden * 2) : Range{0, 0},
                       range_of(noise_hidden, static_cast<size_t>(B) * Lq * hidden * 2),
                       range_of(w_kv_a, static_cast<size_t>(R + Dr) * hidden * 2), range_of(gamma_kv, static_cast<size_t>(R) * 2),
                       range_of(w_kv_b, static_cast<size_t>(H) * (Dn + Dv) * R * 2), Range{0, 0}};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 10; ++j)
      if (i != j && overlaps(r[i], r[j])) return fail(DFLASH_ERR_INVALID_ARG, "an output or the workspace overlaps another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* latent = static_cast<uint16_t*>(workspace);
  float* stats = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(M) * R * 2, 256));
  dflash::LinearArgs l = linear_args();
  l.a1 = static_cast<const uint16_t*>(ctx_hidden);
  l.a2 = static_cast<const uint16_t*>(noise_hidden);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(ctx);
  l.T2 = static_cast<int>(Lq);
  l.K = static_cast<int>(hidden);
  l.w = static_cast<const uint16_t*>(w_kv_a);
  l.N = static_cast<int>(R + Dr);
  l.mode = dflash::kLinearSplit;
  l.y1 = latent;
  l.y2 = static_cast<uint16_t*>(k_rope_shared);
  l.N1 = static_cast<int>(R);
  l.stats_out = stats;
  l.Nstat = static_cast<int>(R);
  st = hip_status(dflash::launch_linear_bf16(l, s), "kv_a_proj_with_mqa launch");
  if (st != DFLASH_OK) return st;
  dflash::LinearArgs e = expand_linear(latent, w_kv_b, k_nope, v, B, Lk, R, H);
  e.stats_in = stats;
  e.stats_parts = static_cast<int>(R / 128);
  e.gamma = static_cast<const uint16_t*>(gamma_kv);
  e.eps = eps;
  return hip_status(dflash::launch_linear_bf16(e, s), "kv_b_proj launch");
}

// ---------------------------------------------------------------- GQA draft (MAX variant)

}  // extern "C"

namespace {

struct GqaSplit {
  int splits, tiles_per_split;
};

// Key splits of the GQA block attention: about one workgroup per compute unit in
// total (256), so every split starts at once and none waits for a second round.
// Measured on 8 rows x 8 KV heads with 8K-32K contexts: 4 splits (256 workgroups)
// beat 6, 8, 16 and 32, and beat splitting each row in proportion to its length
// from the device-side context lengths (the rounding up of every row's share
// pushed some workgroups into a second round).
GqaSplit gqa_split(int64_t B, int64_t Hkv, int64_t Lmax) {
  const int64_t ntiles = (Lmax + 63) / 64;
  int64_t want = (256 + B * Hkv - 1) / (B * Hkv);
  want = std::max<int64_t>(1, std::min(want, ntiles));
  const int64_t tps = (ntiles + want - 1) / want;
  return {static_cast<int>((ntiles + tps - 1) / tps), static_cast<int>(tps)};
}

bool gqa_layout(int64_t B, int64_t bs, int64_t Hq, int64_t Hkv, int64_t Lmax, size_t* q_off, size_t* o_off,
                size_t* ml_off, size_t* total) {
  if (B <= 0 || bs <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || B > 65535 || Hq > 4096 || Lmax > INT32_MAX) return false;
  const GqaSplit sp = gqa_split(B, Hkv, Lmax);
  const size_t rows = static_cast<size_t>(B) * Hkv * sp.splits * 64;
  *q_off = 0;
  *o_off = align_up(static_cast<size_t>(B) * Hq * bs * 128 * 2, 256);
  *ml_off = *o_off + align_up(rows * 128 * 4, 256);
  // split-K scratch for the block's projections (the widest is q: B*bs rows x Hq*128)
  *total = *ml_off + align_up(rows * 2 * 4, 256) +
           align_up(static_cast<size_t>(dflash::kLinearMaxSplits) * B * bs * Hq * 128 * 4, 256);
  return true;
}

double yarn_mscale(double scale, double m) { return scale <= 1.0 ? 1.0 : 0.1 * m * std::log(scale) + 1.0; }

// yarn RoPE as DeepSeek-V3 defines it (fp64): per rotary pair i of the 128-wide
// head, the extrapolated frequency theta^(-2i/d) and the interpolated one (divided
// by factor) blended by a linear ramp between the correction dimensions of
// beta_fast and beta_slow rotations at the original context length; cos / sin
// are scaled by mscale(factor, mscale) / mscale(factor, mscale_all_dim).
// rope = {theta, factor, original length, beta_fast, beta_slow, mscale, mscale_all_dim}.
dflash::NormRopeArgs norm_rope_args(const float* rope, const void* gamma, float eps) {
  dflash::NormRopeArgs n = {};
  n.gamma = static_cast<const uint16_t*>(gamma);
  n.eps = eps;
  const double theta = rope[0], factor = rope[1], omp = rope[2], beta_fast = rope[3], beta_slow = rope[4];
  const double d = 128.0, two_pi = 6.283185307179586, lb = 2.0 * std::log(theta);
  double low = std::floor(d * std::log(omp / (beta_fast * two_pi)) / lb);
  double high = std::ceil(d * std::log(omp / (beta_slow * two_pi)) / lb);
  low = std::fmax(low, 0.0);
  high = std::fmin(high, d - 1.0);
  if (low == high) high += 0.001;
  for (int i = 0; i < 64; ++i) {
    const double extra = 1.0 / std::pow(theta, 2.0 * i / d);
    const double inter = extra / factor;
    const double ramp = std::fmin(std::fmax((i - low) / (high - low), 0.0), 1.0);
    n.inv_freq[i] = inter * ramp + extra * (1.0 - ramp);
  }
  n.mscale = static_cast<float>(yarn_mscale(factor, rope[5]) / yarn_mscale(factor, rope[6]));
  return n;
}

dflash_status check_rope(const float* rope) {
  if (!rope) return fail(DFLASH_ERR_INVALID_ARG, "rope parameters are NULL");
  for (int i = 0; i < 7; ++i)
    if (!std::isfinite(rope[i])) return fail(DFLASH_ERR_INVALID_ARG, "rope parameter %d is not finite", i);
  if (!(rope[0] > 1.f) || !(rope[1] > 0.f) || !(rope[2] > 0.f) || !(rope[3] > 0.f) || !(rope[4] > 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "rope: theta > 1 and factor, original length, beta_fast, beta_slow > 0");
  return ok();
}

}  // namespace

extern "C" {

size_t dflash_gqa_workspace_bytes(int64_t B, int64_t bs, int64_t Hq, int64_t Hkv, int64_t Lmax) {
  size_t q, o, ml, total;
  return gqa_layout(B, bs, Hq, Hkv, Lmax, &q, &o, &ml, &total) ? total : 0;
}

dflash_status dflash_gqa_materialize(const void* ctx_hidden, const void* w_k, const void* w_v, const void* gamma_k,
                                     float eps, const float* rope, void* k_cache, void* v_cache_t, int64_t B,
                                     int64_t Lc, int64_t Lmax, int64_t hidden, int64_t Hkv, int64_t head_dim,
                                     void* stream) {
  if (!ctx_hidden || !w_k || !w_v || !gamma_k || !k_cache || !v_cache_t)
    return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(ctx_hidden) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(gamma_k) || !aligned16(k_cache) ||
      !aligned16(v_cache_t))
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  dflash_status st = check_rope(rope);
  if (st != DFLASH_OK) return st;
  if (B <= 0 || Lc <= 0 || Lmax <= 0 || hidden <= 0 || Hkv <= 0 || head_dim <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DFLASH_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (Lc > Lmax) return fail(DFLASH_ERR_INVALID_ARG, "Lc exceeds the cache length");
  if (head_dim != 128 || hidden % 32 != 0 || Lmax % 8 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "head_dim must be 128, hidden a multiple of 32, Lmax of 8");
  int64_t M, tmp;
  if (!mul_ok(B, Lc, &M) || M > INT32_MAX || B > 65535 || Lmax > INT32_MAX || hidden > INT32_MAX ||
      !mul_ok(B * Hkv, Lmax * 128, &tmp) || Hkv * 128 > INT32_MAX || !mul_ok(M, hidden, &tmp))
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  const size_t cache = static_cast<size_t>(B) * Hkv * Lmax * 128 * 2;
  const Range r[6] = {range_of(k_cache, cache), range_of(v_cache_t, cache),
                      range_of(ctx_hidden, static_cast<size_t>(M) * hidden * 2),
                      range_of(w_k, static_cast<size_t>(Hkv) * 128 * hidden * 2),
                      range_of(w_v, static_cast<size_t>(Hkv) * 128 * hidden * 2), range_of(gamma_k, 256)};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && overlaps(r[i], r[j])) return fail(DFLASH_ERR_INVALID_ARG, "a cache overlaps another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dflash::LinearArgs l = linear_args();
  l.a1 = static_cast<const uint16_t*>(ctx_hidden);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(Lc);
  l.K = static_cast<int>(hidden);
  l.w = static_cast<const uint16_t*>(w_k);
  l.N = static_cast<int>(Hkv * 128);
  l.mode = dflash::kLinearHeads;
  l.D = 128;
  l.Lt = static_cast<int>(Lmax);
  l.y1 = static_cast<uint16_t*>(k_cache);
  st = hip_status(dflash::launch_linear_bf16(l, s), "k projection launch");
  if (st != DFLASH_OK) return st;
  dflash::NormRopeArgs n = norm_rope_args(rope, gamma_k, eps);
  n.x = static_cast<uint16_t*>(k_cache);
  n.B = static_cast<int>(B);
  n.H = static_cast<int>(Hkv);
  n.Lt = static_cast<int>(Lmax);
  n.T = static_cast<int>(Lc);
  st = hip_status(dflash::launch_norm_rope_bf16(n, s), "k norm / rope launch");
  if (st != DFLASH_OK) return st;
  l.w = static_cast<const uint16_t*>(w_v);
  l.mode = dflash::kLinearHeadsT;
  l.y1 = static_cast<uint16_t*>(v_cache_t);
  return hip_status(dflash::launch_linear_bf16(l, s), "v projection launch");
}

dflash_status dflash_gqa_forward_block(const void* blk_hidden, const void* w_q, const void* w_k, const void* w_v,
                                       const void* gamma_q, const void* gamma_k, float eps, const float* rope,
                                       void* k_cache, void* v_cache_t, const int32_t* ctx_len, void* out, int64_t B,
                                       int64_t bs, int64_t Lmax, int64_t hidden, int64_t Hq, int64_t Hkv,
                                       int64_t head_dim, float scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!blk_hidden || !w_q || !w_k || !w_v || !gamma_q || !gamma_k || !k_cache || !v_cache_t || !ctx_len || !out)
    return fail(DFLASH_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(blk_hidden) || !aligned16(w_q) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(gamma_q) ||
      !aligned16(gamma_k) || !aligned16(k_cache) || !aligned16(v_cache_t) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(ctx_len) & 3u) != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned (ctx_len 4-byte)");
  dflash_status st = check_rope(rope);
  if (st != DFLASH_OK) return st;
  if (B <= 0 || bs <= 0 || Lmax <= 0 || hidden <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "sizes must be positive");
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(scale) || !(scale > 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "eps must be >= 0 and scale > 0, both finite");
  if (bs > Lmax) return fail(DFLASH_ERR_INVALID_ARG, "the block is longer than the cache");
  if (head_dim != 128 || hidden % 32 != 0 || Lmax % 8 != 0 || Hq % Hkv != 0 || (Hq / Hkv) * bs > 64)
    return fail(DFLASH_ERR_UNSUPPORTED, "head_dim 128, hidden %% 32 == 0, Lmax %% 8 == 0, Hq %% Hkv == 0 and (Hq / Hkv) * bs <= 64 required");
  if (Lmax * 128 * 2 > INT32_MAX)   // one (batch row, KV head) slice of the cache is read through a 32-bit buffer range
    return fail(DFLASH_ERR_UNSUPPORTED, "Lmax must be below 2^23 keys");
  size_t qo, oo, mlo, need;
  if (!gqa_layout(B, bs, Hq, Hkv, Lmax, &qo, &oo, &mlo, &need) || hidden > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "sizes too large");
  st = check_ws(workspace, workspace_bytes, need);
  if (st != DFLASH_OK) return st;
  const size_t cache = static_cast<size_t>(B) * Hkv * Lmax * 128 * 2;
  const Range r[10] = {range_of(k_cache, cache), range_of(v_cache_t, cache),
                       range_of(out, static_cast<size_t>(B) * Hq * bs * 128 * 2), range_of(workspace, need),
                       range_of(blk_hidden, static_cast<size_t>(B) * bs * hidden * 2),
                       range_of(w_q, static_cast<size_t>(Hq) * 128 * hidden * 2),
                       range_of(w_k, static_cast<size_t>(Hkv) * 128 * hidden * 2),
                       range_of(w_v, static_cast<size_t>(Hkv) * 128 * hidden * 2), range_of(gamma_q, 256),
                       range_of(ctx_len, static_cast<size_t>(B) * 4)};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 10; ++j)
      if (i != j && overlaps(r[i], r[j])) return fail(DFLASH_ERR_INVALID_ARG, "an output or the workspace overlaps another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* qbuf = reinterpret_cast<uint16_t*>(ws + qo);
  const size_t split_off = mlo + align_up(static_cast<size_t>(B) * Hkv * gqa_split(B, Hkv, Lmax).splits * 64 * 2 * 4, 256);
  float* split = reinterpret_cast<float*>(ws + split_off);
  const size_t split_bytes = need - split_off;
  const int off_max = static_cast<int>(Lmax - bs);
  // q: projection, then qk-norm + RoPE at positions ctx_len + t
  dflash::LinearArgs l = linear_args();
  l.a1 = static_cast<const uint16_t*>(blk_hidden);
  l.B = static_cast<int>(B);
  l.T1 = static_cast<int>(bs);
  l.K = static_cast<int>(hidden);
  l.w = static_cast<const uint16_t*>(w_q);
  l.N = static_cast<int>(Hq * 128);
  l.mode = dflash::kLinearHeads;
  l.D = 128;
  l.y1 = qbuf;
  st = hip_status(dflash::launch_linear_bf16(l, s, split, split_bytes), "q projection launch");
  if (st != DFLASH_OK) return st;
  dflash::NormRopeArgs n = norm_rope_args(rope, gamma_q, eps);
  n.x = qbuf;
  n.B = static_cast<int>(B);
  n.H = static_cast<int>(Hq);
  n.Lt = static_cast<int>(bs);
  n.T = static_cast<int>(bs);
  n.row_off = ctx_len;
  n.off_max = off_max;
  n.rows_local = 1;
  st = hip_status(dflash::launch_norm_rope_bf16(n, s), "q norm / rope launch");
  if (st != DFLASH_OK) return st;
  // the block's k and v appended to the caches at ctx_len
  l.w = static_cast<const uint16_t*>(w_k);
  l.N = static_cast<int>(Hkv * 128);
  l.y1 = static_cast<uint16_t*>(k_cache);
  l.Lt = static_cast<int>(Lmax);
  l.row_off = ctx_len;
  l.off_max = off_max;
  st = hip_status(dflash::launch_linear_bf16(l, s, split, split_bytes), "k projection launch");
  if (st != DFLASH_OK) return st;
  dflash::NormRopeArgs nk = norm_rope_args(rope, gamma_k, eps);
  nk.x = static_cast<uint16_t*>(k_cache);
  nk.B = static_cast<int>(B);
  nk.H = static_cast<int>(Hkv);
  nk.Lt = static_cast<int>(Lmax);
  nk.T = static_cast<int>(bs);
  nk.row_off = ctx_len;
  nk.off_max = off_max;
  st = hip_status(dflash::launch_norm_rope_bf16(nk, s), "k norm / rope launch");
  if (st != DFLASH_OK) return st;
  l.w = static_cast<const uint16_t*>(w_v);
  l.mode = dflash::kLinearHeadsT;
  l.y1 = static_cast<uint16_t*>(v_cache_t);
  st = hip_status(dflash::launch_linear_bf16(l, s, split, split_bytes), "v projection launch");
  if (st != DFLASH_OK) return st;
  const GqaSplit sp = gqa_split(B, Hkv, Lmax);
  dflash::GqaAttnArgs g = {};
  g.q = qbuf;
  g.k = static_cast<const uint16_t*>(k_cache);
  g.vt = static_cast<const uint16_t*>(v_cache_t);
  g.out = static_cast<uint16_t*>(out);
  g.ctx_len = ctx_len;
  g.B = static_cast<int>(B);
  g.Hq = static_cast<int>(Hq);
  g.Hkv = static_cast<int>(Hkv);
  g.bs = static_cast<int>(bs);
  g.Lmax = static_cast<int>(Lmax);
  g.splits = sp.splits;
  g.tiles_per_split = sp.tiles_per_split;
  g.scale = scale;
  g.part_o = reinterpret_cast<float*>(ws + oo);
  g.part_ml = reinterpret_cast<float*>(ws + mlo);
  return hip_status(dflash::launch_gqa_attn_bf16(g, s), "block attention launch");
}

dflash_status dflash_mla_block_occupancy(const int32_t* anchors, const int32_t* ctx_valid, int64_t B, int64_t A,
                                         int64_t block_size, int64_t ctx, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  TileLayout t;
  int64_t Lq, Lk;
  dflash_status st = check_block_args(anchors, ctx_valid, B, A, block_size, ctx, workspace, workspace_bytes, &t, &Lq, &Lk);
  if (st != DFLASH_OK) return st;
  const dflash::OccupancyArgs o = block_args(anchors, ctx_valid, B, A, block_size, ctx, Lq, Lk, workspace, t);
  return hip_status(dflash::launch_block_occupancy(o, static_cast<hipStream_t>(stream)), "block occupancy launch");
}

dflash_status dflash_mla_attn_blocks(const void* q, const void* k_nope, const void* k_rope_shared, const void* v,
                                     const int32_t* anchors, const int32_t* ctx_valid, void* out, int64_t B,
                                     int64_t H, int64_t A, int64_t block_size, int64_t ctx, int64_t Dn, int64_t Dr,
                                     int64_t Dv, float scale, dflash_dtype dt, void* workspace,
                                     size_t workspace_bytes, uint32_t flags, void* stream) {
  if (flags & ~(DFLASH_ATTN_REUSE_TILE_MAP | DFLASH_ATTN_SPLIT_KEYS))
    return fail(DFLASH_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (valid_dtype(dt) && dt != DFLASH_BF16) return fail(DFLASH_ERR_UNSUPPORTED, "the block-structure path is BF16 only");
  TileLayout t;
  int64_t Lq, Lk;
  dflash_status st = check_block_args(anchors, ctx_valid, B, A, block_size, ctx, workspace, workspace_bytes, &t, &Lq, &Lk);
  if (st != DFLASH_OK) return st;
  // the attention on the workspace's map alone: its shape, pointer and workspace checks
  const uint32_t attn_flags = (flags & DFLASH_ATTN_SPLIT_KEYS) | DFLASH_ATTN_REUSE_TILE_MAP;
  st = attn_impl(q, k_nope, k_rope_shared, v, nullptr, out, nullptr, B, H, Lq, Lk, Dn, Dr, Dv, scale, dt,
                 DFLASH_F32, workspace, workspace_bytes, attn_flags | DFLASH_ATTN_CHECK_ONLY, stream);
  if (st != DFLASH_OK) return st;
  const Range ro = range_of(out, static_cast<size_t>(B) * H * Lq * Dv * 2);
  if (overlaps(ro, range_of(anchors, static_cast<size_t>(B) * A * 4)) ||
      (ctx_valid && overlaps(ro, range_of(ctx_valid, static_cast<size_t>(B) * 4))))
    return fail(DFLASH_ERR_INVALID_ARG, "out overlaps anchors / ctx_valid");
  if (!(flags & DFLASH_ATTN_REUSE_TILE_MAP)) {
    const dflash::OccupancyArgs o = block_args(anchors, ctx_valid, B, A, block_size, ctx, Lq, Lk, workspace, t);
    st = hip_status(dflash::launch_block_occupancy(o, static_cast<hipStream_t>(stream)), "block occupancy launch");
    if (st != DFLASH_OK) return st;
  }
  return attn_impl(q, k_nope, k_rope_shared, v, nullptr, out, nullptr, B, H, Lq, Lk, Dn, Dr, Dv, scale, dt,
                   DFLASH_F32, workspace, workspace_bytes, attn_flags, stream);
}

}  // extern "C"
