// Mask-occupancy pass: classify every kTileM x kTileN tile of the dense additive
// DFlash mask (NeMo AutoModel DFlash page, KimiK3DFlashAttention.forward: the
// mask [batch, 1, Lq, ctx+Lq] is added to the scores unchanged) and build, per
// (batch, q-tile), the ordered list of tiles that contribute anything.
//
// Classes: 0 every entry exactly -inf (skipped), 1 every entry +-0 (no mask
// work), 2 only +-0 and -inf (a 64-bit visibility word per row is written so
// the attention kernel reads 8 bytes per query instead of the values),
// 3 anything else (the attention kernel adds the values).
//
// The mask is head-independent, so this runs once per call (or once for every
// draft layer, which all receive the same mask) and is pure HBM streaming:
// each mask entry is read exactly once.  Masks whose rows start 16-byte aligned
// are read 16 bytes per lane; others one entry per lane, where a wave load
// covers a 64-entry row segment and a ballot of the lanes is that row's
// visibility word.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kClassifyThreads = 256;
constexpr int kClassifyWaves = kClassifyThreads / 64;

// One workgroup per tile; grid x enumerates (b, qt, kt) with kt fastest.
template <bool BF16>
__global__ void __launch_bounds__(kClassifyThreads) classify_tiles(OccupancyArgs a) {
  __shared__ uint64_t s_vis[kTileM];
  __shared__ int s_flags[kClassifyWaves];
  const int64_t tile = blockIdx.x;
  const int kt = static_cast<int>(tile % a.nkt);
  const int64_t rest = tile / a.nkt;
  const int qt = static_cast<int>(rest % a.nqt);
  const int b = static_cast<int>(rest / a.nqt);
  const int r0 = qt * kTileM, c0 = kt * kTileN;
  const int rows = min(kTileM, a.Lq - r0);
  const int cols = min(kTileN, a.Lk - c0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool col_ok = lane < cols;
  if (tile == 0 && threadIdx.x == 0) *a.sync = 0u;   // the list pass that follows counts its workgroups
  const uint64_t valid = cols == 64 ? ~0ull : ((1ull << cols) - 1ull);

  // flag bits: 1 = some entry is not -inf, 2 = some entry is not +-0, 4 = some entry is neither
  int flags = 0;
  const size_t row0 = (static_cast<size_t>(b) * a.Lq + r0) * a.Lk + c0 + lane;
  constexpr int kRowsPerWave = kTileM / kClassifyWaves;
  uint32_t w[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = wave + kClassifyWaves * i;
    w[i] = 0xFF800000u;  // rows/cols outside the mask read as -inf and are excluded below
    if (r < rows && col_ok) {
      const size_t idx = row0 + static_cast<size_t>(r) * a.Lk;
      w[i] = BF16 ? (static_cast<uint32_t>(static_cast<const uint16_t*>(a.mask)[idx]) << 16)
                  : static_cast<const uint32_t*>(a.mask)[idx];
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = wave + kClassifyWaves * i;
    const bool zero = (w[i] & 0x7FFFFFFFu) == 0u;  // bf16 was shifted into the f32 position
    const bool ninf = w[i] == 0xFF800000u;
    const uint64_t vz = __ballot(zero) & valid;
    const uint64_t vn = __ballot(ninf) & valid;
    if (r < rows) {
      const uint64_t other = valid & ~(vz | vn);
      if ((vz | other) != 0) flags |= 1;
      if ((vn | other) != 0) flags |= 2;
      if (other != 0) flags |= 4;
      if (lane == 0) s_vis[r] = vz;
    }
  }
  if (lane == 0) s_flags[wave] = flags;
  __syncthreads();
  int f = 0;
#pragma unroll
  for (int i = 0; i < kClassifyWaves; ++i) f |= s_flags[i];
  const int cls = !(f & 1) ? 0 : (!(f & 2) ? 1 : ((f & 4) ? 3 : 2));
  if (threadIdx.x == 0) a.classes[tile] = static_cast<uint8_t>(cls);
  if (cls == 2) {
    uint64_t* dst = a.bits + static_cast<size_t>(tile) * kTileM;
    for (int r = threadIdx.x; r < kTileM; r += kClassifyThreads) dst[r] = r < rows ? s_vis[r] : 0ull;
  }
}

// Same classification with 16-byte loads, for masks whose rows start 16-byte
// aligned (Lk a multiple of 8 for bf16, of 4 for f32): lane t reads chunk t % CH
// (EPL consecutive entries) of rows t / CH + (256 / CH) * i.  A chunk's
// visibility bits are assembled into the row words through LDS.
template <bool BF16>
__global__ void __launch_bounds__(kClassifyThreads) classify_tiles_vec(OccupancyArgs a) {
  constexpr int EPL = BF16 ? 8 : 4;                 // entries per 16-byte chunk
  constexpr int CH = kTileN / EPL;                  // chunks per tile row
  constexpr int RPB = kClassifyThreads / CH;        // rows per block-wide load
  constexpr int NIT = kTileM / RPB;
  __shared__ uint8_t s_vis[kTileM][CH];
  __shared__ int s_flags[kClassifyWaves];
  // (the tile count is far below 2^31: 32-bit index arithmetic)
  const uint32_t tile = blockIdx.x;
  const uint32_t kt = tile % static_cast<uint32_t>(a.nkt);
  const uint32_t rest = tile / static_cast<uint32_t>(a.nkt);
  const uint32_t qt = rest % static_cast<uint32_t>(a.nqt);
  const uint32_t b = rest / static_cast<uint32_t>(a.nqt);
  const int r0 = static_cast<int>(qt) * kTileM, c0 = static_cast<int>(kt) * kTileN;
  const int rows = min(kTileM, a.Lq - r0);
  const int cols = min(kTileN, a.Lk - c0);          // a multiple of EPL here
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t % CH, rr = t / CH;
  if (tile == 0 && t == 0) *a.sync = 0u;              // the list pass that follows counts its workgroups
  const bool col_ok = c * EPL < cols;
  const size_t esz = BF16 ? 2 : 4;
  // chunks outside the mask read a valid chunk of the tile instead (row 0 or chunk 0,
  // always inside) and are left out of the flags and visibility bits below
  const char* base = static_cast<const char*>(a.mask) +
                     ((static_cast<size_t>(b) * a.Lq + r0) * a.Lk + c0 + (col_ok ? c * EPL : 0)) * esz;

  u32x4_t w[NIT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {                   // all loads in flight together, no branches
    const int r = rr + RPB * i;
    w[i] = ldg16(base + static_cast<size_t>(r < rows ? r : 0) * a.Lk * esz);
  }
  bool any_vis = false, any_nonzero = false, any_other = false;
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int r = rr + RPB * i;
    uint32_t vis = 0, nz_acc = 0, nn_acc = 0, ot_acc = 0;
    if constexpr (BF16) {
      // two entries per word: with a = |x| per half (< 0x8000), a + 0x7FFF has bit 15
      // of the half set exactly when that half is nonzero (no carry between halves);
      // x ^ -inf is zero exactly at -inf, and its own bit 15 covers halves >= 0x8000
      uint32_t zsh = 0;                             // zero flags of entry 2q at bit 2q, of 2q+1 at 16 + 2q
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = w[i][q];
        const uint32_t nz = ((x & 0x7FFF7FFFu) + 0x7FFF7FFFu) & 0x80008000u;        // not +-0
        const uint32_t n = x ^ 0xFF80FF80u;
        const uint32_t nn = (((n & 0x7FFF7FFFu) + 0x7FFF7FFFu) | n) & 0x80008000u;   // not -inf
        nz_acc |= nz;
        nn_acc |= nn;
        ot_acc |= nz & nn;
        zsh |= (~nz & 0x80008000u) >> (15 - 2 * q);
      }
      vis = (zsh & 0x55u) | ((zsh >> 15) & 0xAAu);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const uint32_t x = w[i][e];
        const uint32_t nz = (x & 0x7FFFFFFFu) != 0u ? 1u : 0u;
        const uint32_t nn = x != 0xFF800000u ? 1u : 0u;
        vis |= (nz ^ 1u) << e;
        nz_acc |= nz;
        nn_acc |= nn;
        ot_acc |= nz & nn;
      }
    }
    const bool in_mask = r < rows && col_ok;       // entries outside the mask do not count
    if (in_mask) {
      any_vis |= nn_acc != 0u;
      any_nonzero |= nz_acc != 0u;
      any_other |= ot_acc != 0u;
    }
    s_vis[r][c] = static_cast<uint8_t>(in_mask ? vis : 0u);
  }
  int flags = (__ballot(any_vis) ? 1 : 0) | (__ballot(any_nonzero) ? 2 : 0) | (__ballot(any_other) ? 4 : 0);
  if (lane == 0) s_flags[wave] = flags;
  __syncthreads();
  int f = 0;
#pragma unroll
  for (int i = 0; i < kClassifyWaves; ++i) f |= s_flags[i];
  const int cls = !(f & 1) ? 0 : (!(f & 2) ? 1 : ((f & 4) ? 3 : 2));
  if (t == 0) a.classes[tile] = static_cast<uint8_t>(cls);
  if (cls == 2 && t < kTileM) {
    uint64_t word = 0;
#pragma unroll
    for (int k = 0; k < CH; ++k) word |= static_cast<uint64_t>(s_vis[t][k]) << (EPL * k);
    a.bits[static_cast<size_t>(tile) * kTileM + t] = t < rows ? word : 0ull;
  }
}

// Bits [c0, c0 + cols) of the key range [lo, hi] (inclusive), relative to c0.
__device__ __forceinline__ uint64_t range_bits(int c0, int cols, int lo, int hi) {
  const int a = max(lo, c0) - c0, b = min(hi, c0 + cols - 1) - c0;
  if (b < a) return 0ull;
  const uint64_t upto = b >= 63 ? ~0ull : ((1ull << (b + 1)) - 1ull);
  const uint64_t below = a == 0 ? 0ull : ((1ull << a) - 1ull);
  return upto & ~below;
}

// Tile classes and visibility words of the DFlash block mask straight from its
// definition (no mask bytes are read): one workgroup per tile, one thread per
// tile row, whose visible keys are two ranges -- context [0, min(anchor, ctx_valid - 1)]
// and its own noise block [ctx + j*bs, ctx + (j+1)*bs).  Same output as the
// dense-mask classification of the 0 / -inf mask with that visibility.
__global__ void __launch_bounds__(kTileM) classify_blocks(OccupancyArgs a) {
  __shared__ int s_flags[kTileM / 64];
  const int64_t tile = blockIdx.x;
  const int kt = static_cast<int>(tile % a.nkt);
  const int64_t rest = tile / a.nkt;
  const int qt = static_cast<int>(rest % a.nqt);
  const int b = static_cast<int>(rest / a.nqt);
  const int r = threadIdx.x, lane = r & 63, wave = r >> 6;
  if (tile == 0 && r == 0) *a.sync = 0u;             // the list pass that follows counts its workgroups
  const int i = qt * kTileM + r;
  const int c0 = kt * kTileN;
  const int cols = min(kTileN, a.Lk - c0);
  const uint64_t valid = cols == 64 ? ~0ull : ((1ull << cols) - 1ull);
  const bool row_ok = i < a.Lq;
  uint64_t word = 0;
  if (row_ok) {
    const int j = i / a.bs;
    // anchors below -1 are clamped there so range_bits never subtracts from INT_MIN
    const int anchor = max(a.anchors[static_cast<size_t>(b) * a.A + j], -1);
    const int cv = a.ctx_valid ? min(max(a.ctx_valid[b], 0), a.ctx) : a.ctx;
    word = range_bits(c0, cols, 0, min(anchor, cv - 1)) |
           range_bits(c0, cols, a.ctx + j * a.bs, a.ctx + (j + 1) * a.bs - 1);
  }
  const int flags = (__ballot(row_ok && word != 0ull) ? 1 : 0) | (__ballot(row_ok && word != valid) ? 2 : 0);
  if (lane == 0) s_flags[wave] = flags;
  __syncthreads();
  const int f = s_flags[0] | s_flags[1];
  const int cls = !(f & 1) ? 0 : (!(f & 2) ? 1 : 2);
  if (r == 0) a.classes[tile] = static_cast<uint8_t>(cls);
  if (cls == 2) a.bits[static_cast<size_t>(tile) * kTileM + r] = word;
}

// Rank rows by decreasing list length (ties: lower index first) so the attention
// launch starts the longest work first: order[rank] = row.  n <= kMaxFusedRank.
constexpr int kRowThreads = 256;
constexpr int kMaxFusedRank = 512;
__device__ void rank_rows_block(const OccupancyArgs& a, int* s_counts, int nthreads) {
  const int nrows = a.B * a.nqt;
  for (int i = threadIdx.x; i < nrows; i += nthreads)
    s_counts[i] = __hip_atomic_load(a.counts + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  for (int i = threadIdx.x; i < nrows; i += nthreads) {
    const int c = s_counts[i];
    int rank = 0;
    for (int j = 0; j < nrows; ++j) {
      const int cj = s_counts[j];
      rank += (cj > c) || (cj == c && j < i);
    }
    a.order[rank] = i;
  }
}

// One workgroup per (b, q-tile) row: compact its non-empty k-tiles into an
// increasing list (ballot prefix counts, 256 candidates per step).  With few
// rows, the last workgroup to finish (counted in a.sync) also ranks the rows.
__global__ void __launch_bounds__(kRowThreads) build_row_lists(OccupancyArgs a, int fuse_rank) {
  __shared__ int s_wave[kRowThreads / 64];
  __shared__ int s_counts[kMaxFusedRank];
  __shared__ int s_last;
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint8_t* cls = a.classes + static_cast<size_t>(row) * a.nkt;
  int32_t* list = a.lists + static_cast<size_t>(row) * a.nkt;
  int base = 0;
  for (int k0 = 0; k0 < a.nkt; k0 += kRowThreads) {
    const int kt = k0 + t;
    const int c = kt < a.nkt ? cls[kt] : 0;
    const uint64_t bal = __ballot(c != 0);
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int before = base;
    for (int i = 0; i < wave; ++i) before += s_wave[i];
    if (c != 0) list[before + __popcll(bal & ((1ull << lane) - 1ull))] = kt | (c << 24);
    for (int i = 0; i < kRowThreads / 64; ++i) base += s_wave[i];
    __syncthreads();
  }
  if (!fuse_rank) {
    if (t == 0) a.counts[row] = base;
    return;
  }
  if (t == 0) {
    __hip_atomic_store(a.counts + row, base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned done = __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == static_cast<unsigned>(a.B * a.nqt - 1);
  }
  __syncthreads();
  if (s_last) {
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
    rank_rows_block(a, s_counts, kRowThreads);
  }
}

// One workgroup ranks many rows (more than kMaxFusedRank).
__global__ void __launch_bounds__(1024) rank_rows(OccupancyArgs a) {
  __shared__ int s_counts[4096];
  const int nrows = a.B * a.nqt;
  if (nrows > 4096) {  // too many q-tiles to rank here: natural order
    for (int i = threadIdx.x; i < nrows; i += 1024) a.order[i] = i;
    return;
  }
  rank_rows_block(a, s_counts, 1024);
}

// Every k-tile of every (b, q-tile), empty ones relabelled class 3 (their -inf
// values are then added like any other mask values and contribute exp(-inf) = 0).
__global__ void __launch_bounds__(256) lists_all_tiles(OccupancyArgs a) {
  const int row = blockIdx.x;
  const uint8_t* cls = a.classes + static_cast<size_t>(row) * a.nkt;
  int32_t* list = a.lists + static_cast<size_t>(row) * a.nkt;
  for (int kt = threadIdx.x; kt < a.nkt; kt += 256) {
    const int c = cls[kt];
    list[kt] = kt | ((c == 0 ? 3 : c) << 24);
  }
  if (threadIdx.x == 0) a.counts[row] = a.nkt;
}

}  // namespace

hipError_t launch_lists_all_tiles(const OccupancyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lists_all_tiles, dim3(static_cast<unsigned>(a.B * a.nqt)), dim3(256), 0, s, a);
  return hipGetLastError();
}

static hipError_t launch_lists(const OccupancyArgs& a, hipStream_t s) {
  const int nrows = a.B * a.nqt;
  const int fuse = nrows <= kMaxFusedRank;
  hipLaunchKernelGGL(build_row_lists, dim3(static_cast<unsigned>(nrows)), dim3(kRowThreads), 0, s, a, fuse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fuse) return e;
  hipLaunchKernelGGL(rank_rows, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_block_occupancy(const OccupancyArgs& a, hipStream_t s) {
  const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
  hipLaunchKernelGGL(classify_blocks, dim3(static_cast<unsigned>(ntiles)), dim3(kTileM), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lists(a, s);
}

hipError_t launch_occupancy(const OccupancyArgs& a, hipStream_t s) {
  const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
  const dim3 grid(static_cast<unsigned>(ntiles)), block(kClassifyThreads);
  const bool vec = a.Lk % (a.mask_bf16 ? 8 : 4) == 0;   // rows start 16-byte aligned (the base is)
  if (a.mask_bf16) {
    if (vec) hipLaunchKernelGGL(classify_tiles_vec<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(classify_tiles<true>, grid, block, 0, s, a);
  } else {
    if (vec) hipLaunchKernelGGL(classify_tiles_vec<false>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(classify_tiles<false>, grid, block, 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lists(a, s);
}

}  // namespace dflash
