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
// each mask row segment is read exactly once, one element per lane, so a wave
// load covers a full 256 B (f32) / 128 B (bf16) row segment and a ballot of the
// lanes is directly that row's visibility word.
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

// One workgroup: (1) each wave compacts the non-empty k-tiles of its
// (b, q-tile) rows into an increasing list; (2) the q-tiles are ranked by
// decreasing list length (ties: lower index first) so the attention launch can
// start the longest work first.
constexpr int kListThreads = 1024;
constexpr int kMaxRankItems = 4096;

__global__ void __launch_bounds__(kListThreads) build_lists(OccupancyArgs a) {
  __shared__ int s_counts[kMaxRankItems];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nrows = a.B * a.nqt;
  for (int row = wave; row < nrows; row += kListThreads / 64) {
    const uint8_t* cls = a.classes + static_cast<size_t>(row) * a.nkt;
    int32_t* list = a.lists + static_cast<size_t>(row) * a.nkt;
    int base = 0;
    for (int k0 = 0; k0 < a.nkt; k0 += 64) {
      const int kt = k0 + lane;
      const int c = kt < a.nkt ? cls[kt] : 0;
      const uint64_t bal = __ballot(c != 0);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (c != 0) list[base + pre] = kt | (c << 24);
      base += __popcll(bal);
    }
    if (lane == 0) a.counts[row] = base;
  }
  __syncthreads();
  if (nrows > kMaxRankItems) {  // too many q-tiles to rank here: natural order
    for (int i = threadIdx.x; i < nrows; i += kListThreads) a.order[i] = i;
    return;
  }
  for (int i = threadIdx.x; i < nrows; i += kListThreads) s_counts[i] = a.counts[i];
  __syncthreads();
  for (int i = threadIdx.x; i < nrows; i += kListThreads) {
    const int c = s_counts[i];
    int rank = 0;
    for (int j = 0; j < nrows; ++j) {
      const int cj = s_counts[j];
      rank += (cj > c) || (cj == c && j < i);
    }
    a.order[rank] = i;
  }
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

hipError_t launch_occupancy(const OccupancyArgs& a, hipStream_t s) {
  const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
  if (a.mask_bf16)
    hipLaunchKernelGGL(classify_tiles<true>, dim3(static_cast<unsigned>(ntiles)), dim3(kClassifyThreads), 0, s, a);
  else
    hipLaunchKernelGGL(classify_tiles<false>, dim3(static_cast<unsigned>(ntiles)), dim3(kClassifyThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(build_lists, dim3(1), dim3(kListThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
