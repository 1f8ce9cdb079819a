// Mask-occupancy pass: classify every kTileM x kTileN tile of the dense additive
// DFlash mask (NeMo AutoModel DFlash page, KimiK3DFlashAttention.forward: the
// mask [batch, 1, Lq, ctx+Lq] is added to the scores unchanged) and build, per
// (batch, q-tile), the ordered list of tiles that contribute anything.
//
// The mask is head-independent, so this runs once per call (or once for every
// draft layer, which all receive the same mask) and is pure HBM streaming:
// each mask byte is read exactly once with 16-byte loads.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kClassifyThreads = 256;

// Bit-pattern tests: only exactly -inf is "masked"; +0 and -0 are "zero".
__device__ __forceinline__ void scan_f32(uint32_t w, bool& all_ninf, bool& all_zero) {
  all_ninf &= (w == 0xFF800000u);
  all_zero &= ((w & 0x7FFFFFFFu) == 0u);
}
__device__ __forceinline__ void scan_bf16x2(uint32_t w, bool& all_ninf, bool& all_zero) {
  all_ninf &= (w == 0xFF80FF80u);
  all_zero &= ((w & 0x7FFF7FFFu) == 0u);
}

// One workgroup per tile.  Grid x enumerates (b, qt, kt) with kt fastest, so
// neighbouring workgroups stream neighbouring 256 B (f32) / 128 B (bf16) row segments.
template <bool BF16>
__global__ void __launch_bounds__(kClassifyThreads) classify_tiles(OccupancyArgs a, int vec_ok) {
  const int64_t tile = blockIdx.x;
  const int kt = static_cast<int>(tile % a.nkt);
  const int64_t rest = tile / a.nkt;
  const int qt = static_cast<int>(rest % a.nqt);
  const int b = static_cast<int>(rest / a.nqt);
  const int r0 = qt * kTileM, c0 = kt * kTileN;
  const int rows = min(kTileM, a.Lq - r0);
  const int cols = min(kTileN, a.Lk - c0);
  const int t = threadIdx.x;
  bool all_ninf = true, all_zero = true;

  const size_t esz = BF16 ? 2 : 4;
  const char* base = static_cast<const char*>(a.mask) +
                     ((static_cast<size_t>(b) * a.Lq + r0) * a.Lk + c0) * esz;
  const size_t row_bytes = static_cast<size_t>(a.Lk) * esz;

  if (vec_ok && cols == kTileN) {
    // 16-byte chunks: a 64-wide row is 16 chunks (f32) or 8 chunks (bf16).
    constexpr int kChunksPerRow = BF16 ? 8 : 16;
    constexpr int kShift = BF16 ? 3 : 4;
    constexpr int kChunks = kTileM * kChunksPerRow;
#pragma unroll
    for (int i = 0; i < kChunks / kClassifyThreads; ++i) {
      const int ch = t + i * kClassifyThreads;
      const int row = ch >> kShift;
      const int c = ch & (kChunksPerRow - 1);
      if (row < rows) {
        const u32x4_t w = ldg16(base + row * row_bytes + c * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) scan_bf16x2(w[j], all_ninf, all_zero);
          else scan_f32(w[j], all_ninf, all_zero);
        }
      }
    }
  } else {
    const int n = rows * cols;
    for (int e = t; e < n; e += kClassifyThreads) {
      const int row = e / cols, col = e % cols;
      const char* p = base + row * row_bytes + col * esz;
      if (BF16) {
        const uint32_t h = *reinterpret_cast<const uint16_t*>(p);
        all_ninf &= (h == 0xFF80u);
        all_zero &= ((h & 0x7FFFu) == 0u);
      } else {
        scan_f32(*reinterpret_cast<const uint32_t*>(p), all_ninf, all_zero);
      }
    }
  }
  const int any_not_ninf = __syncthreads_or(!all_ninf);
  const int any_not_zero = __syncthreads_or(!all_zero);
  if (t == 0) a.classes[tile] = any_not_ninf ? (any_not_zero ? 2 : 1) : 0;
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

}  // namespace

hipError_t launch_occupancy(const OccupancyArgs& a, hipStream_t s) {
  const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
  const size_t esz = a.mask_bf16 ? 2 : 4;
  const int vec_ok = ((static_cast<size_t>(a.Lk) * esz) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.mask) % 16 == 0);
  if (a.mask_bf16)
    hipLaunchKernelGGL(classify_tiles<true>, dim3(static_cast<unsigned>(ntiles)), dim3(kClassifyThreads), 0, s, a, vec_ok);
  else
    hipLaunchKernelGGL(classify_tiles<false>, dim3(static_cast<unsigned>(ntiles)), dim3(kClassifyThreads), 0, s, a, vec_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(build_lists, dim3(1), dim3(kListThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
