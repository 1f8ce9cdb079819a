// The projections on either side of the draft attention, bf16 MFMA on gfx950.
//
// The draft's MLA (DFlash page, module text: Q-LoRA and a compressed KV latent,
// fp32-variance RMSNorm; DSpark page, KimiK3DSparkAttention attributes
// q_a_proj / q_a_layernorm / q_b_proj, kv_a_proj_with_mqa / kv_a_layernorm /
// kv_b_proj, and KimiK3DSparkModel._forward_backbone: the target context is
// projected by fc and normed once) is a chain of Linear layers with RMSNorms
// between them.  One kernel serves every Linear of the chain:
//
//   y[m, n] = sum_k a[m, k] * W[n, k]        (a from up to two row sources)
//
// with two fusions that keep the norms off HBM:
//  * statistics out: the epilogue sums the squares of its bf16-rounded outputs
//    per row over its 128-column tile and writes one partial per (row, tile);
//  * norm on load: a consumer whose input rows are an RMSNorm of the previous
//    output reads those partials (fixed order), forms r = rsqrt(mean + eps) and
//    normalises each operand chunk as it stages it into LDS:
//    a = bf16(bf16(x * r) * gamma[k]), the rounding sequence of an RMSNorm that
//    computes in fp32 and returns its input dtype times the weight.
// The tile is 128 outputs x 128 rows with four waves (2 x 2 of 64 x 64), the
// transposed product C^T = W a^T so a lane owns one row and runs of four
// consecutive outputs (8-byte stores), K staged 32 at a time through a double
// buffer with 80-byte LDS rows (conflict-free 16-byte operand reads).
#include "common.h"
#include "dma.h"
#include "launch.h"
#include "rmsnorm.h"

namespace dflash {
namespace {

// Tile shapes: NT outputs x MT rows per workgroup, K staged KS at a time, WN x WM
// waves each covering (NT / WN) x (MT / WM) as 32 x 32 MFMA blocks.
template <int NT, int MT, int KS, int WN, int WM>
struct Tile {
  static constexpr int kThreads = 64 * WN * WM;
  static constexpr int kFN = NT / WN / 32, kFM = MT / WM / 32;
  static constexpr int kRow = KS + 8;                       // bf16 per LDS row: 16 * odd bytes
  static constexpr int kStage = (NT + MT) * kRow;
  static constexpr int kChunks = KS / 8;                    // 16-byte chunks per row and stage
  static constexpr int kCW = NT * kChunks / kThreads, kCA = MT * kChunks / kThreads;
  static_assert(kFN >= 1 && kFM >= 1 && kCW >= 1 && kCA >= 1, "tile shape");
  static_assert(NT * kChunks % kThreads == 0 && MT * kChunks % kThreads == 0, "tile shape");
  static_assert(NT / WN == 64 && NT % 128 == 0, "two waves per 128-column statistics group");
};
using BigTile = Tile<256, 256, 64, 4, 2>;     // 8 waves, 64 x 128 each
using SmallTile = Tile<128, 128, 32, 2, 2>;   // 4 waves, 64 x 64 each

// Store four consecutive bf16 outputs n .. n + 3 of row m (batch row b, time tt)
// in the layout of the output mode.
template <int MODE = -1>
__device__ __forceinline__ void emit4(const LinearArgs& a, int64_t m, int64_t b, int tt, int T, int n, uint32_t p0,
                                      uint32_t p1) {
  uint16_t* dst;
  if (MODE == kLinearKV || (MODE < 0 && a.mode == kLinearKV)) {   // per head [k_nope (128) | v (128)]
    const int h = n >> 8, e = n & 255;
    dst = (e < kDn ? a.y1 : a.y2) + ((static_cast<size_t>(b) * (a.N >> 8) + h) * T + tt) * kDn + (e & 127);
  } else if (a.mode == kLinearPlain) {
    dst = a.y1 + static_cast<size_t>(m) * a.N + n;
  } else if (a.mode == kLinearSplit) {
    dst = n < a.N1 ? a.y1 + static_cast<size_t>(m) * a.N1 + n
                   : a.y2 + static_cast<size_t>(m) * (a.N - a.N1) + (n - a.N1);
  } else if (a.mode == kLinearHeads || a.mode == kLinearHeadsT) {
    const int h = n / a.D, d = n % a.D;
    const int Lt = a.Lt ? a.Lt : T;
    const int ti = (a.row_off ? min(max(a.row_off[b], 0), a.off_max) : 0) + tt;
    const size_t bh = static_cast<size_t>(b) * (a.N / a.D) + h;
    if (a.mode == kLinearHeadsT) {                  // [B, N / D, D, Lt]
      uint16_t* col = a.y1 + (bh * a.D + d) * Lt + ti;
      col[0] = static_cast<uint16_t>(p0 & 0xFFFFu);
      col[Lt] = static_cast<uint16_t>(p0 >> 16);
      col[2 * static_cast<size_t>(Lt)] = static_cast<uint16_t>(p1 & 0xFFFFu);
      col[3 * static_cast<size_t>(Lt)] = static_cast<uint16_t>(p1 >> 16);
      return;
    }
    dst = a.y1 + (bh * Lt + ti) * a.D + d;          // [B, N / D, Lt, D]
  } else {
    return;
  }
  *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{p0, p1};
}

template <int NT, int MT, int KS, int WN, int WM>
__global__ void __launch_bounds__(64 * WN * WM) linear_bf16(LinearArgs a) {
  using TL = Tile<NT, MT, KS, WN, WM>;
  constexpr int FN = TL::kFN, FM = TL::kFM, ROW = TL::kRow, CH = TL::kChunks, NTH = TL::kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TL::kStage];
  __shared__ float s_part[WN][MT];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int li = lane & 31, hi = lane >> 5;
  const int T = a.T1 + a.T2;
  const int64_t M = static_cast<int64_t>(a.B) * T;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * MT;
  const int n0 = blockIdx.y * NT;

  // this thread's staging rows (A side: rows m, with their sources and norm scales)
  const uint16_t* arow[TL::kCA];
  bool aok[TL::kCA];
  float rsc[TL::kCA];
#pragma unroll
  for (int i = 0; i < TL::kCA; ++i) {
    const int row = (t + NTH * i) / CH;
    const int64_t m = m0 + row;
    aok[i] = m < M;
    const int64_t mm = aok[i] ? m : 0;
    const int64_t b = mm / T;
    const int tt = static_cast<int>(mm % T);
    arow[i] = tt < a.T1 ? a.a1 + (static_cast<size_t>(b) * a.T1 + tt) * a.K
                        : a.a2 + (static_cast<size_t>(b) * a.T2 + (tt - a.T1)) * a.K;
    rsc[i] = (a.stats_in && aok[i]) ? rms_row_scale(a.stats_in, a.stats_parts, m, a.K, a.eps) : 1.f;
  }

  u32x4_t sw[TL::kCW], sl[TL::kCA];
  auto load = [&](int k0) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < TL::kCW; ++i) {
      const int ci = t + NTH * i, row = ci / CH, c = ci % CH;
      sw[i] = n0 + row < a.N ? ldg16(a.w + static_cast<size_t>(n0 + row) * a.K + k0 + c * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < TL::kCA; ++i) {
      const int c = (t + NTH * i) % CH;
      sl[i] = aok[i] ? ldg16(arow[i] + k0 + c * 8) : z;
      if (a.stats_in && aok[i]) sl[i] = rms_norm_chunk(sl[i], rsc[i], ldg16(a.gamma + k0 + c * 8));
    }
  };
  auto store = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < TL::kCW; ++i) {
      const int ci = t + NTH * i;
      stg16(buf + (ci / CH) * ROW + (ci % CH) * 8, sw[i]);
    }
#pragma unroll
    for (int i = 0; i < TL::kCA; ++i) {
      const int ci = t + NTH * i;
      stg16(buf + (NT + ci / CH) * ROW + (ci % CH) * 8, sl[i]);
    }
  };

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int kc = a.split_part ? a.K / gridDim.z : a.K;   // this workgroup's share of K
  const int kbeg = blockIdx.z * kc;
  const int nk = kc / KS;
  load(kbeg);
  store(smem);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const bool more = it + 1 < nk;
    if (more) load(kbeg + (it + 1) * KS);
    const uint16_t* Ws = smem + (it & 1) * TL::kStage;
    const uint16_t* Ls = Ws + NT * ROW;
#pragma unroll
    for (int ks = 0; ks < KS / 16; ++ks) {
      bf16x8_t af[FN], bf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ws + ((NT / WN) * wn + 32 * i + li) * ROW + 16 * ks + 8 * hi));
#pragma unroll
      for (int j = 0; j < FM; ++j)
        bf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ls + ((MT / WM) * wm + 32 * j + li) * ROW + 16 * ks + 8 * hi));
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (more) store(smem + ((it + 1) & 1) * TL::kStage);
    __syncthreads();
  }

  // epilogue: lane owns row m (column li of sub-tile j) and outputs
  // n = n0 + (NT/WN)*wn + 32*i + 8*g + 4*hi + 0..3 (registers 4g + 0..3 of acc[i][j])
  if (a.split_part) {                                 // split K: fp32 partials, reduced in order later
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + (MT / WM) * wm + 32 * j + li;
      if (m >= M) continue;
      float* prow = a.split_part + (static_cast<size_t>(blockIdx.z) * M + m) * a.N;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + (NT / WN) * wn + 32 * i + 8 * g + 4 * hi;
          if (n < a.N)
            *reinterpret_cast<f32x4_t*>(prow + n) =
                f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
    }
    return;
  }
  const bool stats = a.stats_out && n0 < a.Nstat;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int rl = (MT / WM) * wm + 32 * j + li;
    const int64_t m = m0 + rl;
    const bool mok = m < M;
    const int64_t mm = mok ? m : 0;
    const int64_t b = mm / T;
    const int tt = static_cast<int>(mm % T);
    float ssq = 0.f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + (NT / WN) * wn + 32 * i + 8 * g + 4 * hi;
        const uint32_t p0 = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        const uint32_t p1 = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if (n < a.N) {
          const float x0 = bf16_bits_to_f32(p0 & 0xFFFFu), x1 = bf16_bits_to_f32(p0 >> 16);
          const float x2 = bf16_bits_to_f32(p1 & 0xFFFFu), x3 = bf16_bits_to_f32(p1 >> 16);
          ssq += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          if (mok) emit4(a, m, b, tt, T, n, p0, p1);
        }
      }
    if (stats) {
      ssq += __shfl_xor(ssq, 32);                     // the other half of this row's outputs
      if (hi == 0) s_part[wn][rl] = ssq;
    }
  }
  if (stats) {                                        // one partial per 128-column group
    __syncthreads();
    constexpr int G = NT / 128;
    const int parts = a.Nstat / 128;
    for (int idx = t; idx < MT * G; idx += NTH) {
      const int r = idx % MT, gi = idx / MT;
      const int part = n0 / 128 + gi;
      const int64_t m = m0 + r;
      if (m < M && part < parts) a.stats_out[m * parts + part] = s_part[2 * gi][r] + s_part[2 * gi + 1][r];
    }
  }
}

// The 256 x 256 tile with its operands copied global -> LDS by the buffer unit
// (no staging registers) three stages deep, K = 32 per stage.  A stage holds 256
// W rows then 256 rows of a, 80 bytes each (64 of data + 16 of padding, which
// keeps the 16-byte operand reads conflict-free): 2560 16-byte chunks = 40 copy
// instructions of 64 lanes, five per wave; waves 0-3 copy W, waves 4-7 copy a.
// Lane l of copy j of wave w fills chunk c = (5w + j) * 64 + l, i.e. row c / 5,
// column c % 5; the padding column re-reads column 0 (any valid address).  Rows
// past N or M read zeros through the descriptors' ranges.  For single-source a
// without norm-on-load.
constexpr int kKS_DMA = 32;
constexpr int kDmaStages = 3;
constexpr int kDmaRow = 80;                                      // bytes per LDS row
constexpr int kDmaStage = 512 * kDmaRow;                         // 40960 bytes

__global__ void __launch_bounds__(512) linear_bf16_dma(LinearArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kDmaStages * kDmaStage];
  __shared__ float s_part[4][256];
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 3, wm = wave >> 2;
  const int li = lane & 31, hi = lane >> 5;
  const int T = a.T1 + a.T2;
  const int64_t M = static_cast<int64_t>(a.B) * T;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int n0 = blockIdx.y * 256;
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2;

  // copy plan of this wave: one descriptor (W or a), five chunk offsets
  const bool is_w = wave < 4;
  const int64_t nrows = is_w ? min(256, a.N - n0) : static_cast<int64_t>(min<int64_t>(256, M - m0));
  const u32x4_t rs = buffer_desc(is_w ? static_cast<const void*>(a.w + static_cast<size_t>(n0) * a.K)
                                      : static_cast<const void*>(a.a1 + static_cast<size_t>(m0) * a.K),
                                 static_cast<uint32_t>(nrows * row_bytes));
  uint32_t voff[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int c = (5 * wave + j) * 64 + lane;
    const int row = c / 5 - (is_w ? 0 : 256), col = c % 5;
    voff[j] = static_cast<uint32_t>(row) * row_bytes + (col == 4 ? 0 : col) * 16;
  }
  const uint32_t lds_copy = lds0 + 5 * wave * 1024;
  auto issue = [&](int it) __attribute__((always_inline)) {
    const uint32_t base = lds_copy + (it % kDmaStages) * kDmaStage;
    const uint32_t soff = static_cast<uint32_t>(it) * (kKS_DMA * 2);
    dma16<0>(rs, base, voff[0], soff);
    dma16<1024>(rs, base, voff[1], soff);
    dma16<2048>(rs, base, voff[2], soff);
    dma16<3072>(rs, base, voff[3], soff);
    dma16<4096>(rs, base, voff[4], soff);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.K / kKS_DMA;
  issue(0);
  if (nk > 1) issue(1);
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) wait_vmem<5>(); else wait_vmem<0>();   // this wave's copies of stage it
    __syncthreads();                                        // everyone's; stage it-1 fully read
    if (it + 2 < nk) issue(it + 2);
    const char* Ws = smem + (it % kDmaStages) * kDmaStage;
    const char* Ls = Ws + 256 * kDmaRow;
#pragma unroll
    for (int ks = 0; ks < kKS_DMA / 16; ++ks) {
      bf16x8_t af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ws + (64 * wn + 32 * i + li) * kDmaRow + (16 * ks + 8 * hi) * 2));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ls + (128 * wm + 32 * j + li) * kDmaRow + (16 * ks + 8 * hi) * 2));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  }

  // epilogue: as linear_bf16 (lane owns row m; outputs n0 + 64 wn + 32 i + 8 g + 4 hi + 0..3)
  const bool stats = a.stats_out && n0 < a.Nstat;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rl = 128 * wm + 32 * j + li;
    const int64_t m = m0 + rl;
    const bool mok = m < M;
    const int64_t mm = mok ? m : 0;
    const int64_t b = mm / T;
    const int tt = static_cast<int>(mm % T);
    float ssq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 64 * wn + 32 * i + 8 * g + 4 * hi;
        const uint32_t p0 = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        const uint32_t p1 = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if (n < a.N) {
          const float x0 = bf16_bits_to_f32(p0 & 0xFFFFu), x1 = bf16_bits_to_f32(p0 >> 16);
          const float x2 = bf16_bits_to_f32(p1 & 0xFFFFu), x3 = bf16_bits_to_f32(p1 >> 16);
          ssq += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          if (mok) emit4(a, m, b, tt, T, n, p0, p1);
        }
      }
    if (stats) {
      ssq += __shfl_xor(ssq, 32);
      if (hi == 0) s_part[wn][rl] = ssq;
    }
  }
  if (stats) {
    __syncthreads();
    const int parts = a.Nstat / 128;
    for (int idx = t; idx < 2 * 256; idx += 512) {
      const int r = idx % 256, gi = idx / 256;
      const int part = n0 / 128 + gi;
      const int64_t m = m0 + r;
      if (m < M && part < parts) a.stats_out[m * parts + part] = s_part[2 * gi][r] + s_part[2 * gi + 1][r];
    }
  }
}

// A deeper copy pipeline for GEMMs whose K is short next to the latency of a
// global load: S stages of K = 32, S - 1 of them in flight, copied global -> LDS
// by the buffer unit.  A stage holds NT W rows then MT rows of a, 64 bytes each,
// as 1 KiB blocks of 16 rows in which the four 16-byte pieces of a row are
// permuted by the row (piece p at position p ^ ((row >> 2) & 3)): the 16-byte
// operand reads of 16 lanes hit distinct banks without padding.  Each wave
// copies the same number of blocks per stage and a stage past the end copies
// with an offset beyond the resources (zeros), so the wait counts are constants.
// For single-source a without norm-on-load.
template <int NT, int MT, int WN, int WM, int S>
struct DmaTile {
  static constexpr int kWaves = WN * WM, kThreads = 64 * kWaves;
  static constexpr int kFN = NT / WN / 32, kFM = MT / WM / 32;
  static constexpr int kWBlocks = NT / 16, kBlocks = (NT + MT) / 16;
  // copy blocks per wave; the last blocks of a stage may be spare (past the end, zeros)
  static constexpr int kPerWave = (kBlocks + kWaves - 1) / kWaves;
  static constexpr int kStage = kPerWave * kWaves * 1024;
  static_assert(kFN >= 1 && kFM >= 1 && NT % 16 == 0 && MT % 32 == 0, "tile shape");
  static_assert(NT / WN == 64 && NT % 128 == 0, "two waves per 128-column statistics group");
  static_assert(kPerWave * (S - 1) < 64 && S * kStage + WN * MT * 4 <= 160 * 1024, "pipeline depth");
};

template <int NT, int MT, int WN, int WM, int S, int MODE>
__global__ void __launch_bounds__(64 * WN * WM) linear_dma(LinearArgs a) {
  using TL = DmaTile<NT, MT, WN, WM, S>;
  constexpr int FN = TL::kFN, FM = TL::kFM, PW = TL::kPerWave;
  __shared__ __attribute__((aligned(1024))) char smem[S * TL::kStage];
  __shared__ float s_part[WN][MT];
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)smem));
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int li = lane & 31, hi = lane >> 5;
  const int T = a.T1 + a.T2;
  const int64_t M = static_cast<int64_t>(a.B) * T;
  // tile of this workgroup: workgroups go to the 8 XCDs in turn, so XCD x gets
  // M quarter x / 2 and N half x % 2 of the tiles (its operands share its L2)
  int bx = blockIdx.x, by = blockIdx.y;
  if (gridDim.x % 4 == 0 && gridDim.y % 2 == 0) {
    const int id = blockIdx.y * gridDim.x + blockIdx.x, x = id % 8, j = id / 8;
    const int mq = gridDim.x / 4;
    bx = mq * (x / 2) + j % mq;
    by = (gridDim.y / 2) * (x % 2) + j / mq;
  }
  const int64_t m0 = static_cast<int64_t>(bx) * MT;
  const int n0 = by * NT;
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2;

  // copy plan: block blk = PW * wave + j of a stage; lane l fills row 16 (blk mod
  // its operand) + l / 4, position l & 3 with piece (l & 3) ^ swz
  constexpr uint32_t kPastEnd = 0x80000000u;           // beyond every resource (the host bounds them by 2^31 bytes)
  const u32x4_t dw = buffer_desc(a.w + static_cast<size_t>(n0) * a.K,
                                 static_cast<uint32_t>(min(NT, a.N - n0)) * row_bytes);
  const u32x4_t da = buffer_desc(a.a1 + static_cast<size_t>(m0) * a.K,
                                 static_cast<uint32_t>(min<int64_t>(MT, M - m0)) * row_bytes);
  uint32_t voff[PW];
  bool isw[PW];
  {
    const int r16 = lane >> 2, pos = lane & 3;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int blk = PW * wave + j;
      isw[j] = blk < TL::kWBlocks;
      const int row = 16 * (isw[j] ? blk : blk - TL::kWBlocks) + r16;
      voff[j] = blk >= TL::kBlocks ? kPastEnd
              : static_cast<uint32_t>(row) * row_bytes + static_cast<uint32_t>((pos ^ ((r16 >> 2) & 3)) * 16);
    }
  }
  const int nk = a.K / 32;
  auto issue = [&](int it) __attribute__((always_inline)) {
    const uint32_t base = lds0 + (it % S) * TL::kStage + PW * wave * 1024;
    const uint32_t soff = it < nk ? static_cast<uint32_t>(it) * 64u : kPastEnd;
#pragma unroll
    for (int j = 0; j < PW; ++j) dma16<0>(isw[j] ? dw : da, base + j * 1024, voff[j], soff);
  };
  // operand reads: row r of the stage, 16-byte piece p
  const int rsw = (li >> 2) & 3;
  auto rd = [&](const char* st, int row, int p) __attribute__((always_inline)) -> bf16x8_t {
    return as_bf16x8(*reinterpret_cast<const u32x4_t*>(st + (row >> 4) * 1024 + (row & 15) * 64 + ((p ^ rsw) << 4)));
  };

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  for (int it = 0; it < nk; ++it) {
    wait_vmem<PW * (S - 2)>();                          // this wave's copies of stage it
    __syncthreads();                                    // everyone's; stage it - 1 fully read
    issue(it + S - 1);
    const char* st = smem + (it % S) * TL::kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[FN], bf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) af[i] = rd(st, (NT / WN) * wn + 32 * i + li, 2 * ks + hi);
#pragma unroll
      for (int j = 0; j < FM; ++j) bf[j] = rd(st, NT + (MT / WM) * wm + 32 * j + li, 2 * ks + hi);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  }
  wait_vmem<0>();

  // epilogue: as linear_bf16 (lane owns row m; outputs n0 + 64 wn + 32 i + 8 g + 4 hi + 0..3);
  // MODE >= 0 fixes the output mode at compile time (no statistics)
  const bool stats = MODE < 0 && a.stats_out && n0 < a.Nstat;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int rl = (MT / WM) * wm + 32 * j + li;
    const int64_t m = m0 + rl;
    const bool mok = m < M;
    const int64_t mm = mok ? m : 0;
    const int64_t b = mm / T;
    const int tt = static_cast<int>(mm % T);
    float ssq = 0.f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 64 * wn + 32 * i + 8 * g + 4 * hi;
        const uint32_t p0 = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        const uint32_t p1 = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if (n < a.N) {
          const float x0 = bf16_bits_to_f32(p0 & 0xFFFFu), x1 = bf16_bits_to_f32(p0 >> 16);
          const float x2 = bf16_bits_to_f32(p1 & 0xFFFFu), x3 = bf16_bits_to_f32(p1 >> 16);
          ssq += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          if (mok) emit4<MODE>(a, m, b, tt, T, n, p0, p1);
        }
      }
    if (stats) {
      ssq += __shfl_xor(ssq, 32);
      if (hi == 0) s_part[wn][rl] = ssq;
    }
  }
  if (stats) {
    __syncthreads();
    constexpr int G = NT / 128;
    const int parts = a.Nstat / 128;
    for (int idx = t; idx < MT * G; idx += TL::kThreads) {
      const int r = idx % MT, gi = idx / MT;
      const int part = n0 / 128 + gi;
      const int64_t m = m0 + r;
      if (m < M && part < parts) a.stats_out[m * parts + part] = s_part[2 * gi][r] + s_part[2 * gi + 1][r];
    }
  }
}

// Split-K reduction: the partials of each output are summed in split order and
// the result goes through the same epilogue (rounding, layout, statistics).  One
// thread per row and 4 columns; 32 threads cover one 128-column group.
__global__ void __launch_bounds__(256) linear_split_reduce(LinearArgs a, int splits) {
  const int T = a.T1 + a.T2;
  const int64_t M = static_cast<int64_t>(a.B) * T;
  const int groups = (a.N + 127) / 128;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (gid >= M * groups) return;                    // whole 32-thread groups leave together
  const int l32 = threadIdx.x & 31;
  const int64_t m = gid / groups;
  const int grp = static_cast<int>(gid % groups);
  const int n = grp * 128 + 4 * l32;
  const int64_t b = m / T;
  const int tt = static_cast<int>(m % T);
  float ssq = 0.f;
  if (n < a.N) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) v += *reinterpret_cast<const f32x4_t*>(a.split_part + (static_cast<size_t>(z) * M + m) * a.N + n);
    const uint32_t p0 = pack_bf16x2(v[0], v[1]), p1 = pack_bf16x2(v[2], v[3]);
    const float x0 = bf16_bits_to_f32(p0 & 0xFFFFu), x1 = bf16_bits_to_f32(p0 >> 16);
    const float x2 = bf16_bits_to_f32(p1 & 0xFFFFu), x3 = bf16_bits_to_f32(p1 >> 16);
    ssq = x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
    emit4(a, m, b, tt, T, n, p0, p1);
  }
  if (a.stats_out && grp * 128 < a.Nstat) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) ssq += __shfl_xor(ssq, o);
    if (l32 == 0) a.stats_out[m * (a.Nstat / 128) + grp] = ssq;
  }
}

// RMSNorm from producer statistics: y = bf16(bf16(x * r) * gamma), r = rsqrt(mean(x^2) + eps).
// One workgroup per row: thread 0 sums the row's partials once, every thread then
// normalises 8-entry chunks of the row.
__global__ void __launch_bounds__(256) rms_apply_bf16(RmsApplyArgs a) {
  __shared__ float s_r;
  const int64_t m = blockIdx.x;
  if (threadIdx.x == 0) s_r = rms_row_scale(a.stats, a.parts, m, a.N, a.eps);
  __syncthreads();
  const float r = s_r;
  const uint16_t* xr = a.x + static_cast<size_t>(m) * a.N;
  uint16_t* yr = a.y + static_cast<size_t>(m) * a.N;
  for (int c = threadIdx.x; c < a.N / 8; c += 256)
    stg16(yr + 8 * c, rms_norm_chunk(ldg16(xr + 8 * c), r, ldg16(a.gamma + 8 * c)));
}

}  // namespace

// The 256 x 256 tile moves half the operand bytes per flop of the 128 x 128 one,
// but one workgroup fills a CU, so it is taken only when its tiles fill the
// 256 CUs in whole rounds (at least 85% of the last round busy, or many rounds)
// and the long K loop amortises the prologue and epilogue.
static bool linear_big_tile(const LinearArgs& a) {
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  const int64_t tiles = ((M + 255) / 256) * ((a.N + 255) / 256);
  if (a.K % 64 != 0 || a.K < 1024 || tiles < 240) return false;
  const int64_t rounds = (tiles + 255) / 256;
  return rounds >= 4 || tiles * 100 >= rounds * 256 * 85;
}

// Splits of K when the 128 x 128 output tiles cannot fill the chip on their own:
// double while the workgroups stay under ~2 per CU and every split keeps >= 256
// of K in whole 32-wide stages.
static int linear_splits(const LinearArgs& a) {
  if (linear_big_tile(a)) return 1;
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  const int64_t tiles = ((M + 127) / 128) * ((a.N + 127) / 128);
  int sp = 1;
  while (sp * 2 <= kLinearMaxSplits && tiles * sp * 2 <= 512 && a.K % (32 * sp * 2) == 0 && a.K / (sp * 2) >= 256)
    sp *= 2;
  return sp;
}

size_t linear_split_bytes(const LinearArgs& a) {
  const int sp = linear_splits(a);
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  return sp > 1 ? static_cast<size_t>(sp) * M * a.N * 4 : 0;
}

// The deep-pipeline tile (288 rows x 256 outputs, 12 waves, four stages) for the
// latent expand: its K (the latent rank) is short next to the copy latency, and
// its output is large.  Taken when the tiles fill the chip's 256 CUs in one
// round of at least 7/8 (a second, partly filled round would cost a whole tile).
constexpr int kDeepMT = 288, kDeepNT = 256;
static bool linear_deep(const LinearArgs& a) {
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  if (a.mode != kLinearKV || a.stats_in || a.stats_out || a.split_part || (a.T2 != 0 && a.a2)) return false;
  if (a.K % 32 != 0 || a.K > 1024) return false;
  const int64_t tiles = ((M + kDeepMT - 1) / kDeepMT) * ((a.N + kDeepNT - 1) / kDeepNT);
  return tiles >= 224 && tiles <= 256;
}

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t s, float* scratch, size_t scratch_bytes) {
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  if (linear_deep(a)) {
    const dim3 grid(static_cast<unsigned>((M + kDeepMT - 1) / kDeepMT), static_cast<unsigned>((a.N + kDeepNT - 1) / kDeepNT));
    hipLaunchKernelGGL((linear_dma<kDeepNT, kDeepMT, 4, 3, 4, kLinearKV>), grid, dim3(768), 0, s, a);
    return hipGetLastError();
  }
  const int sp = linear_splits(a);
  if (sp > 1 && scratch && scratch_bytes >= linear_split_bytes(a)) {
    LinearArgs b = a;
    b.split_part = scratch;
    const dim3 grid(static_cast<unsigned>((M + 127) / 128), static_cast<unsigned>((a.N + 127) / 128), sp);
    hipLaunchKernelGGL((linear_bf16<128, 128, 32, 2, 2>), grid, dim3(SmallTile::kThreads), 0, s, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = M * ((a.N + 127) / 128);
    hipLaunchKernelGGL(linear_split_reduce, dim3(static_cast<unsigned>((items + 7) / 8)), dim3(256), 0, s, b, sp);
    return hipGetLastError();
  }
  if (linear_big_tile(a)) {
    const dim3 grid(static_cast<unsigned>((M + 255) / 256), static_cast<unsigned>((a.N + 255) / 256));
    const bool dma = !a.stats_in && (a.T2 == 0 || !a.a2) && static_cast<int64_t>(a.K) * 2 * 256 <= INT32_MAX;
    if (dma) hipLaunchKernelGGL(linear_bf16_dma, grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((linear_bf16<256, 256, 64, 4, 2>), grid, dim3(BigTile::kThreads), 0, s, a);
  } else {
    const dim3 grid(static_cast<unsigned>((M + 127) / 128), static_cast<unsigned>((a.N + 127) / 128));
    hipLaunchKernelGGL((linear_bf16<128, 128, 32, 2, 2>), grid, dim3(SmallTile::kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rms_apply_bf16(const RmsApplyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rms_apply_bf16, dim3(static_cast<unsigned>(a.M)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
