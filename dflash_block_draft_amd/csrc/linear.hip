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
#include "launch.h"
#include "rmsnorm.h"

namespace dflash {
namespace {

constexpr int kNT = 128;            // outputs per tile
constexpr int kMT = 128;            // rows per tile
constexpr int kKS = 32;             // k per LDS stage
constexpr int kRowStride = kKS + 8; // bf16 per LDS row
constexpr int kStage = (kNT + kMT) * kRowStride;

__global__ void __launch_bounds__(256) linear_bf16(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
  __shared__ float s_part[2][kMT];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int li = lane & 31, hi = lane >> 5;
  const int T = a.T1 + a.T2;
  const int64_t M = static_cast<int64_t>(a.B) * T;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kMT;
  const int n0 = blockIdx.y * kNT;
  const uint16_t* W = a.w;

  // this thread's two staging rows (A side) and their sources
  const uint16_t* arow[2];
  bool aok[2], wok[2];
  float rsc[2] = {1.f, 1.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ci = t + 256 * i, row = ci >> 2;
    const int64_t m = m0 + row;
    aok[i] = m < M;
    const int64_t mm = aok[i] ? m : 0;
    const int64_t b = mm / T;
    const int tt = static_cast<int>(mm % T);
    arow[i] = tt < a.T1 ? a.a1 + (static_cast<size_t>(b) * a.T1 + tt) * a.K
                        : a.a2 + (static_cast<size_t>(b) * a.T2 + (tt - a.T1)) * a.K;
    wok[i] = n0 + row < a.N;
    if (a.stats_in && aok[i]) rsc[i] = rms_row_scale(a.stats_in, a.stats_parts, m, a.K, a.eps);
  }

  u32x4_t sw[2], sl[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + 256 * i, row = ci >> 2, c = ci & 3;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      sw[i] = wok[i] ? ldg16(W + static_cast<size_t>(n0 + row) * a.K + k0 + c * 8) : z;
      sl[i] = aok[i] ? ldg16(arow[i] + k0 + c * 8) : z;
      if (a.stats_in && aok[i]) sl[i] = rms_norm_chunk(sl[i], rsc[i], ldg16(a.gamma + k0 + c * 8));
    }
  };
  auto store = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + 256 * i, row = ci >> 2, c = ci & 3;
      stg16(buf + row * kRowStride + c * 8, sw[i]);
      stg16(buf + (kNT + row) * kRowStride + c * 8, sl[i]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.K / kKS;
  load(0);
  store(smem);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const bool more = it + 1 < nk;
    if (more) load((it + 1) * kKS);
    const uint16_t* Ws = smem + (it & 1) * kStage;
    const uint16_t* Ls = Ws + kNT * kRowStride;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ws + (64 * wn + 32 * i + li) * kRowStride + 16 * ks + 8 * hi));
        bf[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ls + (64 * wm + 32 * i + li) * kRowStride + 16 * ks + 8 * hi));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (more) store(smem + ((it + 1) & 1) * kStage);
    __syncthreads();
  }

  // epilogue: lane owns row m (column li of sub-tile j) and outputs
  // n = n0 + 64*wn + 32*i + 8*g + 4*hi + 0..3 (register 4g + 0..3 of acc[i][j])
  const bool stats = a.stats_out && n0 < a.Nstat;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rl = 64 * wm + 32 * j + li;
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
          if (mok) {
            uint16_t* dst;
            if (a.mode == kLinearPlain) {
              dst = a.y1 + static_cast<size_t>(m) * a.N + n;
            } else if (a.mode == kLinearSplit) {
              dst = n < a.N1 ? a.y1 + static_cast<size_t>(m) * a.N1 + n
                             : a.y2 + static_cast<size_t>(m) * (a.N - a.N1) + (n - a.N1);
            } else {                                   // heads: [B, N / D, T, D]
              const int h = n / a.D, d = n % a.D;
              dst = a.y1 + ((static_cast<size_t>(b) * (a.N / a.D) + h) * T + tt) * a.D + d;
            }
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{p0, p1};
          }
        }
      }
    if (stats) {
      ssq += __shfl_xor(ssq, 32);                     // the other half of this row's outputs
      if (hi == 0) s_part[wn][rl] = ssq;
    }
  }
  if (stats) {
    __syncthreads();
    if (t < kMT) {
      const int64_t m = m0 + t;
      if (m < M) a.stats_out[m * (a.Nstat / kNT) + blockIdx.y] = s_part[0][t] + s_part[1][t];
    }
  }
}

// RMSNorm from producer statistics: y = bf16(bf16(x * r) * gamma), r = rsqrt(mean(x^2) + eps).
// One thread per 8 consecutive entries.
__global__ void __launch_bounds__(256) rms_apply_bf16(RmsApplyArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = a.N / 8;
  if (i >= a.M * per_row) return;
  const int64_t m = i / per_row;
  const int c = static_cast<int>(i % per_row);
  const float r = rms_row_scale(a.stats, a.parts, m, a.N, a.eps);
  const u32x4_t x = ldg16(a.x + static_cast<size_t>(m) * a.N + 8 * c);
  stg16(a.y + static_cast<size_t>(m) * a.N + 8 * c, rms_norm_chunk(x, r, ldg16(a.gamma + 8 * c)));
}

}  // namespace

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(a.B) * (a.T1 + a.T2);
  const dim3 grid(static_cast<unsigned>((M + kMT - 1) / kMT), static_cast<unsigned>((a.N + kNT - 1) / kNT));
  hipLaunchKernelGGL(linear_bf16, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rms_apply_bf16(const RmsApplyArgs& a, hipStream_t s) {
  const int64_t n = a.M * (a.N / 8);
  hipLaunchKernelGGL(rms_apply_bf16, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
