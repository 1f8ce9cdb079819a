// kv_b_proj latent expansion (NeMo AutoModel DFlash page, KimiK3DFlashAttention
// class text: kv_b_proj emits one qk_nope_head_dim + v_head_dim slice per query
// head; Kimi K3 model page, MLA context-parallel forward: the latent is expanded
// locally into per-head keys and values).
//
//   kv[m, n] = sum_r latent[m, r] * W[n, r]      m = b*Lk + t,  n = h*256 + e
//   e < 128 -> k_nope[b,h,t,e];   e >= 128 -> v[b,h,t,e-128]
//
// Both operands are r-contiguous, which is exactly what the MFMA operands
// want (8 consecutive r per lane).  The kernel computes the transposed tile
// C^T = W . latent^T so that a lane owns one token and 4-long runs of
// consecutive e, which become 8-byte stores into the [B,H,Lk,128] outputs; a
// 128-wide n tile is exactly one head's k_nope or v slice, so the scatter is
// free.
#include "common.h"
#include "launch.h"
#include "rmsnorm.h"

namespace dflash {
namespace {

constexpr int kEM = 128;            // e rows per tile (one slice of one head)
constexpr int kTM = 128;            // tokens per tile
constexpr int kRK = 32;             // r per LDS stage
constexpr int kRowStride = kRK + 8; // bf16 per LDS row (80 B: conflict-free b128 reads)
constexpr int kStage = (kEM + kTM) * kRowStride;

__global__ void __launch_bounds__(256) expand_bf16(ExpandArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int we = wave & 1, wt = wave >> 1;
  const int li = lane & 31, hi = lane >> 5;
  const int nt = blockIdx.y;                 // (head, slice)
  const int h = nt >> 1, part = nt & 1;
  const int64_t M = static_cast<int64_t>(a.B) * a.Lk;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kTM;
  const uint16_t* W = static_cast<const uint16_t*>(a.w) + (static_cast<size_t>(h) * 256 + part * 128) * a.R;
  const uint16_t* L = static_cast<const uint16_t*>(a.latent);

  // optional RMSNorm of the latent rows (kv_a_layernorm) applied as they are staged
  float rsc[2] = {1.f, 1.f};
  if (a.stats) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m0 + ((t + 256 * i) >> 2);
      if (m < M) rsc[i] = rms_row_scale(a.stats, a.stats_parts, m, a.R, a.eps);
    }
  }
  u32x4_t sw[2], sl[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + 256 * i, row = ci >> 2, c = ci & 3;
      sw[i] = ldg16(W + static_cast<size_t>(row) * a.R + k0 + c * 8);
      const int64_t m = m0 + row;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      sl[i] = m < M ? ldg16(L + static_cast<size_t>(m) * a.R + k0 + c * 8) : z;
      if (a.stats && m < M) sl[i] = rms_norm_chunk(sl[i], rsc[i], ldg16(a.gamma + k0 + c * 8));
    }
  };
  auto store = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + 256 * i, row = ci >> 2, c = ci & 3;
      stg16(buf + row * kRowStride + c * 8, sw[i]);
      stg16(buf + (kEM + row) * kRowStride + c * 8, sl[i]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.R / kRK;
  load(0);
  store(smem);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const bool more = it + 1 < nk;
    if (more) load((it + 1) * kRK);
    const uint16_t* Ws = smem + (it & 1) * kStage;
    const uint16_t* Ls = Ws + kEM * kRowStride;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ws + (64 * we + 32 * i + li) * kRowStride + 16 * ks + 8 * hi));
        bf[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ls + (64 * wt + 32 * i + li) * kRowStride + 16 * ks + 8 * hi));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (more) store(smem + ((it + 1) & 1) * kStage);
    __syncthreads();
  }

  uint16_t* dst = static_cast<uint16_t*>(part ? a.v : a.kn);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + 64 * wt + 32 * j + li;
    if (m >= M) continue;
    const int64_t b = m / a.Lk, tok = m % a.Lk;
    uint16_t* row = dst + ((static_cast<size_t>(b) * a.H + h) * a.Lk + tok) * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = 64 * we + 32 * i + 8 * g + 4 * hi;
        u32x2_t w2 = {pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                      pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        *reinterpret_cast<u32x2_t*>(row + e0) = w2;
      }
  }
}

// fp32: plain LDS-tiled FMA GEMM (64 tokens x 64 outputs per workgroup).
__global__ void __launch_bounds__(256) expand_f32(ExpandArgs a) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t M = static_cast<int64_t>(a.B) * a.Lk;
  const int N = a.H * 256;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int n0 = blockIdx.y * 64;
  const float* L = static_cast<const float*>(a.latent);
  const float* W = static_cast<const float*>(a.w);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.R; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int r = e >> 4, k = e & 15;
      const int64_t m = m0 + r;
      As[k][r] = (m < M) ? L[static_cast<size_t>(m) * a.R + k0 + k] : 0.f;
      const int n = n0 + r;
      Bs[k][r] = (n < N) ? W[static_cast<size_t>(n) * a.R + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(As[k][ty + 16 * i], Bs[k][tx + 16 * j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= M) continue;
    const int64_t b = m / a.Lk, tok = m % a.Lk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= N) continue;
      const int h = n >> 8, e = n & 255;
      float* dst = static_cast<float*>(e < 128 ? a.kn : a.v);
      dst[((static_cast<size_t>(b) * a.H + h) * a.Lk + tok) * 128 + (e & 127)] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_expand_bf16(const ExpandArgs& a, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(a.B) * a.Lk;
  dim3 grid(static_cast<unsigned>((M + kTM - 1) / kTM), 2 * a.H);
  hipLaunchKernelGGL(expand_bf16, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(a.B) * a.Lk;
  dim3 grid(static_cast<unsigned>((M + 63) / 64), (a.H * 256 + 63) / 64);
  hipLaunchKernelGGL(expand_f32, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
