// kv_b_proj latent expansion, fp32 path (NeMo AutoModel DFlash page,
// KimiK3DFlashAttention class text: kv_b_proj emits one qk_nope_head_dim +
// v_head_dim slice per query head; Kimi K3 model page, MLA context-parallel
// forward: the latent is expanded locally into per-head keys and values).
//
//   kv[m, n] = sum_r latent[m, r] * W[n, r]      m = b*Lk + t,  n = h*256 + e
//   e < 128 -> k_nope[b,h,t,e];   e >= 128 -> v[b,h,t,e-128]
//
// The bf16 expansion runs on the MFMA linear kernel (linear.hip, per-head
// k_nope / v output mode); this file keeps the plain fp32 FMA version.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

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

hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(a.B) * a.Lk;
  dim3 grid(static_cast<unsigned>((M + 63) / 64), (a.H * 256 + 63) / 64);
  hipLaunchKernelGGL(expand_f32, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
