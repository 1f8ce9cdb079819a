// Backward of the fused draft MLA attention, bf16 MFMA on gfx950.
//
// The draft is trained (NeMo AutoModel DFlash page, KimiK3DFlashDraftModel: the
// DFlash trainer drives it; DSpark page, module text: speculative-decoding
// training), so the attention of the forward kernel needs its gradients.  With
// p = exp(s - lse) recomputed from the saved per-row normaliser lse,
//   dp = dout . v_j,  D = rowsum(dout * out),  ds = p * (dp - D)
//   dv_j = sum_i p_ij dout_i          dk_j = scale * sum_i ds_ij q_i
//   dq_i = scale * sum_j ds_ij k_j    dk_rope_j = sum over heads of dk_j[Dn:]
// and the score matrix is never stored: both passes recompute their tile of p.
//
// The launches, on one ordered stream (no atomics: bitwise deterministic):
//  1. prep_q: per 32-query chunk the exponent offsets -lse log2(e) (-inf for
//     dead or padded rows, so their p is exactly 0) and -D, and transposed
//     copies of q and dout.
//  2. prep_k: transposed copies of k_nope (per head) and k_rope (per row).
//  3. prep_bits (bwd_dkdv.hip): the visibility words of the masked (class-2)
//     tiles transposed to one word per key.
//  4. dkdv (bwd_dkdv.hip): dK, dV and the per-head k_rope parts, one workgroup
//     per (b, h, 128 keys).
//  5. dq (bwd_dq.hip): one workgroup per (b, q-tile, h) in the forward's ranked
//     order.
//  6. rope_reduce: dk_rope = sum over heads of the per-head parts, in head order.
// The transposed copies hold, per 16-entry group, entry 16g + k at position
// 16g + k with bits 2 and 3 of k swapped: the order in which the rows of an
// MFMA accumulator become the reduction index of the next product.
#include "common.h"
#include "dma.h"
#include "launch.h"

#include <type_traits>

namespace dflash {
namespace {

template <int N>
using IC = std::integral_constant<int, N>;

constexpr int kThreads = 256;
constexpr int kQC = 32;                         // queries per prep_q workgroup
// LDS row strides (bytes): row + 16, so 16-lane column reads hit distinct banks
constexpr int kSQ = kDqk * 2 + 16;              // 400: q / k rows
constexpr int kSO = kDv * 2 + 16;               // 272: dout / v rows

// Position k of a 16-entry group holds entry relabel16(k): bits 2 and 3 swapped.
__device__ __forceinline__ int relabel16(int k) { return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------- 1. prep_q
// grid (Lqp / 32, B*H): the exponent offsets and -D of 32 queries, and their transposed q / dout.
__global__ void __launch_bounds__(kThreads) bwd_prep_q(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) char sq[kQC * kSQ];
  __shared__ __attribute__((aligned(16))) char so[kQC * kSO];
  const int t = threadIdx.x;
  const int q0 = blockIdx.x * kQC;
  const size_t bh = blockIdx.y;
  for (int i = t; i < kQC * 24; i += kThreads) {
    const int r = i / 24, c = i % 24, qi = q0 + r;
    *reinterpret_cast<u32x4_t*>(sq + r * kSQ + c * 16) =
        qi < a.Lq ? ldg16(a.q + (bh * a.Lq + qi) * kDqk + c * 8) : zero4();
  }
  for (int i = t; i < kQC * 16; i += kThreads) {
    const int r = i / 16, c = i % 16, qi = q0 + r;
    *reinterpret_cast<u32x4_t*>(so + r * kSO + c * 16) =
        qi < a.Lq ? ldg16(a.dout + (bh * a.Lq + qi) * kDv + c * 8) : zero4();
  }
  {  // D: 8 lanes per row, 16 dims each
    const int r = t >> 3, part = t & 7, qi = q0 + r;
    float acc = 0.f;
    if (qi < a.Lq) {
      const uint16_t* op = a.out + (bh * a.Lq + qi) * kDv + part * 16;
      const uint16_t* gp = a.dout + (bh * a.Lq + qi) * kDv + part * 16;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4_t o = ldg16(op + 8 * h2), g = ldg16(gp + 8 * h2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc += bf16_bits_to_f32(o[j] & 0xFFFFu) * bf16_bits_to_f32(g[j] & 0xFFFFu);
          acc += bf16_bits_to_f32(o[j] >> 16) * bf16_bits_to_f32(g[j] >> 16);
        }
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (part == 0) {
      const float l = qi < a.Lq ? a.lse[bh * a.Lq + qi] : -INFINITY;
      // per 32-query chunk: the exponent offsets, then -D
      float* ld = a.ld + (bh * (a.Lqp / kQC) + blockIdx.x) * 64;
      ld[r] = l == -INFINITY ? -INFINITY : -l * kLog2e;
      ld[kQC + r] = -acc;
    }
  }
  __syncthreads();
  const uint16_t* sq16 = reinterpret_cast<const uint16_t*>(sq);
  const uint16_t* so16 = reinterpret_cast<const uint16_t*>(so);
  // transposed rows: 4 chunks of 8 positions per 32-query row
  for (int i = t; i < (kDqk + kDv) * 4; i += kThreads) {
    const int d = i >> 2, g = i & 3;
    const bool isq = d < kDqk;
    const int dd = isq ? d : d - kDqk;
    const uint16_t* src = isq ? sq16 : so16;
    const int stride = (isq ? kSQ : kSO) / 2;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 8; p += 2) {
      const int k0 = 8 * g + p, k1 = k0 + 1;
      const int r0 = (k0 & 16) | relabel16(k0 & 15), r1 = (k1 & 16) | relabel16(k1 & 15);
      w[p >> 1] = static_cast<uint32_t>(src[r0 * stride + dd]) | (static_cast<uint32_t>(src[r1 * stride + dd]) << 16);
    }
    uint16_t* dst = isq ? a.qT + (bh * kDqk + dd) * a.Lqp : a.doT + (bh * kDv + dd) * a.Lqp;
    stg16(dst + q0 + 8 * g, u32x4_t{w[0], w[1], w[2], w[3]});
  }
}

// ---------------------------------------------------------------- 2. prep_k
// grid (Lkp / 64, B*H): transposed k_nope of 64 keys; the h == 0 workgroups also
// transpose the batch row's k_rope.
__global__ void __launch_bounds__(kThreads) bwd_prep_k(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[kTileN * (kDn + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sr[kTileN * (kDr + 8)];
  const int t = threadIdx.x;
  const int k0 = blockIdx.x * kTileN;
  const size_t bh = blockIdx.y;
  const int b = static_cast<int>(bh / a.H), h = static_cast<int>(bh % a.H);
  const bool rope = h == 0;
  for (int i = t; i < kTileN * 16; i += kThreads) {
    const int r = i >> 4, c = i & 15, kj = k0 + r;
    *reinterpret_cast<u32x4_t*>(sk + r * (kDn + 8) + c * 8) =
        kj < a.Lk ? ldg16(a.kn + (bh * a.Lk + kj) * kDn + c * 8) : zero4();
  }
  if (rope) {
    for (int i = t; i < kTileN * 8; i += kThreads) {
      const int r = i >> 3, c = i & 7, kj = k0 + r;
      *reinterpret_cast<u32x4_t*>(sr + r * (kDr + 8) + c * 8) =
          kj < a.Lk ? ldg16(a.kr + (static_cast<size_t>(b) * a.Lk + kj) * kDr + c * 8) : zero4();
    }
  }
  __syncthreads();
  const int rows = rope ? kDn + kDr : kDn;
  for (int i = t; i < rows * 8; i += kThreads) {
    const int d = i >> 3, g = i & 7;
    const bool isn = d < kDn;
    const int dd = isn ? d : d - kDn;
    const uint16_t* src = isn ? sk : sr;
    const int stride = isn ? kDn + 8 : kDr + 8;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 8; p += 2) {
      const int j0 = 8 * g + p, j1 = j0 + 1;
      const int r0 = (j0 & 48) | relabel16(j0 & 15), r1 = (j1 & 48) | relabel16(j1 & 15);
      w[p >> 1] = static_cast<uint32_t>(src[r0 * stride + dd]) | (static_cast<uint32_t>(src[r1 * stride + dd]) << 16);
    }
    uint16_t* dst = isn ? a.knT + (bh * kDn + dd) * a.Lkp : a.krT + (static_cast<size_t>(b) * kDr + dd) * a.Lkp;
    stg16(dst + k0 + 8 * g, u32x4_t{w[0], w[1], w[2], w[3]});
  }
}

// ---------------------------------------------------------------- 3. dK / dV: bwd_dkdv.hip

// ---------------------------------------------------------------- 4. dQ: bwd_dq.hip

// ---------------------------------------------------------------- 5. dk_rope
// One thread per 4 consecutive dims of one (b, key): sum over heads in order.
__global__ void __launch_bounds__(kThreads) bwd_rope_reduce(AttnBwdArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.B) * a.Lk * (kDr / 4);
  if (i >= total) return;
  const int d4 = static_cast<int>(i % (kDr / 4));
  const int64_t bk = i / (kDr / 4);
  const int b = static_cast<int>(bk / a.Lk), kj = static_cast<int>(bk % a.Lk);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < a.H; ++h) {
    const size_t row = (static_cast<size_t>(b) * a.H + h) * a.Lk + kj;
    acc += *reinterpret_cast<const f32x4_t*>(a.rope_part + row * kDr + 4 * d4);
  }
  const u32x2_t w2 = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2_t*>(a.dkr + (static_cast<size_t>(b) * a.Lk + kj) * kDr + 4 * d4) = w2;
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t s) {
  const unsigned bh = static_cast<unsigned>(a.B) * a.H;
  hipLaunchKernelGGL(bwd_prep_q, dim3(a.Lqp / kQC, bh), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_prep_k, dim3(a.Lkp / kTileN, bh), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_bwd_dkdv(a, s)) != hipSuccess) return e;
  if ((e = launch_bwd_dq(a, s)) != hipSuccess) return e;
  const int64_t n4 = static_cast<int64_t>(a.B) * a.Lk * (kDr / 4);
  hipLaunchKernelGGL(bwd_rope_reduce, dim3(static_cast<unsigned>((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
