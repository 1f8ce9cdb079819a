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
// Four launches (one ordered stream, no atomics, bitwise deterministic):
//  1. prep_q: D, lse in log2 units (+inf for dead or padded rows, so their p is
//     exactly 0), and transposed copies of q and dout.
//  2. prep_k: transposed copies of k_nope (per head) and k_rope (per row).
//  3. dkdv: one workgroup per (b, h, 128 keys); wave w owns 32 keys, keeps their
//     K and V operands in registers and dK (32 x 192) and dV (32 x 128) in
//     accumulators, and walks the 32-query chunks of every q-tile whose tiles
//     with these keys are not empty.  S = Q K^T and dP = dO V^T put one key per
//     lane, which is the A-operand layout of dV += P^T dO and dK += dS^T Q, so
//     P and dS go from accumulator to operand without moving; the other
//     operands (q and dout, reduction over queries) come from the transposed
//     copies with 16-byte LDS reads.  dk_rope is written per head (fp32).
//  4. dq: one workgroup per (b, q-tile, h) in the forward's ranked order; wave w
//     owns 32 queries, keeps Q and dO in registers and walks the tile list:
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, and dS^T is the
//     B operand of dQ^T += K^T dS^T, with K^T from the transposed copy.
//  5. rope_reduce: dk_rope = sum over heads of the per-head parts, in head order.
//
// Operand staging: dK/dV copies each 32-query chunk global -> LDS through the
// buffer unit (no staging registers) into a three-stage ring, two chunks ahead;
// dQ loads each 64-key tile into registers one tile ahead and stores it into the
// other half of a double buffer.  LDS rows are padded by 16 bytes so the 16-byte
// column reads of 16 lanes hit distinct banks.  Every staging load is issued
// unconditionally (past the end: an offset beyond the resource, zeros, no
// traffic) and the loads the compiler must wait for are issued before them, so
// no wait in the loops drains the copies in flight.  Masks: class-0 tiles are skipped, class-1 tiles need no
// mask work, class-2 tiles zero p for keys whose visibility bit is clear,
// class-3 tiles add the mask values; keys past Lk get p = 0.
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
constexpr int kSKT = kTileN * 2 + 16;           // 144: transposed k rows (64 keys)
// dQ stage: K, V, K^T
constexpr int kB_K = 0;
constexpr int kB_V = kB_K + kTileN * kSQ;
constexpr int kB_KT = kB_V + kTileN * kSO;
constexpr int kB_Stage = kB_KT + kDqk * kSKT;
static_assert(2 * kB_Stage <= 160 * 1024, "LDS budget");

// Position k of a 16-entry group holds entry relabel16(k): bits 2 and 3 swapped.
__device__ __forceinline__ int relabel16(int k) { return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Buffer resource over `bytes` bytes at p: loads at offsets >= bytes return zeros,
// which is how rows past the end of a tensor read as zero without a compare.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
// 16 bytes at voffset (per lane) + soffset (uniform)
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}

__device__ __forceinline__ bf16x8_t lds_frag(const char* p) { return as_bf16x8(*reinterpret_cast<const u32x4_t*>(p)); }

// 8 floats -> one bf16x8 operand (round to nearest even)
__device__ __forceinline__ bf16x8_t pack8(const float* x) {
  const u32x4_t w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
  return as_bf16x8(w);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

template <bool MASK_BF16>
__device__ __forceinline__ float mask_value(const void* mask, size_t idx) {
  if (MASK_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(mask)[idx]);
  return static_cast<const float*>(mask)[idx];
}

// ---------------------------------------------------------------- 1. prep_q
// grid (Lqp / 32, B*H): D, lse2 and the transposed q / dout of 32 queries.
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
      a.dd[bh * a.Lqp + qi] = acc;
      const float l = qi < a.Lq ? a.lse[bh * a.Lq + qi] : -INFINITY;
      a.lse2[bh * a.Lqp + qi] = l == -INFINITY ? INFINITY : l * kLog2e;
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

// ---------------------------------------------------------------- 4. dQ
template <bool MASK_BF16>
__global__ void __launch_bounds__(kThreads) bwd_dq(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kB_Stage];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 31, hi = lane >> 5;
  const int rank = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int row = a.order ? a.order[rank] : rank;      // b * nqt + qt
  const int b = row / a.nqt, qt = row % a.nqt;
  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int qi = qt * kTileM + 32 * w + li;            // this lane's query
  const bool q_ok = qi < a.Lq;

  bf16x8_t qreg[12], oreg[8];
#pragma unroll
  for (int s = 0; s < 12; ++s)
    qreg[s] = as_bf16x8(q_ok ? ldg16(a.q + (bh * a.Lq + qi) * kDqk + 16 * s + 8 * hi) : zero4());
#pragma unroll
  for (int s = 0; s < 8; ++s)
    oreg[s] = as_bf16x8(q_ok ? ldg16(a.dout + (bh * a.Lq + qi) * kDv + 16 * s + 8 * hi) : zero4());
  const float lse2 = a.lse2[bh * a.Lqp + qi];
  const float dd = a.dd[bh * a.Lqp + qi];

  f32x16_t dq[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) dq[i] = zero16();

  const int n = a.lists ? a.counts[row] : a.nkt;
  const int32_t* list = a.lists ? a.lists + static_cast<size_t>(row) * a.nkt : nullptr;
  auto entry = [&](int e) -> int { return list ? list[e] : (e | (1 << 24)); };

  // staging: per-lane byte offsets are fixed, the tile moves the uniform offset
  const __amdgpu_buffer_rsrc_t r_kn = rsrc(a.kn + bh * a.Lk * kDn, static_cast<size_t>(a.Lk) * kDn * 2);
  const __amdgpu_buffer_rsrc_t r_kr = rsrc(a.kr + static_cast<size_t>(b) * a.Lk * kDr, static_cast<size_t>(a.Lk) * kDr * 2);
  const __amdgpu_buffer_rsrc_t r_v = rsrc(a.v + bh * a.Lk * kDv, static_cast<size_t>(a.Lk) * kDv * 2);
  const __amdgpu_buffer_rsrc_t r_knt = rsrc(a.knT + bh * kDn * a.Lkp, static_cast<size_t>(kDn) * a.Lkp * 2);
  const __amdgpu_buffer_rsrc_t r_krt = rsrc(a.krT + static_cast<size_t>(b) * kDr * a.Lkp, static_cast<size_t>(kDr) * a.Lkp * 2);
  // chunk c of this thread's i-th load: K nope rows 64 x 16 (i < 4), K rope rows 64 x 8 (2),
  // V rows 64 x 16 (4), K^T nope rows 128 x 8 (4), K^T rope rows 64 x 8 (2)
  u32x4_t pre[16];
  // issued every step (past the last tile: an offset beyond every resource, zeros
  // and no traffic), so the compiler's wait counts for the loads around it are exact
  constexpr uint32_t kPastEnd = 0x80000000u;
  auto prefetch = [&](int kt, bool live) {
    const uint32_t k0 = static_cast<uint32_t>(kt) * kTileN;
    const uint32_t so_kn = live ? k0 * (kDn * 2) : kPastEnd, so_kr = live ? k0 * (kDr * 2) : kPastEnd;
    const uint32_t so_v = live ? k0 * (kDv * 2) : kPastEnd, so_t = live ? k0 * 2 : kPastEnd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      pre[i] = bload16(r_kn, (ci >> 4) * (kDn * 2) + (ci & 15) * 16, so_kn);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + kThreads * i;
      pre[4 + i] = bload16(r_kr, (ci >> 3) * (kDr * 2) + (ci & 7) * 16, so_kr);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      pre[6 + i] = bload16(r_v, (ci >> 4) * (kDv * 2) + (ci & 15) * 16, so_v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      pre[10 + i] = bload16(r_knt, (ci >> 3) * (a.Lkp * 2) + (ci & 7) * 16, so_t);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + kThreads * i;
      pre[14 + i] = bload16(r_krt, (ci >> 3) * (a.Lkp * 2) + (ci & 7) * 16, so_t);
    }
  };
  auto commit = [&](char* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      *reinterpret_cast<u32x4_t*>(st + kB_K + (ci >> 4) * kSQ + (ci & 15) * 16) = pre[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + kThreads * i;
      *reinterpret_cast<u32x4_t*>(st + kB_K + (ci >> 3) * kSQ + kDn * 2 + (ci & 7) * 16) = pre[4 + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      *reinterpret_cast<u32x4_t*>(st + kB_V + (ci >> 4) * kSO + (ci & 15) * 16) = pre[6 + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + kThreads * i;
      *reinterpret_cast<u32x4_t*>(st + kB_KT + (ci >> 3) * kSKT + (ci & 7) * 16) = pre[10 + i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = t + kThreads * i;
      *reinterpret_cast<u32x4_t*>(st + kB_KT + (kDn + (ci >> 3)) * kSKT + (ci & 7) * 16) = pre[14 + i];
    }
  };

  const float scale_log2 = a.scale * kLog2e;
  // visibility word of this lane's query in a class-2 tile (zero elsewhere): loaded
  // unconditionally through a resource, before the next tile's staging loads are
  // issued, so the wait for it is a count that leaves those in flight
  const __amdgpu_buffer_rsrc_t r_bits =
      rsrc(a.bits, a.bits ? static_cast<size_t>(a.B) * a.nqt * a.nkt * kTileM * 8 : 0);
  const uint32_t vo_bits = q_ok ? static_cast<uint32_t>(32 * w + li) * 8 : kPastEnd;
  auto vis_word = [&](int kt, int cls) -> uint64_t {
    const uint32_t so = cls == 2 ? static_cast<uint32_t>((static_cast<size_t>(row) * a.nkt + kt) * kTileM * 8) : kPastEnd;
    const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(r_bits, vo_bits, so, 0);
    return __builtin_bit_cast(uint64_t, v2);
  };
  auto compute = [&](const char* st, int kt, int cls, uint64_t word) {
    bf16x8_t bS[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16_t S = zero16(), dP = zero16();
#pragma unroll
      for (int s = 0; s < 12; ++s)
        S = mfma32(lds_frag(st + kB_K + (32 * half + li) * kSQ + (16 * s + 8 * hi) * 2), qreg[s], S);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        dP = mfma32(lds_frag(st + kB_V + (32 * half + li) * kSO + (16 * s + 8 * hi) * 2), oreg[s], dP);
      __builtin_amdgcn_sched_barrier(0);
      float madd[16];                                 // log2(e) * mask values (general tiles only)
#pragma unroll
      for (int r = 0; r < 16; ++r) madd[r] = 0.f;
      if (cls == 3 && a.mask) {
        for (int r = 0; r < 16; ++r) {
          const int kj = kt * kTileN + 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (kj < a.Lk && q_ok)
            madd[r] = mask_value<MASK_BF16>(a.mask, (static_cast<size_t>(b) * a.Lq + qi) * a.Lk + kj) * kLog2e;
        }
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);   // key within the tile
        bool vis = kt * kTileN + kl < a.Lk;
        if (cls == 2) vis = vis && ((word >> kl) & 1ull);
        const float pr = vis ? __builtin_amdgcn_exp2f(S[r] * scale_log2 - lse2 + madd[r]) : 0.f;
        ds[r] = pr * (dP[r] - dd);
      }
      bS[2 * half] = pack8(ds);
      bS[2 * half + 1] = pack8(ds + 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < 6; ++mt) {
      const char* rowp = st + kB_KT + (32 * mt + li) * kSKT + 16 * hi;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) dq[mt] = mfma32(lds_frag(rowp + 32 * kk), bS[kk], dq[mt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (n > 0) {
    int e0 = entry(0);
    prefetch(e0 & 0xFFFFFF, true);
    commit(smem);
    __syncthreads();
    for (int e = 0; e < n; ++e) {
      const bool more = e + 1 < n;
      const uint64_t word = vis_word(e0 & 0xFFFFFF, e0 >> 24);
      const int e1 = more ? entry(e + 1) : 0;
      prefetch(e1 & 0xFFFFFF, more);
      compute(smem + (e & 1) * kB_Stage, e0 & 0xFFFFFF, e0 >> 24, word);
      if (!more) break;
      commit(smem + ((e + 1) & 1) * kB_Stage);
      __syncthreads();
      e0 = e1;
    }
  }

  // accumulator row r <-> dim 32*mt + 8*(r/4) + 4*hi + r%4, column <-> this lane's query
  if (q_ok) {
    uint16_t* op = a.dq + (bh * a.Lq + qi) * kDqk;
#pragma unroll
    for (int mt = 0; mt < 6; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t w2 = {pack_bf16x2(dq[mt][4 * g] * a.scale, dq[mt][4 * g + 1] * a.scale),
                            pack_bf16x2(dq[mt][4 * g + 2] * a.scale, dq[mt][4 * g + 3] * a.scale)};
        *reinterpret_cast<u32x2_t*>(op + 32 * mt + 8 * g + 4 * hi) = w2;
      }
  }
}

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
  const dim3 gq(static_cast<unsigned>(a.B) * a.nqt * a.H);
  if (a.mask && a.mask_bf16) hipLaunchKernelGGL(bwd_dq<true>, gq, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(bwd_dq<false>, gq, dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n4 = static_cast<int64_t>(a.B) * a.Lk * (kDr / 4);
  hipLaunchKernelGGL(bwd_rope_reduce, dim3(static_cast<unsigned>((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
