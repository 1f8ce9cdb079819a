// dQ of the draft MLA attention (backward), bf16 MFMA on gfx950.
//
// With p = exp(s - lse) recomputed from the forward's row normaliser and
// ds = p (dout . v_j - D), D = rowsum(dout * out) (the softmax backward of the
// attention the DFlash trainer differentiates: NeMo AutoModel DFlash page,
// KimiK3DFlashDraftModel; DSpark page, speculative-decoding training):
//   dq_i = scale * sum_j ds_ij [k_nope_j | k_rope_j].
//
// One workgroup per (b, q-tile of 128 queries, h) in the forward's ranked order;
// wave w owns 32 queries: their q and dout operands stay in accumulator
// registers, dQ^T (192 x 32) accumulates in accumulator registers.  The
// workgroup walks the 32-key steps of its q-tile's tile list (copied to LDS at
// the start).  S^T = K Q^T and dP^T = V dO^T put one query per lane, so the row
// values (lse, D) are one register each and dS^T is directly the B operand of
// dQ^T += K^T dS^T, with K^T from the transposed copy.
//
// Step j is one block of 32 MFMA slots scheduled by hand (one MFMA, its operand
// reads issued about eight slots ahead, a share of the vector work and copies):
//   slots 0-11  S^T(j+1)      vector: dS(j) = P(j) (dP(j) - D), packed; the
//   slots 12-19 dP^T(j+1) - D         exponent offsets of step j+1
//   slots 20-31 dQ(j)         vector: P(j+1) = exp2(S(j+1) scale log2(e) + offset)
// (a tile with general mask values takes its offsets between slots 13 and 14).
// The matrix work of a slot and its vector work belong to different steps.
// Staging: the F part of step m (K and V rows, the tile's visibility words) is
// copied global -> LDS in step m - 4, the T part (transposed K) in step m - 2.
#include <type_traits>
#include <utility>

#include "common.h"
#include "dma.h"
#include "launch.h"
#include "bwd_plan.h"

namespace dflash {
namespace {

template <int N>
using IC = std::integral_constant<int, N>;
template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(IC<Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
typedef __attribute__((address_space(3))) int lds_int_t;

constexpr int kThreads = 256;
constexpr int kListMax = 2048;                      // tile-list entries per window
constexpr int kFRing = 0;
constexpr int kTRing = kFRing + kQFSlots * kQF_Slot;
constexpr int kList = kTRing + kQTSlots * kQT_Slot;
constexpr int kLdsBytes = kList + kListMax * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr uint32_t kNegInfBits = 0xFF800000u;

// A wave's barrier with the workgroup, without the LDS fence of __syncthreads:
// operand reads still in flight target slots that are rewritten only after a
// later barrier, and the copies are waited for explicitly before it.
__device__ __forceinline__ void step_barrier() { asm volatile("s_barrier" ::: "memory"); }

// MFMA forms as asm, so the register file of every operand is fixed: S^T and
// dP^T accumulate in vector registers (the vector unit reads them), their B
// operand (the wave's q or dout) in accumulator registers; dQ^T accumulates in
// accumulator registers.  The compiler does not see their latencies: the
// vector readers of S^T come two MFMA issues after its last MFMA, dP^T is read
// in the next step.
template <bool FIRST>
__device__ __forceinline__ void mfma_s(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  if (FIRST) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
template <bool FIRST>
__device__ __forceinline__ void mfma_dp(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  if (FIRST) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(a), "a"(b), "v"(c));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <bool MASK_BF16>
__device__ __forceinline__ float mask_value(const void* mask, size_t idx) {
  if (MASK_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(mask)[idx]);
  return static_cast<const float*>(mask)[idx];
}

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

template <bool MASK_BF16>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dq(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  lds_char_t* const lds = (lds_char_t*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 31, hi = lane >> 5;
  const int rank = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int row = a.order ? a.order[rank] : rank;      // b * nqt + qt
  const int b = row / a.nqt, qt = row % a.nqt;
  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int ql = 32 * w + li;                          // this lane's query in the q-tile
  const int qi = qt * kTileM + ql;
  const bool q_ok = qi < a.Lq;

  // ---- this lane's q and dout operands (B operands of S^T and dP^T: query li,
  // dims 16s + 8hi .. +8), its row values, and the q-tile's tile count
  u32x4_t qf[kDqk / 16], of[kDv / 16];
  u32x4_t qv[kDqk / 16], ov[kDv / 16];
#pragma unroll
  for (int s = 0; s < kDqk / 16; ++s) qv[s] = q_ok ? ldg16(a.q + (bh * a.Lq + qi) * kDqk + 16 * s + 8 * hi) : zero4();
#pragma unroll
  for (int s = 0; s < kDv / 16; ++s) ov[s] = q_ok ? ldg16(a.dout + (bh * a.Lq + qi) * kDv + 16 * s + 8 * hi) : zero4();
  const float* ldrow = a.ld + (bh * (a.Lqp / kQC) + (qt * kTileM + 32 * w) / kQC) * 64;
  const float nlse = ldrow[li];                        // -lse log2(e), -inf for dead or padded rows
  const float ndd = ldrow[kQC + li];                   // -D
  const float lse_nat = q_ok ? a.lse[bh * a.Lq + qi] : -INFINITY;
  const int n_all = a.lists ? a.counts[row] : a.nkt;
  const int32_t* glist = a.lists ? a.lists + static_cast<size_t>(row) * a.nkt : nullptr;

  f32x16_t dq[kDqk / 32];
#pragma unroll
  for (int i = 0; i < kDqk / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;
  f32x16_t nd;                                         // C operand of dP^T: -D in every row
#pragma unroll
  for (int r = 0; r < 16; ++r) nd[r] = ndd;

  // ---- copy plan (bwd_plan.h): per-lane source offsets fixed for the kernel
  const u32x4_t d_kn = buffer_desc(a.kn + bh * a.Lk * kDn, static_cast<uint32_t>(a.Lk) * kDn * 2);
  const u32x4_t d_kr = buffer_desc(a.kr + static_cast<size_t>(b) * a.Lk * kDr, static_cast<uint32_t>(a.Lk) * kDr * 2);
  const u32x4_t d_v = buffer_desc(a.v + bh * a.Lk * kDv, static_cast<uint32_t>(a.Lk) * kDv * 2);
  const u32x4_t d_bits = buffer_desc(a.bits ? a.bits + static_cast<size_t>(row) * a.nkt * kTileM : nullptr,
                                     a.bits ? static_cast<uint32_t>(a.nkt) * 1024u : 0u);
  const u32x4_t d_ktn = buffer_desc(a.knT + bh * kDn * a.Lkp, static_cast<uint32_t>(kDn) * a.Lkp * 2);
  const u32x4_t d_ktr = buffer_desc(a.krT + static_cast<size_t>(b) * kDr * a.Lkp, static_cast<uint32_t>(kDr) * a.Lkp * 2);
  uint32_t vo[kQCopiesPerStep];
#pragma unroll
  for (int j = 0; j < kQCopiesPerStep; ++j) vo[j] = q_voff(w, j, lane, a.Lkp);
  // copy j of this wave for the step with tile entry e and half hf, into the slot at LDS byte slot_base
  auto copy = [&](auto J, uint32_t slot_base, int e, int hf) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int reg = q_src_region(j);
    const bool live = (e >> 24) != 0;
    const uint32_t kt = static_cast<uint32_t>(e & 0xFFFFFF);
    const uint32_t key0 = kt * kTileN + 32u * static_cast<uint32_t>(hf);
    const uint32_t so = !live ? kPastEnd
                      : reg == kSrcKN || reg == kSrcV ? key0 * 256u : reg == kSrcKR ? key0 * 128u
                      : reg == kSrcBits ? kt * 1024u : key0 * 2u;
    const u32x4_t d = reg == kSrcKN ? d_kn : reg == kSrcKR ? d_kr : reg == kSrcV ? d_v : reg == kSrcBits ? d_bits
                    : reg == kSrcKTN ? d_ktn : d_ktr;
    dma16s(d, slot_base, static_cast<uint32_t>(q_dst_base(w, j)), vo[j], so);
  };

  // ---- per-lane LDS read offsets inside a slot (bwd_plan.h); chunk s of K at
  // k_lane[s&1] (k_nope, s < 8) or kr_lane[s&1] (k_rope) + (s/2 mod 4) KiB
  const int k_lane0 = rd_k(0, li, hi), k_lane1 = rd_k(1, li, hi);
  const int kr_lane0 = rd_k(kDn / 16, li, hi), kr_lane1 = rd_k(kDn / 16 + 1, li, hi);
  const int v_lane0 = rd_v(0, li, hi), v_lane1 = rd_v(1, li, hi);
  const int kt_lane0 = rd_kt(0, 0, li, hi), kt_lane1 = rd_kt(0, 1, li, hi);
  const int w_lane = rd_qword(ql);
  auto k_off = [&](int s) __attribute__((always_inline)) -> int {
    return s < kDn / 16 ? ((s & 1) ? k_lane1 : k_lane0) + (s >> 1) * 1024
                        : ((s & 1) ? kr_lane1 : kr_lane0) + ((s - kDn / 16) >> 1) * 1024;
  };
  auto kt_off = [&](int m) __attribute__((always_inline)) -> int {   // m = 2 mt + kk
    const int mt = m >> 1;
    return ((m & 1) ? kt_lane1 : kt_lane0) + (mt < kDn / 32 ? mt * 2048 : (kQ_KTR - kQ_KTN) + (mt - kDn / 32) * 2048);
  };
  int one;                                             // bit-field width 1 from an opaque register
  asm("s_mov_b32 %0, 1" : "=s"(one));
  const float c_log2 = a.scale * kLog2e;

  lds_int_t* const list = (lds_int_t*)(lds + kList);
  // ---- the window of the tile list from tile index tb: entries k-tile | class << 24
  auto load_list = [&](int tb) -> int {
    const int n = min(kListMax, n_all - tb);
    for (int i = t; i < n; i += kThreads) list[i] = glist ? glist[tb + i] : ((tb + i) | (1 << 24));
    __syncthreads();
    return n;
  };
  int nent = load_list(0);
#pragma unroll
  for (int s = 0; s < kDqk / 16; ++s) asm volatile("" : "=a"(qf[s]) : "0"(qv[s]));
#pragma unroll
  for (int s = 0; s < kDv / 16; ++s) asm volatile("" : "=a"(of[s]) : "0"(ov[s]));
  // the row values have landed before any copy is issued: the compiler cannot
  // count the copies, so a wait of its own for them later would drain those too
  asm volatile("" :: "v"(nlse), "v"(ndd), "v"(lse_nat));

  for (int tb = 0; tb < n_all; tb += kListMax, nent = tb < n_all ? load_list(tb) : 0) {
    const int nsteps = 2 * nent;
    if (nsteps == 0) continue;
    // entry of step m (0 past the end: no copy, class 0)
    auto ent = [&](int m) __attribute__((always_inline)) -> int {
      const int v = list[min(m, nsteps - 1) >> 1];
      return __builtin_amdgcn_readfirstlane(m < nsteps ? v : 0);
    };
    auto f_slot = [&](int m) __attribute__((always_inline)) -> int { return kFRing + (m % kQFSlots) * kQF_Slot; };
    auto t_slot = [&](int m) __attribute__((always_inline)) -> int { return kTRing + (m % kQTSlots) * kQT_Slot; };
    auto copy_f = [&](int m, int e) __attribute__((always_inline)) {
      const uint32_t base = lds0 + f_slot(m);
      static_for<6>([&](auto J) __attribute__((always_inline)) { copy(J, base, e, m & 1); });
    };
    auto copy_t = [&](int m, int e) __attribute__((always_inline)) {
      const uint32_t base = lds0 + t_slot(m);
      static_for<3>([&](auto J) __attribute__((always_inline)) { copy(IC<6 + decltype(J)::value>{}, base, e, m & 1); });
    };
    // visible keys of step m (entry e): bit i <-> key i of the step, shifted for
    // the lane half (accumulator row r <-> key 8(r/4) + 4hi + r%4)
    auto vis_bits = [&](int e, int m, uint64_t word) __attribute__((always_inline)) -> int {
      const int cls = e >> 24;
      const int key0 = (e & 0xFFFFFF) * kTileN + 32 * (m & 1);
      const int nvalid = a.Lk - key0;
      const uint32_t range = nvalid >= 32 ? ~0u : nvalid <= 0 ? 0u : (1u << nvalid) - 1u;
      const uint32_t w32 = static_cast<uint32_t>((m & 1) ? (word >> 32) : word);
      const uint32_t vm = cls == 0 ? 0u : cls == 2 ? (w32 & range) : range;
      return static_cast<int>(vm >> (4 * hi));
    };
    auto offset_entry = [&](int r, int hv) __attribute__((always_inline)) -> float {
      const int vis = __builtin_amdgcn_sbfe(hv, 8 * (r >> 2) + (r & 3), one);
      return __int_as_float((vis & __float_as_int(nlse)) | (~vis & static_cast<int>(kNegInfBits)));
    };
    // general mask values: offsets (m - lse) log2(e) in natural units first (m and
    // lse may both be near -FLT_MAX), -inf for keys past Lk or a dead row
    auto general_offsets = [&](int e, int m, float* adn) __attribute__((always_inline)) {
      const int key0 = (e & 0xFFFFFF) * kTileN + 32 * (m & 1);
      float mv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        mv[r] = q_ok && kj < a.Lk ? mask_value<MASK_BF16>(a.mask, (static_cast<size_t>(b) * a.Lq + qi) * a.Lk + kj)
                                  : -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) adn[r] = lse_nat == -INFINITY ? -INFINITY : (mv[r] - lse_nat) * kLog2e;
    };

    // ---- prologue: F(0..3), T(0), T(1) copied; S^T(0), dP^T(0), P(0); K operands
    // of step 1's first eight score MFMAs read
    int e1 = ent(1), e2 = ent(2), e3 = ent(3), e4 = ent(4);
    {
      const int e0 = ent(0);
      copy_f(0, e0);
      copy_f(1, e1);
      copy_t(0, e0);
      copy_f(2, e2);
      copy_t(1, e1);
      copy_f(3, e3);
    }
    wait_vmem<2 * kQCopiesPerStep>();                  // F(0), F(1) landed; T(0), F(2), T(1), F(3) in flight
    __syncthreads();

    f32x16_t acc;                                      // S^T of the next step
    float p[16];                                       // P of the current step (fp32)
    f32x16_t dpp;                                      // dP - D of the current step
    u32x4_t pkS[2];                                    // dS^T operand (bf16 pairs)
    float adn[16];                                     // exponent offsets of the next step
    u32x4_t fk[12], fv[8], ft[12];                     // operand fragments read ahead

    {
      const int e0 = ent(0);
      const lds_char_t* const fs = lds + f_slot(0);
      const uint64_t word = *(const lds_u64_t*)(fs + w_lane);
      const int hv = vis_bits(e0, 0, word);
#pragma unroll
      for (int r = 0; r < 16; ++r) adn[r] = offset_entry(r, hv);
      if (a.mask && (e0 >> 24) == 3) general_offsets(e0, 0, adn);
      static_for<12>([&](auto S) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        fk[s] = *(const lds_u32x4_t*)(fs + k_off(s));
        mfma_s<s == 0>(acc, fk[s], qf[s]);
      });
      static_for<8>([&](auto S) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        fv[s] = *(const lds_u32x4_t*)(fs + ((s & 1) ? v_lane1 : v_lane0) + (s >> 1) * 1024);
        mfma_dp<s == 0>(dpp, fv[s], of[s], nd);
      });
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc), "+v"(dpp));
#pragma unroll
      for (int u = 0; u < 16; ++u) p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[u], c_log2, adn[u]));
      const lds_char_t* const f1 = lds + f_slot(1);
#pragma unroll
      for (int s = 0; s < 8; ++s) fk[s] = *(const lds_u32x4_t*)(f1 + k_off(s));
    }
    wait_vmem<kQCopiesPerStep>();                      // T(0), F(2) landed (read in step 0)
    __syncthreads();                                   // F(0)'s slot is rewritten in step 0

    // Step j.  Entering: p = P(j), dpp = dP(j) - D, fk[0..7] = K operands 0-7 of
    // S^T(j+1).  e1 .. e4: entries of steps j+1 .. j+4.
    // ring slot offsets of steps j .. j+3 (F, 4 slots) and j .. j+2 (T, 3 slots),
    // rotated once per step instead of recomputed modulo the ring sizes
    int fs0 = f_slot(0), fs1 = f_slot(1), fs2 = f_slot(2), fs3 = f_slot(3);
    int ts0 = t_slot(0), ts1 = t_slot(1), ts2 = t_slot(2);
    for (int j = 0; j < nsteps; ++j) {
      const lds_char_t* const f1 = lds + fs1;                           // F(j+1)
      const lds_char_t* const f2 = lds + fs2;                           // F(j+2): next step's first K operands
      const lds_char_t* const t0 = lds + ts0;                           // T(j)
      const uint32_t fdst = lds0 + fs0;                                 // F(j+4) (slot of F(j)) <- copies
      const uint32_t tdst = lds0 + ts2;                                 // T(j+2) <- copies
      int e5v = 0;
      uint64_t word = 0;
      int hv = 0;

      // ---- slots 0-13: S^T(j+1), dP^T(j+1) begins; dS(j); offsets of step j+1
      // Every operand is read 8 slots ahead of its MFMA, one read per slot (slot
      // 0 also reads the visibility word and a list entry).  One wait per 4
      // slots, for the 4 operands read 8 to 5 slots back, replaces a wait in
      // front of every MFMA.
      static_for<14>([&](auto K) __attribute__((always_inline)) {
        constexpr int k = decltype(K)::value;
        if constexpr (k % 4 == 0) wait_lgkm<k == 4 ? 6 : 4>();
        if constexpr (k < 4) fk[8 + k] = *(const lds_u32x4_t*)(f1 + k_off(8 + k));
        if constexpr (k >= 4 && k < 12) fv[k - 4] = *(const lds_u32x4_t*)(f1 + (((k - 4) & 1) ? v_lane1 : v_lane0) + ((k - 4) >> 1) * 1024);
        if constexpr (k >= 12) ft[k - 12] = *(const lds_u32x4_t*)(t0 + kt_off(k - 12));
        if constexpr (k == 0) {
          word = *(const lds_u64_t*)(f1 + w_lane);
          e5v = list[min(j + 5, nsteps - 1) >> 1];
        }
        if constexpr (k < 12) mfma_s<k == 0>(acc, fk[k], qf[k]);
        else mfma_dp<k == 12>(dpp, fv[k - 12], of[k - 12], nd);
        if constexpr (k % 2 == 1 && k / 2 < 6) copy(IC<k / 2>{}, fdst, e4, (j + 4) & 1);   // F copies 0..5
        if constexpr (k < 8) {                       // dS(j) = P(j) (dP(j) - D), pair k, in place
          p[2 * k] *= dpp[2 * k];
          p[2 * k + 1] *= dpp[2 * k + 1];
          pkS[k >> 2][k & 3] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
          asm volatile("" :: "v"(pkS[k >> 2][k & 3]));
        }
        if constexpr (k == 7) {
          hv = vis_bits(e1, j + 1, word);
          asm volatile("" :: "v"(hv));
        }
        if constexpr (k >= 8) {                      // offsets of step j+1: 3, 3, 3, 3, 2, 2 per slot
          constexpr int lo = k < 12 ? 3 * (k - 8) : 12 + 2 * (k - 12);
          constexpr int cnt = k < 12 ? 3 : 2;
#pragma unroll
          for (int r = lo; r < lo + cnt; ++r) {
            adn[r] = offset_entry(r, hv);
            asm volatile("" :: "v"(adn[r]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (__builtin_expect(a.mask != nullptr && (e1 >> 24) == 3, 0)) general_offsets(e1, j + 1, adn);

      // ---- slots 14-31: dP^T(j+1) ends, dQ(j); P(j+1)
      static_for<18>([&](auto K0) __attribute__((always_inline)) {
        constexpr int k = decltype(K0)::value + 14;
        if constexpr (k % 4 == 0) wait_lgkm<4>();
        if constexpr (k < 24) ft[k - 12] = *(const lds_u32x4_t*)(t0 + kt_off(k - 12));
        if constexpr (k >= 24) fk[k - 24] = *(const lds_u32x4_t*)(f2 + k_off(k - 24));
        if constexpr (k < 20) mfma_dp<false>(dpp, fv[k - 12], of[k - 12], nd);
        else mfma_acc(dq[(k - 20) >> 1], ft[k - 20], pkS[k & 1]);
        if constexpr (k == 16 || k == 20 || k == 24) copy(IC<6 + (k - 16) / 4>{}, tdst, e2, (j + 2) & 1);   // T copies
        if constexpr (k < 30) {
          constexpr int u = k - 14;
          p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[u], c_log2, adn[u]));
          asm volatile("" :: "v"(p[u]));
        }
        __builtin_amdgcn_sched_barrier(0);
      });

      // this wave's copies of step j-1 done (those of step j may be in flight),
      // then F(j+3) and T(j+1) are published and F(j+1) / T(j) are free
      wait_vmem<kQCopiesPerStep>();
      step_barrier();
      e1 = e2;
      e2 = e3;
      e3 = e4;
      e4 = __builtin_amdgcn_readfirstlane(j + 5 < nsteps ? e5v : 0);
      const int fr = fs0;
      fs0 = fs1; fs1 = fs2; fs2 = fs3; fs3 = fr;
      const int tr = ts0;
      ts0 = ts1; ts1 = ts2; ts2 = tr;
    }
    wait_vmem<0>();
    __syncthreads();
  }

  // ---- store: accumulator row r <-> dim 32mt + 8(r/4) + 4hi + r%4, column <-> this lane's query
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dq[0]), "+a"(dq[1]), "+a"(dq[2]), "+a"(dq[3]), "+a"(dq[4]),
               "+a"(dq[5]));
  if (q_ok) {
    uint16_t* op = a.dq + (bh * a.Lq + qi) * kDqk;
#pragma unroll
    for (int mt = 0; mt < kDqk / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t w2 = {pack_bf16x2(dq[mt][4 * g] * a.scale, dq[mt][4 * g + 1] * a.scale),
                            pack_bf16x2(dq[mt][4 * g + 2] * a.scale, dq[mt][4 * g + 3] * a.scale)};
        *reinterpret_cast<u32x2_t*>(op + 32 * mt + 8 * g + 4 * hi) = w2;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const AttnBwdArgs& a, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(a.B) * a.nqt * a.H);
  if (a.mask && a.mask_bf16) hipLaunchKernelGGL(bwd_dq<true>, g, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(bwd_dq<false>, g, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
