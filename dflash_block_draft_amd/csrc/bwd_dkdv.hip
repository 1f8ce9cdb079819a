// dK and dV of the draft MLA attention (backward), bf16 MFMA on gfx950.
//
// With p = exp(s - lse) recomputed from the forward's row normaliser and
// ds = p (dout . v_j - D), D = rowsum(dout * out) (the softmax backward, stated
// for the attention the DFlash trainer differentiates: NeMo AutoModel DFlash
// page, KimiK3DFlashDraftModel; DSpark page, speculative-decoding training):
//   dv_j = sum_i p_ij dout_i,   dk_j = scale * sum_i ds_ij q_i.
//
// One workgroup per (b, h, 128 keys = two k-tiles); wave w owns 32 keys: their
// K and V operands stay in accumulator registers, dK (32 x 192) and dV (32 x 128)
// accumulate in accumulator registers.  The workgroup walks the 32-query chunks
// of every q-tile with a non-empty tile among its two k-tiles (a chunk list
// built in LDS at the start).  S = Q K^T and dP = dO V^T put one key per lane,
// which is the operand layout of dV += P^T dO and dK += dS^T Q, so P and dS go
// from the accumulator to the next operand without moving; the other operands
// (q and dout with the reduction over queries) come from transposed copies.
//
// Step i is software-pipelined over two chunks and split into two phases of 20
// MFMA slots, scheduled by hand (one MFMA, its operand reads issued eight slots
// ahead, a share of the vector work and of the copies per slot):
//   phase A: dV(i) from P(i); scores S(i+1);   vector: dS(i) = P(i) (dP(i) - D),
//            the exponent offsets of chunk i+1 (visibility and normaliser)
//   phase B: dP(i+1) - D(i+1) (the MFMA starts from -D); dK(i) from dS(i);
//            vector: P(i+1) = exp2(S(i+1) scale log2(e) + offset)
// so the matrix and vector work of a phase are independent.  Chunk j's q and
// dout rows, exponent offsets and visibility words (the F part) are read in step
// j - 1, its transposed q and dout (the T part) from the end of step j - 1 on;
// both are copied global -> LDS through the buffer unit in step j - 3 (rings of
// three and four slots), so every copy has a whole step to land.
//
// Masks: the exponent offset of a hidden (query, key) pair is -inf (binary tiles
// from the transposed visibility words, keys past Lk, dead or padded rows); a
// tile with general mask values takes offsets (m - lse) log2(e) computed between
// the phases from the mask and the normaliser in natural units.
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
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) int lds_int_t;

constexpr int kThreads = kKvWaves * 64;
constexpr int kListMax = 2048;                      // q-tiles per window of the chunk list
constexpr int kFRing = 0;
constexpr int kTRing = kFRing + kFSlots * kF_Slot;
constexpr int kList = kTRing + kTSlots * kT_Slot;
constexpr int kCnt = kList + kListMax * 4;
constexpr int kLdsBytes = kCnt + 64;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr uint32_t kNegInfBits = 0xFF800000u;

// A wave's barrier with the workgroup, without the LDS fence of __syncthreads:
// operand reads still in flight target slots that are rewritten only after a
// later barrier, and the copies are waited for explicitly before it.
__device__ __forceinline__ void step_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The four MFMA kinds, as asm so that the register file of every operand is
// fixed: S and dP accumulate in vector registers (the vector unit reads them),
// with their B operand (the wave's K or V) in accumulator registers; dK and dV
// accumulate in accumulator registers.  The compiler does not see their
// latencies: every vector reader of S is placed two MFMA issues after the last
// S MFMA, dP is read a phase later, and the registers of dP's C operand are held
// until the phase ends.
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
bwd_dkdv(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  lds_char_t* const lds = (lds_char_t*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 31, hi = lane >> 5;
  const int kb = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int b = static_cast<int>(bh / a.H);
  const int kt0 = 2 * kb;
  const bool has_kt1 = kt0 + 1 < a.nkt;
  const int my_t = w >> 1;                              // the wave's k-tile: kt0 + my_t
  const int key = kb * kKB + 32 * w + li;               // this lane's key
  const bool key_ok = key < a.Lk;

  // ---- the wave's K and V operands (B operands of S = Q K^T and dP = dO V^T:
  // key li, dims 16s + 8hi .. +8), moved to accumulator registers
  // (loaded here, moved once the first chunk list is built: the loads and the
  // tile classes of the list travel together)
  u32x4_t kq[kDqk / 16], vq[kDv / 16];
  u32x4_t kv[kDqk / 16], vv[kDv / 16];
#pragma unroll
  for (int s = 0; s < kDqk / 16; ++s) {
    kv[s] = zero4();
    if (key_ok) kv[s] = s < kDn / 16 ? ldg16(a.kn + (bh * a.Lk + key) * kDn + 16 * s + 8 * hi)
                                      : ldg16(a.kr + (static_cast<size_t>(b) * a.Lk + key) * kDr +
                                              16 * (s - kDn / 16) + 8 * hi);
  }
#pragma unroll
  for (int s = 0; s < kDv / 16; ++s) vv[s] = key_ok ? ldg16(a.v + (bh * a.Lk + key) * kDv + 16 * s + 8 * hi) : zero4();

  f32x16_t dk[kDqk / 32], dv[kDv / 32];
#pragma unroll
  for (int i = 0; i < kDqk / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = 0.f;
#pragma unroll
  for (int i = 0; i < kDv / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[i][r] = 0.f;

  // ---- copy plan (bwd_plan.h): per-lane source offsets fixed for the kernel
  const u32x4_t d_q = buffer_desc(a.q + bh * a.Lq * kDqk, static_cast<uint32_t>(a.Lq) * kDqk * 2);
  const u32x4_t d_o = buffer_desc(a.dout + bh * a.Lq * kDv, static_cast<uint32_t>(a.Lq) * kDv * 2);
  const u32x4_t d_ld = buffer_desc(a.ld + bh * a.Lqp * 2, static_cast<uint32_t>(a.Lqp) * 8);
  const u32x4_t d_b = buffer_desc(a.bitsT ? a.bitsT + (static_cast<size_t>(b) * a.nkt + kt0) * a.nqt * 256 : nullptr,
                                  a.bitsT ? static_cast<uint32_t>(has_kt1 ? 2 : 1) * a.nqt * 1024 : 0u);
  const u32x4_t d_qt = buffer_desc(a.qT + bh * kDqk * a.Lqp, static_cast<uint32_t>(kDqk) * a.Lqp * 2);
  const u32x4_t d_ot = buffer_desc(a.doT + bh * kDv * a.Lqp, static_cast<uint32_t>(kDv) * a.Lqp * 2);
  uint32_t vo[kCopiesPerStep];
#pragma unroll
  for (int j = 0; j < kCopiesPerStep; ++j) vo[j] = voff(w, j, lane, a.Lqp, a.nqt);
  // copy j of this wave for the chunk whose first query is q0 (live: a listed
  // chunk), into the slot at LDS byte slot_base
  auto copy = [&](auto J, uint32_t slot_base, bool live, uint32_t q0) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int reg = src_region(j);
    const uint32_t so = !live ? kPastEnd
                      : reg == kSrcQ ? q0 * (kDqk * 2) : reg == kSrcO ? q0 * (kDv * 2)
                      : reg == kSrcLD || reg == kSrcB ? q0 * 8 : q0 * 2;
    const u32x4_t d = reg == kSrcQ ? d_q : reg == kSrcO ? d_o : reg == kSrcLD ? d_ld : reg == kSrcB ? d_b
                    : reg == kSrcQT ? d_qt : d_ot;
    dma16s(d, slot_base, static_cast<uint32_t>(dst_base(w, j)), vo[j], so);
  };

  // ---- per-lane LDS read offsets inside a slot (bwd_plan.h)
  const int q_lane0 = rd_q(0, li, hi), q_lane1 = rd_q(1, li, hi);
  const int o_lane0 = rd_o(0, li, hi), o_lane1 = rd_o(1, li, hi);
  const int t_lane0 = rd_qt(0, 0, li, hi), t_lane1 = rd_qt(0, 1, li, hi);
  const int w_lane = rd_word(my_t, (w & 1) * 32 + li);
  int one;                                              // bit-field width 1 from an opaque register
  asm("s_mov_b32 %0, 1" : "=s"(one));
  const float c_log2 = a.scale * kLog2e;

  lds_int_t* const list = (lds_int_t*)(lds + kList);
  lds_int_t* const cnt = (lds_int_t*)(lds + kCnt);

  // ---- chunk list of the window of q-tiles from qb: the q-tiles with a non-empty
  // tile among the two k-tiles, entry = q-tile | class(kt0) << 24 | class(kt0 + 1) << 28
  auto build_list = [&](int qb) -> int {
    const int qe = min(a.nqt, qb + kListMax);
    int n = 0;
    for (int base = qb; base < qe; base += kThreads) {
      const int qt = base + t;
      int c0 = 0, c1 = 0;
      if (qt < qe) {
        if (!a.classes) {
          c0 = 1;
          c1 = has_kt1 ? 1 : 0;
        } else {
          const size_t row = (static_cast<size_t>(b) * a.nqt + qt) * a.nkt + kt0;
          c0 = a.classes[row];
          c1 = has_kt1 ? a.classes[row + 1] : 0;
        }
      }
      const bool nz = (c0 | c1) != 0;
      const uint64_t m = __ballot(nz);
      if (lane == 0) cnt[w] = __popcll(m);
      __syncthreads();
      int off = n;
      for (int j = 0; j < w; ++j) off += cnt[j];
      const int tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
      if (nz) list[off + __popcll(m & ((1ull << lane) - 1ull))] = qt | (c0 << 24) | (c1 << 28);
      n += tot;
      __syncthreads();
    }
    return n;
  };
  int n = build_list(0);
#pragma unroll
  for (int s = 0; s < kDqk / 16; ++s) asm volatile("" : "=a"(kq[s]) : "0"(kv[s]));
#pragma unroll
  for (int s = 0; s < kDv / 16; ++s) asm volatile("" : "=a"(vq[s]) : "0"(vv[s]));

  for (int qb = 0; qb < a.nqt; qb += kListMax, n = qb < a.nqt ? build_list(qb) : 0) {
    const int nch = 4 * n;                              // every q-tile in four chunks
    if (nch == 0) continue;
    // entry of chunk j (0 past the end: no copy, class 0)
    auto ent = [&](int j) __attribute__((always_inline)) -> int {
      const int v = list[min(j, nch - 1) >> 2];
      return __builtin_amdgcn_readfirstlane(j < nch ? v : 0);
    };
    auto q0_of = [&](int e, int j) __attribute__((always_inline)) -> uint32_t {
      return static_cast<uint32_t>((e & 0xFFFFFF) * kTileM + kQC * (j & 3));
    };
    auto cls_of = [&](int e) __attribute__((always_inline)) -> int { return (e >> (24 + 4 * my_t)) & 15; };
    auto f_slot = [&](int j) __attribute__((always_inline)) -> int { return kFRing + (j % kFSlots) * kF_Slot; };
    auto t_slot = [&](int j) __attribute__((always_inline)) -> int { return kTRing + (j % kTSlots) * kT_Slot; };
    auto copy_f = [&](int j, int e) __attribute__((always_inline)) {
      const uint32_t base = lds0 + f_slot(j);
      const bool live = (e >> 24) != 0;
      const uint32_t q0 = q0_of(e, j);
      static_for<7>([&](auto J) __attribute__((always_inline)) { copy(J, base, live, q0); });
    };
    auto copy_t = [&](int j, int e) __attribute__((always_inline)) {
      const uint32_t base = lds0 + t_slot(j);
      const bool live = (e >> 24) != 0;
      const uint32_t q0 = q0_of(e, j);
      static_for<5>([&](auto J) __attribute__((always_inline)) { copy(IC<7 + decltype(J)::value>{}, base, live, q0); });
    };

    // exponent offsets of chunk e: -lse log2(e) where the key is visible, -inf
    // where it is hidden (fast tiles), from the slot's LD block and word
    auto vis_bits = [&](int cls, uint32_t word) __attribute__((always_inline)) -> int {
      const uint32_t vm = !key_ok ? 0u : cls == 2 ? word : cls == 0 ? 0u : ~0u;
      return static_cast<int>(vm >> (4 * hi));
    };
    auto offset_entry = [&](int r, int hv, float nl) __attribute__((always_inline)) -> float {
      const int vis = __builtin_amdgcn_sbfe(hv, 8 * (r >> 2) + (r & 3), one);
      return __int_as_float((vis & __float_as_int(nl)) | (~vis & static_cast<int>(kNegInfBits)));
    };
    // general mask values: offsets (m - lse) log2(e) in natural units first
    // (m and lse may both be near -FLT_MAX), -inf for hidden keys or dead rows
    auto general_offsets = [&](int e, int j, float* adn) __attribute__((always_inline)) {
      const uint32_t q0 = q0_of(e, j);
      float mv[16], lv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = static_cast<int>(q0) + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool ok = key_ok && q < a.Lq;
        mv[r] = ok ? mask_value<MASK_BF16>(a.mask, (static_cast<size_t>(b) * a.Lq + q) * a.Lk + key) : 0.f;
        lv[r] = ok ? a.lse[bh * a.Lq + q] : -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) adn[r] = lv[r] == -INFINITY ? -INFINITY : (mv[r] - lv[r]) * kLog2e;
    };

    // ---- prologue: F(0), F(1), F(2), T(0), T(1), T(2) copied; chunk 0's S, dP, P
    int e0 = ent(0), e1 = ent(1), e2 = ent(2), e3 = ent(3);
    copy_f(0, e0);
    copy_t(0, e0);
    copy_f(1, e1);
    copy_t(1, e1);
    copy_f(2, e2);
    copy_t(2, e2);
    wait_vmem<2 * kCopiesPerStep>();                    // chunk 0's parts landed, chunks 1 and 2 in flight
    __syncthreads();

    f32x16_t acc;                                       // S of the next chunk
    float sp[16];                                       // P of the current chunk (fp32)
    f32x16_t dpp;                                       // dP - D of the current chunk
    u32x4_t pkP[2], pkS[2];                             // P^T and dS^T operands (bf16 pairs)
    float adn[16];                                      // exponent offsets of the next chunk
    f32x16_t nd;                                        // -D of the next chunk (C operand of its dP)
    u32x4_t fq[12], fd[8], ft[12], fo[8];               // operand fragments read ahead

    {
      const lds_char_t* const fs = lds + f_slot(0);
      const uint32_t word = *(const lds_u32_t*)(fs + w_lane);
      f32x4_t nl4[4], nd4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        nl4[g] = *(const lds_f32x4_t*)(fs + rd_nl(g, hi));
        nd4[g] = *(const lds_f32x4_t*)(fs + rd_nd(g, hi));
      }
      nd = f32x16_t{nd4[0][0], nd4[0][1], nd4[0][2], nd4[0][3], nd4[1][0], nd4[1][1], nd4[1][2], nd4[1][3],
                    nd4[2][0], nd4[2][1], nd4[2][2], nd4[2][3], nd4[3][0], nd4[3][1], nd4[3][2], nd4[3][3]};
      const int cls = cls_of(e0);
      const int hv = vis_bits(cls, word);
#pragma unroll
      for (int r = 0; r < 16; ++r) adn[r] = offset_entry(r, hv, nl4[r >> 2][r & 3]);
      if (a.mask && cls == 3) general_offsets(e0, 0, adn);
      static_for<12>([&](auto S) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        fq[s] = *(const lds_u32x4_t*)(fs + ((s & 1) ? q_lane1 : q_lane0) + (s >> 1) * 1024);
        mfma_s<s == 0>(acc, fq[s], kq[s]);
      });
      static_for<8>([&](auto S) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        fd[s] = *(const lds_u32x4_t*)(fs + ((s & 1) ? o_lane1 : o_lane0) + (s >> 1) * 1024);
        mfma_dp<s == 0>(dpp, fd[s], vq[s], nd);
      });
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc), "+v"(dpp));
#pragma unroll
      for (int u = 0; u < 16; ++u) sp[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[u], c_log2, adn[u]));
#pragma unroll
      for (int u = 0; u < 8; ++u) pkP[u >> 2][u & 3] = pack_bf16x2(sp[2 * u], sp[2 * u + 1]);
      const lds_char_t* const ts = lds + t_slot(0) + (kT_OT - kT_QT);
#pragma unroll
      for (int v = 0; v < 8; ++v) fo[v] = *(const lds_u32x4_t*)(ts + ((v & 1) ? t_lane1 : t_lane0) + (v >> 1) * 2048);
    }
    wait_vmem<kCopiesPerStep>();                        // chunk 1's parts landed (read in step 0)
    __syncthreads();                                    // F(0)'s slot is rewritten in step 0

    // Step i.  Entering: sp, pkP = P(i); dpp = dP(i) - D(i); fo = dO^T(i) operands.
    // e1, e2, e3: entries of chunks i+1 .. i+3.
    // ring slot offsets of steps i .. i+2 (F, 3 slots) and i .. i+3 (T, 4 slots),
    // rotated once per step instead of recomputed modulo the ring sizes
    int fs0 = f_slot(0), fs1 = f_slot(1), fs2 = f_slot(2);
    int ts0 = t_slot(0), ts1 = t_slot(1), ts2 = t_slot(2), ts3 = t_slot(3);
    for (int i = 0; i < nch; ++i) {
      const lds_char_t* const f1 = lds + fs1;                           // F(i+1)
      const lds_char_t* const t0 = lds + ts0;                           // T(i)
      const lds_char_t* const t1 = lds + ts1 + (kT_OT - kT_QT);         // T(i+1), dO^T
      const uint32_t fdst = lds0 + fs0;                                 // F(i+3) (slot of F(i)) <- copies
      const uint32_t tdst = lds0 + ts3;                                 // T(i+3) <- copies
      const bool live3 = (e3 >> 24) != 0;
      const uint32_t q3 = q0_of(e3, i + 3);
      const int cls1 = cls_of(e1);
      int e4v = 0;
      uint32_t word = 0;
      f32x4_t nl4[4], nd4[4];
      int hv = 0;

      // ---- phase A: dV(i) (slots 0-7), S(i+1) (slots 8-19); dS(i), offsets(i+1)
      // Every operand is read 8 slots ahead of its MFMA.  One wait per 4 slots,
      // for the operands (and the words and normalisers) read 8 to 5 slots back,
      // replaces a wait in front of every MFMA; N counts the LDS reads issued
      // since (slot 0 of phase A reads 4 values, slots 1-7 two, the rest one).
      static_for<20>([&](auto K) __attribute__((always_inline)) {
        constexpr int k = decltype(K)::value;
        if constexpr (k == 0 || k == 12 || k == 16) wait_lgkm<4>();
        if constexpr (k == 4) wait_lgkm<10>();
        if constexpr (k == 8) wait_lgkm<8>();
        if constexpr (k < 12) fq[k] = *(const lds_u32x4_t*)(f1 + ((k & 1) ? q_lane1 : q_lane0) + (k >> 1) * 1024);
        if constexpr (k == 0) {
          word = *(const lds_u32_t*)(f1 + w_lane);
          e4v = list[min(i + 4, nch - 1) >> 2];
        }
        if constexpr (k < 4) nl4[k] = *(const lds_f32x4_t*)(f1 + rd_nl(k, hi));
        if constexpr (k >= 4 && k < 8) nd4[k - 4] = *(const lds_f32x4_t*)(f1 + rd_nd(k - 4, hi));
        if constexpr (k >= 12) fd[k - 12] = *(const lds_u32x4_t*)(f1 + ((k & 1) ? o_lane1 : o_lane0) + ((k - 12) >> 1) * 1024);
        if constexpr (k < 8) mfma_acc(dv[k >> 1], pkP[k & 1], fo[k]);
        else mfma_s<k == 8>(acc, fq[k - 8], kq[k - 8]);
        if constexpr (k % 3 == 1) copy(IC<k / 3>{}, fdst, live3, q3);             // F copies 0..6
        if constexpr (k < 8) {
          const float d0 = sp[2 * k] * dpp[2 * k], d1 = sp[2 * k + 1] * dpp[2 * k + 1];
          pkS[k >> 2][k & 3] = pack_bf16x2(d0, d1);
          asm volatile("" :: "v"(pkS[k >> 2][k & 3]));
        }
        if constexpr (k == 8) {
          hv = vis_bits(cls1, word);
          asm volatile("" :: "v"(hv));
        }
        if constexpr (k == 12) {
          nd = f32x16_t{nd4[0][0], nd4[0][1], nd4[0][2], nd4[0][3], nd4[1][0], nd4[1][1], nd4[1][2], nd4[1][3],
                        nd4[2][0], nd4[2][1], nd4[2][2], nd4[2][3], nd4[3][0], nd4[3][1], nd4[3][2], nd4[3][3]};
          asm volatile("" :: "v"(nd));   // formed here, well before the MFMA that reads it
        }
        if constexpr (k >= 9 && k < 17) {
          constexpr int r0 = 2 * (k - 9);
          adn[r0] = offset_entry(r0, hv, nl4[r0 >> 2][r0 & 3]);
          adn[r0 + 1] = offset_entry(r0 + 1, hv, nl4[r0 >> 2][(r0 + 1) & 3]);
          asm volatile("" :: "v"(adn[r0]), "v"(adn[r0 + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (__builtin_expect(a.mask != nullptr && cls1 == 3, 0)) general_offsets(e1, i + 1, adn);

      // ---- phase B: dP(i+1) (slots 0-7), dK(i) (slots 8-19); P(i+1)
      static_for<20>([&](auto K) __attribute__((always_inline)) {
        constexpr int k = decltype(K)::value;
        if constexpr (k % 4 == 0) wait_lgkm<4>();   // one read per slot in this phase
        if constexpr (k < 12) ft[k] = *(const lds_u32x4_t*)(t0 + ((k & 1) ? t_lane1 : t_lane0) + (k >> 1) * 2048);
        else fo[k - 12] = *(const lds_u32x4_t*)(t1 + ((k & 1) ? t_lane1 : t_lane0) + ((k - 12) >> 1) * 2048);
        if constexpr (k < 8) mfma_dp<k == 0>(dpp, fd[k], vq[k], nd);
        else mfma_acc(dk[(k - 8) >> 1], pkS[k & 1], ft[k - 8]);
        if constexpr (k % 4 == 1) copy(IC<7 + k / 4>{}, tdst, live3, q3);         // T copies 7..11
        if constexpr (k >= 2 && k < 18) {
          constexpr int u = k - 2;
          sp[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[u], c_log2, adn[u]));
          asm volatile("" :: "v"(sp[u]));
          if constexpr (u & 1) {
            pkP[u >> 3][(u >> 1) & 3] = pack_bf16x2(sp[u - 1], sp[u]);
            asm volatile("" :: "v"(pkP[u >> 3][(u >> 1) & 3]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      asm volatile("" :: "v"(nd));                      // the first dP MFMA's C operand, held to here

      // this wave's copies of step i-1 done (those of step i may be in flight),
      // then F(i+2) and T(i+2) are published and F(i+1) / T(i) are free
      wait_vmem<kCopiesPerStep>();
      step_barrier();
      e1 = e2;
      e2 = e3;
      e3 = __builtin_amdgcn_readfirstlane(i + 4 < nch ? e4v : 0);
      const int fr = fs0;
      fs0 = fs1; fs1 = fs2; fs2 = fr;
      const int tr = ts0;
      ts0 = ts1; ts1 = ts2; ts2 = ts3; ts3 = tr;
    }
    // The last dK / dV MFMAs (inline asm, invisible to the hazard checks) must
    // finish before the vector unit reads their accumulators: 24 wait states
    // here, ahead of the barrier that every read below follows.  (An asm naming
    // the accumulators as operands would make the allocator copy them into
    // fresh register tuples.)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    wait_vmem<0>();
    __syncthreads();
  }

  // ---- store: accumulator row r <-> key 8(r/4) + 4hi + r%4 of the wave's 32, column <-> dim.
  // Rows r and r+1 are adjacent keys: the even lane of a lane pair stores dims
  // (2c, 2c+1) of row r and the odd lane those of row r+1, two elements per
  // store.  For bf16 each lane packs its own (row r, row r+1) values of its dim,
  // takes its partner's pack and picks one half of each (a byte permute).  The
  // stores go through buffer resources spanning the (b, h) slice, whose range
  // check drops the rows past Lk: no per-row tests.
  const bool odd = (li & 1) != 0;
  auto swap_pair = [](uint32_t x) __attribute__((always_inline)) -> uint32_t {   // value of lane l ^ 1
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xB1, 0xF, 0xF, false));
  };
  // byte selector over {partner (bytes 4-7), own (bytes 0-3)}: even lane (own.lo,
  // partner.lo), odd lane (partner.hi, own.hi)
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  const uint32_t slice = static_cast<uint32_t>(a.Lk);
  const __amdgpu_buffer_rsrc_t r_dk = __builtin_amdgcn_make_buffer_rsrc(a.dkn + bh * a.Lk * kDn, 0,
                                                                       static_cast<int>(slice * (kDn * 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t r_dv = __builtin_amdgcn_make_buffer_rsrc(a.dv + bh * a.Lk * kDv, 0,
                                                                       static_cast<int>(slice * (kDv * 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t r_rp = __builtin_amdgcn_make_buffer_rsrc(a.rope_part + bh * a.Lk * kDr, 0,
                                                                       static_cast<int>(slice * (kDr * 4)), 0x00020000);
  const int col = li & ~1;
  const uint32_t row0 = static_cast<uint32_t>(kb * kKB + 32 * w + 4 * hi + (odd ? 1 : 0));
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const uint32_t row = row0 + 8 * (r >> 2) + (r & 3);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint32_t kown = pack_bf16x2(dk[nt][r] * a.scale, dk[nt][r + 1] * a.scale);
      const uint32_t vown = pack_bf16x2(dv[nt][r], dv[nt][r + 1]);
      const uint32_t kp = __builtin_amdgcn_perm(swap_pair(kown), kown, sel);
      const uint32_t vp = __builtin_amdgcn_perm(swap_pair(vown), vown, sel);
      __builtin_amdgcn_raw_buffer_store_b32(kp, r_dk, static_cast<int>(row * (kDn * 2) + (32 * nt + col) * 2), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(vp, r_dv, static_cast<int>(row * (kDv * 2) + (32 * nt + col) * 2), 0, 0);
    }
#pragma unroll
    for (int nt = 4; nt < 6; ++nt) {
      const float k0 = dk[nt][r] * a.scale, k1 = dk[nt][r + 1] * a.scale;
      const float kx = __uint_as_float(swap_pair(__float_as_uint(odd ? k0 : k1)));
      const u32x2_t pr = odd ? u32x2_t{__float_as_uint(kx), __float_as_uint(k1)}
                             : u32x2_t{__float_as_uint(k0), __float_as_uint(kx)};
      __builtin_amdgcn_raw_buffer_store_b64(pr, r_rp, static_cast<int>(row * (kDr * 4) + (32 * (nt - 4) + col) * 4), 0, 0);
    }
  }
}

// ---- the transposed visibility words of the class-2 tiles: one wave per tile,
// lane q holds rows q and 64 + q; the ballot over lanes of bit k gives key k's
// column
__global__ void __launch_bounds__(256) bwd_prep_bits(AttnBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (b * nqt + qt) * nkt + kt
  const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
  if (tile >= ntiles || a.classes[tile] != 2) return;
  const int kt = static_cast<int>(tile % a.nkt);
  const int64_t bq = tile / a.nkt;
  const int qt = static_cast<int>(bq % a.nqt), b = static_cast<int>(bq / a.nqt);
  const uint64_t w0 = a.bits[tile * kTileM + lane], w1 = a.bits[tile * kTileM + 64 + lane];
  uint64_t r0 = 0, r1 = 0;
#pragma unroll 8
  for (int k = 0; k < 64; ++k) {
    const uint64_t m0 = __ballot((w0 >> k) & 1ull), m1 = __ballot((w1 >> k) & 1ull);
    if (lane == k) {
      r0 = m0;
      r1 = m1;
    }
  }
  uint32_t* dst = a.bitsT + ((static_cast<size_t>(b) * a.nkt + kt) * a.nqt + qt) * 256 + lane;
  dst[0] = static_cast<uint32_t>(r0);
  dst[64] = static_cast<uint32_t>(r0 >> 32);
  dst[128] = static_cast<uint32_t>(r1);
  dst[192] = static_cast<uint32_t>(r1 >> 32);
}

}  // namespace

hipError_t launch_bwd_dkdv(const AttnBwdArgs& a, hipStream_t s) {
  if (a.bits) {
    const int64_t ntiles = static_cast<int64_t>(a.B) * a.nqt * a.nkt;
    hipLaunchKernelGGL(bwd_prep_bits, dim3(static_cast<unsigned>((ntiles + 3) / 4)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 g((a.Lk + kKB - 1) / kKB, static_cast<unsigned>(a.B) * a.H);
  if (a.mask && a.mask_bf16) hipLaunchKernelGGL(bwd_dkdv<true>, g, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(bwd_dkdv<false>, g, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
