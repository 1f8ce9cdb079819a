// Fused non-causal draft MLA attention forward, bf16 MFMA on gfx950: one wave
// per SIMD holding 64 queries.
//
// What it computes (NeMo AutoModel DFlash page, KimiK3DFlashAttention.forward;
// DSpark page, KimiK3DSparkAttention): for every (batch, head, noise query)
//   s_j = scale * (q_nope . k_nope[h][j] + q_rope . k_rope[j]) + mask[i][j]
//   out = softmax_j(s) @ v[h]
// over the keys [context | noise block], with no materialised score matrix.
//
// Decomposition (one workgroup = one (batch, head, 128-query tile), two waves,
// two workgroups per CU so every SIMD holds exactly one wave):
//  * Wave w owns queries 64w .. 64w+63 of the tile as two streams of 32
//    (stream i: queries 64w + 32i + lane%32).  Each K and V operand read from
//    LDS feeds one MFMA of each stream.
//  * The key loop walks the tile list in steps of 32 keys (half a 64-key tile),
//    each in two phases of 20 MFMAs with one workgroup barrier per step:
//      phase A: score MFMAs of stream 0 for the next step, PV of stream 0
//               || softmax of stream 1 for the current step
//      phase B: score MFMAs of stream 1 for the next step, PV of stream 1
//               || softmax of stream 0 for the next step
//    The matrix and vector work of a phase belong to different streams, so the
//    wave keeps the matrix core busy while its VALU does exponentials (the
//    ping-pong of FlashAttention-3's warp-group scheduling, inside one wave).
//    Each phase is hand-scheduled into 20 slots (one MFMA, its operand reads
//    and one unit of softmax work per slot, with scheduling barriers between
//    slots).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane holds one query and 16 of its 32 keys, so row sums are in-lane (one
//    permlane32 swap joins the halves), and the packed bf16 P^T is directly the
//    B operand of O^T = V^T P^T (keys are relabelled to the accumulator order).
//    V^T operands come from the V tile with the transposing LDS read.
//  * Keys hidden by a binary (0 / -inf) tile are removed by the first score
//    MFMA itself: its C operand is a bias block of 0 / -inf built from the
//    tile's per-query visibility words.  Tiles with other mask values, ragged
//    key tails and the first visible step take an exact path that reads them.
//  * K = [k_nope | head-shared k_rope], V and the visibility words go global ->
//    LDS with buffer_load ... lds (no VGPR staging; out-of-range rows read
//    zeros, so ragged and phantom steps need no branches) into rings of 4 (K),
//    3 (V) and 3 (words) slots; the copies of a step are spread over the MFMA
//    slots of its two phases.  LDS tiles are 16-row x 64 B blocks with
//    XOR-swizzled K chunks: conflict-free 16-byte operand reads.
//  * Q (2 x 32 x 192 bf16) stays in accumulator registers for the whole loop.
//    The K operands of a step (32 keys x 192) sit in vector registers: read
//    once from LDS, a whole phase before their first use, they serve the score
//    MFMAs of both streams.
//  * Online softmax in fp32 with the hardware exp2 and a stabiliser m fixed at
//    the first visible step of each row: later steps form exp(s - m) without
//    rescaling O.  Any stabiliser gives the same result in exact arithmetic
//    because it scales O and l alike; it only has to keep every exp(s - m)
//    within fp32 range and the bf16 P operand accurate, so a step whose scores
//    exceed m by more than 20 ln 2 (p > 2^20) marks the workgroup, and a
//    marked workgroup runs again in two passes: the exact row maxima first,
//    then the accumulation with those maxima as stabilisers.  The row sum l
//    adds the fp32 probabilities on the fast path and, on the exact path
//    (general mask values, where peaked rows come from), the bf16-rounded
//    values PV applies: the stabiliser is no row maximum, so no weight is
//    exactly 1, and there the rounding of a dominant weight would otherwise
//    show in full.  (Summing rounded values costs a dot2 per pair, which waits
//    on the matrix core: 5% of the loop on the fast path.)
#include "common.h"
#include "dma.h"
#include "launch.h"

#include <cfloat>
#include <type_traits>
#include <utility>

namespace dflash {
namespace {

constexpr int kWaves = 2;
constexpr int kThreads = kWaves * 64;
constexpr int kKSlot = 32 * kDqk * 2;               // 12 KiB: 2 row blocks x 6 chunk quads x 1 KiB
constexpr int kVSlot = 32 * kDv * 2;                // 8 KiB: 2 row blocks x 4 chunk quads x 1 KiB
constexpr int kBitsSlot = kTileM * 8;               // 1 KiB: one visibility word per query of a 64-key tile
constexpr int kNK = 4;                              // K ring slots (32-key steps)
constexpr int kNV = 3;                              // V ring slots (32-key steps)
constexpr int kNB = 3;                              // visibility-word ring slots (64-key tiles)
constexpr int kKRing = 0;
constexpr int kVRing = kKRing + kNK * kKSlot;
constexpr int kBitsRing = kVRing + kNV * kVSlot;
constexpr int kLdsBytes = kBitsRing + kNB * kBitsSlot;
// MFMA order of a phase: score chunks c (0-11, one dependent chain) and PV
// operations 100 + v (v = 4*st + j: four independent accumulators), placed so
// that only three score MFMAs directly follow their predecessor in the chain and
// the chain ends in the last slot
constexpr int kSlotOp[20] = {0, 100, 1, 101, 2, 102, 3, 103, 4, 104, 5, 105, 6, 106, 7, 8, 107, 9, 10, 11};
static_assert(kLdsBytes <= 80 * 1024, "two workgroups per CU");
constexpr float kSumLimit = 1048576.0f;              // fast path keeps every probability <= 2^20
constexpr float kHeadroom = 13.8629436f;             // 20 ln 2: scores may exceed the stabiliser by this much
constexpr int kPassNormal = 0;                       // accumulate O and l
constexpr int kPassMax = 1;                          // row maxima only (second pass of a rare item)
constexpr uint32_t kNegInfBits = 0xFF800000u;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
typedef __attribute__((address_space(3))) char lds_char_t;

template <int N>
using IC = std::integral_constant<int, N>;

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ s16x4_t ds_read_tr(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// 16 bytes per lane from a buffer straight into LDS at lds_base + 16*lane, from
// byte voff + SOFF of the buffer, lds_base a uniform LDS address and LOFF a
// constant added to it (one scalar add into m0).  SOFF selects a 64-byte chunk quad inside a
// row and goes in the scalar offset (the instruction's immediate offset would
// move the LDS destination too); the row offset is in voff, so a row is in or
// out of the buffer's range as a whole and out-of-range rows read zeros.
// Inline asm for the same reason as dma16: the compiler must not make unrelated
// LDS reads wait for this write; completion is awaited with wait_vmem before
// the barrier that publishes the slot.
template <int SOFF, int LOFF>
__device__ __forceinline__ void dma16i(u32x4_t rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dwordx4 %0, %1, %4 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_base), "i"(LOFF), "s"(SOFF) : "scc");
}

template <bool MASK_BF16>
__device__ __forceinline__ float load_mask(const void* mask, size_t idx) {
  if (MASK_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(mask)[idx]);
  return static_cast<const float*>(mask)[idx];
}

// acc + the two bf16 values of a packed pair (a dot product with (1, 1))
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                         acc, false);
}

// Workgroup barrier of the key loop.  It publishes the LDS copies each wave has
// already waited for (wait_vmem); the operand reads a wave has in flight need no
// wait here (__syncthreads would add one): the slots they read are rewritten
// only after a later barrier, and their registers are waited for where they are
// used.  The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void step_barrier() { asm volatile("s_barrier" ::: "memory"); }

// f(IC<0>{}), ..., f(IC<N-1>{}) in order
template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(IC<Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// One chunk of S^T = K Q^T with the accumulator in vector registers, where the
// softmax reads it with plain VALU instructions (the accumulators of O stay in
// accumulator registers, written by the compiler's own MFMAs); the B operand
// (Q) sits in accumulator registers.  The first chunk adds the bias block
// that hides the masked keys of a binary tile (0 elsewhere).  Written as asm,
// the compiler does not know the result arrives one MFMA latency later: every
// reader of acc is placed at least two MFMA issues later, or behind
// s_nop_after_mfma.
template <int KIND>   // 0: continue the chain; 1: start it from bias; 2: start it from zero
__device__ __forceinline__ void mfma_s(f32x16_t& acc, bf16x8_t k, const u32x4_t& q, const f32x16_t& bias) {
  const u32x4_t kk = __builtin_bit_cast(u32x4_t, k);
  if constexpr (KIND == 1)   // the chain starts from the hidden-key bias (0 or -inf per key)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(kk), "a"(q), "v"(bias));
  else if constexpr (KIND == 2)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(kk), "a"(q));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(kk), "a"(q));
}
// first chunk of a chain: from the bias block when the step's tile is binary
// (class 2), else from zero; the choice is one scalar branch around the MFMA
__device__ __forceinline__ void mfma_s_first(int cls, f32x16_t& acc, bf16x8_t k, const u32x4_t& q,
                                             const f32x16_t& bias) {
  const u32x4_t kk = __builtin_bit_cast(u32x4_t, k);
  asm("s_cmp_lg_u32 %4, 2\n\t"
      "s_cbranch_scc1 1f\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n"
      "2:"
      : "=&v"(acc) : "v"(kk), "a"(q), "v"(bias), "s"(cls) : "scc");
}
// the MFMA result in acc is readable by the VALU after this (16 wait states)
__device__ __forceinline__ void s_nop_after_mfma(f32x16_t& acc) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc));
}

template <bool MASK_BF16, bool LIST>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_bf16(AttnBf16Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  lds_char_t* const lds = (lds_char_t*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: heads of one (batch, q-tile, split) are adjacent in launch
  // order; split sp takes the sp-th of nsplit contiguous runs of the tile list
  const int h = blockIdx.x % a.H;
  const int item = blockIdx.x / a.H;
  const int sp = item % a.nsplit;
  const int rank = item / a.nsplit;
  const int bq = a.order ? a.order[rank] : rank;
  const int b = bq / a.nqt;
  const int qt = bq % a.nqt;
  const int n_all = LIST ? a.counts[bq] : a.nkt;
  const int t_begin = static_cast<int>(static_cast<int64_t>(n_all) * sp / a.nsplit);
  const int ntiles = static_cast<int>(static_cast<int64_t>(n_all) * (sp + 1) / a.nsplit) - t_begin;
  const int nsteps = 2 * ntiles;

  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const size_t tile_row0 = static_cast<size_t>(bq) * a.nkt;
  int q_local[2], q_row[2];
  bool q_ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    q_local[i] = 64 * wave + 32 * i + li;
    q_row[i] = qt * kTileM + q_local[i];
    q_ok[i] = q_row[i] < a.Lq;
  }

  // ---- tile list (entry: k-tile | class << 24).  Entries past the end repeat
  // the last one: the steps they feed are never used (their scores are dropped,
  // their copies land in slots no used step reads), so they only need addresses
  // the copies may read, which any entry gives (the copies are range checked).
  // Without a list every k-tile of the run is class 1.  The list is read through
  // a window of 64 entries held one per lane of a vector register (readlane per
  // entry, a refill every 64 tiles): no scalar loads in the key loop, whose
  // completion, out of order with LDS reads, would make every LDS wait drain.
  const int32_t* list = LIST ? a.lists + tile_row0 + t_begin : nullptr;
  const int last = max(ntiles - 1, 0);
  int wbase = 0;                               // entries wbase .. wbase+63 are in lwin
  // In the kernel an entry also carries bit 26, set for a slow tile (general
  // mask values, or keys past Lk: its steps go to the exact path), added when
  // the window is filled so the loop tests one bit.
  auto tag_slow = [&](int32_t x) __attribute__((always_inline)) -> int32_t {
    const bool slow = (x >> 24) == 3 || (x & 0xFFFFFF) * kTileN + kTileN > a.Lk;
    return x | (slow ? 1 << 26 : 0);
  };
  int32_t lwin = LIST ? tag_slow(list[min(lane, last)]) : 0;
  auto entry = [&](int i) __attribute__((always_inline)) -> int {
    const int j = min(i, last);
    if constexpr (LIST) {
      if (j - wbase >= 64) {                   // entries are read in increasing order
        wbase = j;
        lwin = tag_slow(list[min(j + lane, last)]);
        asm volatile("" :: "v"(lwin));       // waited for here, not where the paths join
      }
      return __builtin_amdgcn_readlane(lwin, j - wbase);
    } else {
      return tag_slow((t_begin + j) | (1 << 24));
    }
  };
  auto ktile = [](int e) __attribute__((always_inline)) -> int { return e & 0xFFFFFF; };
  auto eclass = [](int e) __attribute__((always_inline)) -> int { return (e >> 24) & 3; };
  auto key0_of = [&](int e, int half) __attribute__((always_inline)) -> int { return ktile(e) * kTileN + 32 * half; };
  auto slow_tile = [](int e) __attribute__((always_inline)) -> bool { return (e >> 26) & 1; };

  // ---- global -> LDS copy plan: wave w copies row block w (keys 16w .. 16w+15
  // of the step) of K (k_nope quads 0-3, k_rope quads 4-5) and of V (quads 0-3);
  // lane l covers row 16w + l/4, LDS slot l%4 of each quad, K chunks swizzled.
  // LDS slot addresses are uniform values plus constants.
  const u32x4_t d_kn = buffer_desc(a.kn + bh * a.Lk * kDn, a.Lk * kDn * 2);
  const u32x4_t d_kr = buffer_desc(a.kr + static_cast<size_t>(b) * a.Lk * kDr, a.Lk * kDr * 2);
  const u32x4_t d_v = buffer_desc(a.v + bh * a.Lk * kDv, a.Lk * kDv * 2);
  const u32x4_t d_bits = buffer_desc(a.bits ? a.bits + tile_row0 * kTileM : nullptr, a.bits ? a.nkt * kBitsSlot : 0);
  const int r16 = lane >> 2, s4 = lane & 3;
  const int crow = wave * 16 + r16;                       // key row of the step this lane copies
  const int kslot = s4 ^ ((r16 >> 2) & 3);
  const uint32_t vo_kn = crow * (kDn * 2) + kslot * 16;
  const uint32_t vo_kr = crow * (kDr * 2) + kslot * 16;
  const uint32_t vo_v = crow * (kDv * 2) + s4 * 16;
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds0 + kKRing + wave * 6 * 1024);
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(lds0 + kVRing + wave * 4 * 1024);
  const uint32_t lds_b = __builtin_amdgcn_readfirstlane(lds0 + kBitsRing);
  // piece P of a step's K copy (k_nope quads 0-3, k_rope quads 4-5) or V copy
  // (quads 0-3) into the slot at LDS address base, for keys key0 .. key0+31
  auto issue_k_piece = [&](auto P, uint32_t base, int key0) __attribute__((always_inline)) {
    constexpr int pc = decltype(P)::value;
    if constexpr (pc < 4) dma16i<pc * 64, pc * 1024>(d_kn, base, vo_kn + static_cast<uint32_t>(key0) * (kDn * 2));
    else dma16i<(pc - 4) * 64, pc * 1024>(d_kr, base, vo_kr + static_cast<uint32_t>(key0) * (kDr * 2));
  };
  auto issue_v_piece = [&](auto P, uint32_t base, int key0) __attribute__((always_inline)) {
    constexpr int pc = decltype(P)::value;
    dma16i<pc * 64, pc * 1024>(d_v, base, vo_v + static_cast<uint32_t>(key0) * (kDv * 2));
  };
  auto issue_k = [&](uint32_t base, int key0) __attribute__((always_inline)) {
    static_for<6>([&](auto P) __attribute__((always_inline)) { issue_k_piece(P, base, key0); });
  };
  auto issue_v = [&](uint32_t base, int key0) __attribute__((always_inline)) {
    static_for<4>([&](auto P) __attribute__((always_inline)) { issue_v_piece(P, base, key0); });
  };
  // visibility words of tile e (1 KiB) into the word slot at byte offset boff;
  // both waves copy the same bytes.  Only binary tiles have words; the slot of
  // any other tile is never read.
  auto issue_bits = [&](uint32_t boff, int e) __attribute__((always_inline)) {
    dma16i<0, 0>(d_bits, lds_b + boff, lane * 16 + static_cast<uint32_t>(ktile(e)) * kBitsSlot);
  };

  // ---- per-lane LDS read offsets inside a slot
  // K operand of chunk c (dims 16c .. 16c+15): 16-byte chunk 2c+hi of key row li
  // -> block (li/16)*6 + c/2, slot (2(c&1) + hi) ^ swz(row)
  const int kq = (li >> 2) & 3;
  const int k_even = ((li >> 4) * 6) * 1024 + (li & 15) * 64 + (hi ^ kq) * 16;
  const int k_odd = ((li >> 4) * 6) * 1024 + (li & 15) * 64 + ((2 + hi) ^ kq) * 16;
  // V^T operand (transposing read): lane i of 16-lane group G addresses row
  // 16*st + 4*hi + i/4 (+8), dims 32*j + 16*(G&1) + 4*(i&3)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vrow = 4 * hi + (i16 >> 2);
  const int v_base = vrow * 64 + (2 * (g16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8;
  const lds_char_t* const ke_ptr = lds + kKRing + k_even;
  const lds_char_t* const ko_ptr = lds + kKRing + k_odd;
  const lds_char_t* const v_ptr = lds + kVRing + v_base;

  // ---- Q fragments (B operand of S^T = K Q^T), stream i, 12 chunks of 16 dims,
  // kept in accumulator registers for the whole loop (the MFMA reads its B
  // operand from either file): the vector registers hold the K operands of a
  // whole step, the V operands and the softmax.  All 24 loads are in flight
  // together; each chunk then moves to accumulator registers (a tied asm
  // operand: the compiler emits the moves).  Rows past Lq read row 0 (their
  // results are never stored).
  u32x4_t qf[2][kDqk / 16];
  {
    u32x4_t qv[2][kDqk / 16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t* qp = a.q + (bh * a.Lq + (q_ok[i] ? q_row[i] : 0)) * kDqk + 8 * hi;
#pragma unroll
      for (int c = 0; c < kDqk / 16; ++c) qv[i][c] = ldg16(qp + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < kDqk / 16; ++c) asm volatile("" : "=a"(qf[i][c]) : "0"(qv[i][c]));
  }

  f32x16_t o[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][j][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};   // stabiliser (natural units), same in both lane halves
  float l_run[2] = {0.f, 0.f};               // this lane's partial row sums
  float l_max[2] = {0.f, 0.f};               // largest fast-path step sum (checked once, after the pass)
  // the C operand of the next phase's first score MFMA when its step's tile is
  // binary: -inf at the keys the tile hides from the phase's stream, 0 elsewhere
  // (one block serves both streams: each phase's block is built just before it)
  f32x16_t biasb;
#pragma unroll
  for (int r = 0; r < 16; ++r) biasb[r] = 0.f;
  bool over = false;                         // a score rose more than kHeadroom above its stabiliser
  bool first[2];                             // some lane of the stream has no stabiliser yet
  // -m * log2e of each stream's stabiliser, the fast path's exponent offset,
  // held within +-FLT_MAX (NaN kept): with m near -FLT_MAX the product
  // overflows, and a hidden key's -inf plus an infinite offset would be NaN where
  // the finite bound gives exp2(-inf) = 0.  Updated wherever m changes.
  float cbs[2];
  auto stab_off = [](float m) __attribute__((always_inline)) -> float {
    const float c = -m * kLog2e;
    return c > FLT_MAX ? FLT_MAX : (c < -FLT_MAX ? -FLT_MAX : c);
  };
  f32x16_t s[2];                             // raw scores of each stream's pending softmax step
  uint32_t pk[2][8];                         // P^T of each stream's step awaiting PV, bf16 pairs
  bf16x8_t kreg[kDqk / 16];                  // K operands of the next step's scores (both streams)
  s16x8_t vf[8];                             // V^T operands of the step awaiting PV (op = 4*st + j)

  const float scale = a.scale;
  const float scale_log2 = a.scale * kLog2e;
  size_t mask_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) mask_row[i] = (static_cast<size_t>(b) * a.Lq + (q_ok[i] ? q_row[i] : 0)) * a.Lk;

  // operand reads from the ring slot at byte offset off
  auto read_k = [&](uint32_t off, int c) __attribute__((always_inline)) -> bf16x8_t {
    const lds_char_t* kp = ((c & 1) ? ko_ptr : ke_ptr) + off + (c >> 1) * 1024;
    return as_bf16x8(*reinterpret_cast<const lds_u32x4_t*>(kp));
  };
  auto read_v = [&](uint32_t off, int op) __attribute__((always_inline)) -> s16x8_t {
    const lds_char_t* vp = v_ptr + off + (op >> 2) * 4096 + (op & 3) * 1024;
    const s16x4_t lo = ds_read_tr(vp);
    const s16x4_t hi4 = ds_read_tr(vp + 512);
    return s16x8_t{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };
  // bias of stream i for half `half` of a binary tile: from the query's
  // visibility word, bit 8g+c <-> key 8g+4hi+c of the step (accumulator r =
  // 4g+c).  The bit-field width comes from an opaque register (it is 1) so each
  // entry compiles to a bit-field extract and an and.
  int one;
  asm("s_mov_b32 %0, 1" : "=s"(one));
  // the visibility word of stream i's query in the word slot at byte offset boff
  auto bias_word = [&](auto I, uint32_t boff) __attribute__((always_inline)) -> uint64_t {
    constexpr int i = decltype(I)::value;
    return *reinterpret_cast<const lds_u64_t*>(lds + kBitsRing + boff + q_local[i] * 8);
  };
  auto bias_build = [&](int half, uint64_t w64) __attribute__((always_inline)) -> f32x16_t {
    const int hv = static_cast<int>(~static_cast<uint32_t>(w64 >> (32 * half + 4 * hi)));   // hidden keys
    f32x16_t bb;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      bb[r] = __int_as_float(__builtin_amdgcn_sbfe(hv, 8 * (r >> 2) + (r & 3), one) & static_cast<int>(kNegInfBits));
    return bb;
  };
  // A phase prefetches the visibility word its stream's next scores need (slot
  // 0); after the phase the block is built from it only when that step's tile is
  // binary (a uniform branch), and the next phase's first score MFMA reads it
  // only then.  Steps of the other tiles, most of them, build nothing.
  auto bias_slot = [&](auto I, auto K, uint32_t boff, uint64_t& w) __attribute__((always_inline)) {
    if constexpr (decltype(K)::value == 0) w = bias_word(I, boff);
  };
  auto bias_fix = [&](int half, int e, uint64_t w) __attribute__((always_inline)) {
    if (eclass(e) == 2) biasb = bias_build(half, w);
  };

  // p = exp2(fma(x, ca, cb)) -> pk (bf16 pairs); returns the lane's sum of the
  // bf16-rounded p, the weights PV applies
  auto probs = [&](uint32_t* pk, const float* x, float ca, float cb) __attribute__((always_inline)) -> float {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], ca, cb));
#pragma unroll
    for (int u = 0; u < 8; ++u) pk[u] = pack_bf16x2(p[2 * u], p[2 * u + 1]);
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      l0 = sum_bf16x2(pk[u], l0);
      l1 = sum_bf16x2(pk[u + 1], l1);
    }
    return l0 + l1;
  };
  // scaled scores of stream i on the step at (entry e, half), natural units:
  // general mask values added and keys past Lk at -inf (the hidden keys of a
  // binary tile are -inf already: the score MFMAs started from their bias)
  auto masked_scores = [&](auto I, int e, int half, const f32x16_t& s, float* x) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    const int cls = eclass(e);
    // accumulator r <-> key kbase + 8*(r>>2) + (r&3)
    const int kbase = (e & 0xFFFFFF) * kTileN + 32 * half + 4 * hi;
    if (cls == 3 && a.mask) {   // (a reused map without its mask: no values to add)
      float mv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {   // all 16 loads in flight together (clamped index, fixed below)
        const int kk = kbase + 8 * (r >> 2) + (r & 3);
        mv[r] = load_mask<MASK_BF16>(a.mask, mask_row[i] + min(kk, a.Lk - 1));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], scale, q_ok[i] ? mv[r] : 0.f);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * scale;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kbase + 8 * (r >> 2) + (r & 3) >= a.Lk) x[r] = -INFINITY;
  };
  // maximum of the lane's query over the step (both lane halves)
  auto step_max = [&](const float* x) __attribute__((always_inline)) -> float {
    float tmax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, x[r]);
    return halves_max(tmax);
  };
  // exact path of stream i.  The stabiliser is never raised once set, so O is
  // never rescaled: a lane without one takes the step's maximum (its O and l are
  // still zero), and a lane whose scores rise more than kHeadroom above its
  // stabiliser marks the work item for the second pass.
  auto soft_exact = [&](auto I, int e, int half, const f32x16_t& s, uint32_t* pk) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    float x[16];
    masked_scores(I, e, half, s, x);
    const float tmax = step_max(x);
    if (m_run[i] == -INFINITY) m_run[i] = tmax;
    else if (!(tmax <= m_run[i] + kHeadroom)) over = true;
    // subtract before scaling: m * log2e can overflow where x - m does not (mask values near -FLT_MAX)
    const float m_use = m_run[i] == -INFINITY ? 0.f : m_run[i];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] -= m_use;
    l_run[i] += probs(pk, x, kLog2e, 0.f);
    first[i] = __any(m_run[i] == -INFINITY);
    cbs[i] = stab_off(m_run[i]);
  };
  // ---- one phase of the accumulation pass, scheduled by hand: 20 slots
  // separated by scheduling barriers.  Slot k issues the k-th MFMA of stream
  // MS's matrix work (scores of the next step into s[MS] from the K operands in
  // kreg; PV of the current step into o[MS] with the V operands vf and P^T
  // pk[MS]; with RELOAD, the second phase of a step, each K and V register is
  // refilled right after its MFMA, K from slot ks (the step after next) and V
  // from slot vsl (the next step): the reads have a whole phase to land, and
  // each K operand is read once per step for both streams) and, from slot 2
  // on, one unit of the fast softmax of stream VS = 1 - MS on s[VS],
  // software-pipelined over its 16 scores (exponential of score u; the bf16
  // pair of scores u-2 and u-1 and the fp32 sum of score u-1).  Starting the softmax two MFMA
  // issues into the phase keeps the other stream's last score MFMA of the
  // previous phase at a safe distance from its readers.  Returns the lane's sum.
  auto phase_fast = [&](auto MSc, auto RELOAD, auto EXTRA, auto VEXTRA, uint32_t ks, uint32_t vsl, int cls)
      __attribute__((always_inline)) -> float {
    constexpr int ms = decltype(MSc)::value;
    constexpr int vs = 1 - ms;
    constexpr bool reload = decltype(RELOAD)::value;
    const float cb = cbs[vs];
    f32x16_t acc;
    float p[16];
    float l0 = 0.f, l1 = 0.f;
    static_for<20>([&](auto K) __attribute__((always_inline)) {
      constexpr int k = decltype(K)::value;
      constexpr int op = kSlotOp[k];
      if constexpr (op < 100) {
        constexpr int c = op;
        if constexpr (c == 0) mfma_s_first(cls, acc, kreg[c], qf[ms][c], biasb);
        else mfma_s<0>(acc, kreg[c], qf[ms][c], biasb);
        if constexpr (reload) kreg[c] = read_k(ks, c);
      } else {
        constexpr int v = op - 100, st = v >> 2, j = v & 3;
        const u32x4_t pb = {pk[ms][4 * st + 0], pk[ms][4 * st + 1], pk[ms][4 * st + 2], pk[ms][4 * st + 3]};
        o[ms][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[v]), as_bf16x8(pb),
                                                           o[ms][j], 0, 0, 0);
        if constexpr (reload) vf[v] = read_v(vsl, v);
      }
      EXTRA(K);
      VEXTRA(K);
      constexpr int u = k - 2;
      // (each value is pinned to its slot by an empty asm that uses it: the
      // compiler would otherwise sink the softmax towards its consumers)
      if constexpr (u >= 0 && u < 16) {
        p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[vs][u], scale_log2, cb));
        asm volatile("" :: "v"(p[u]));
      }
      if constexpr (u >= 1 && u <= 16) {
        constexpr int w = u - 1;
        if constexpr (w & 1) {
          pk[vs][w >> 1] = pack_bf16x2(p[w - 1], p[w]);
          asm volatile("" :: "v"(pk[vs][w >> 1]));
          l1 += p[w];
        } else {
          l0 += p[w];
        }
        asm volatile("" :: "v"(l0), "v"(l1));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // The first score MFMA reads the bias block as its C operand over its whole
    // execution; an asm MFMA is opaque to the compiler's hazard checks, so keep
    // those registers out of reuse (e.g. by the other stream's bias formed in
    // this phase) until the phase is over.
    asm volatile("" :: "v"(biasb));
    s[ms] = acc;
    return l0 + l1;
  };
  // ---- one phase of the max-only pass: scores of the next step for stream MS,
  // the maximum of stream VS's step
  auto phase_max = [&](auto MSc, auto RELOAD, auto EXTRA, auto VEXTRA, uint32_t ks, int e, int half, bool live,
                       int cls)
      __attribute__((always_inline)) {
    constexpr int ms = decltype(MSc)::value;
    constexpr int vs = 1 - ms;
    static_for<20>([&](auto K) __attribute__((always_inline)) { EXTRA(K); });
    f32x16_t acc;
    static_for<kDqk / 16>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value;
      if constexpr (c == 0) mfma_s_first(cls, acc, kreg[c], qf[ms][c], biasb);
      else mfma_s<0>(acc, kreg[c], qf[ms][c], biasb);
      if constexpr (decltype(RELOAD)::value) kreg[c] = read_k(ks, c);
    });
    static_for<20>([&](auto K) __attribute__((always_inline)) { VEXTRA(K); });
    s_nop_after_mfma(acc);
    s[ms] = acc;
    if (live) {
      float x[16];
      masked_scores(IC<vs>{}, e, half, s[vs], x);
      m_run[vs] = fmaxf(m_run[vs], step_max(x));
    }
  };
  // ---- one phase: matrix work of stream MS and softmax of stream VS = 1 - MS
  // for the step at (entry e, half); the exact path follows when the step's tile
  // is slow (slow_tile) or a lane without a stabiliser sees a key in the step
  auto phase = [&](auto MSc, auto MODE, auto RELOAD, auto EXTRA, auto VEXTRA, uint32_t ks, uint32_t vsl, int e,
                   int half, bool live, int cls, bool slow_e)
      __attribute__((always_inline)) {
    constexpr int vs = 1 - decltype(MSc)::value;
    if constexpr (decltype(MODE)::value == kPassMax) {
      phase_max(MSc, RELOAD, EXTRA, VEXTRA, ks, e, half, live, cls);
    } else {
      const float lsum = phase_fast(MSc, RELOAD, EXTRA, VEXTRA, ks, vsl, cls);
      // the fast path's results are used on every path, so the compiler keeps it
      // in the scheduled block instead of moving it behind the test below
      asm volatile("" :: "v"(lsum), "v"(pk[vs][0]), "v"(pk[vs][1]), "v"(pk[vs][2]), "v"(pk[vs][3]), "v"(pk[vs][4]),
                   "v"(pk[vs][5]), "v"(pk[vs][6]), "v"(pk[vs][7]));
      // A fast step whose probabilities exceed the headroom (or are not
      // finite) is not redone here: l_max and l_run record it, and the pass's
      // end sends the item to the two-pass rerun, which recomputes every step
      // (the test costs one max per phase instead of a branch on fresh sums).
      // The fast step's sums are added without a branch (nothing for a step
      // past the end or one the exact path may redo); the exact path is the
      // only branch, rarely taken.
      const bool slow = slow_e || first[vs];
      const bool exact = live && slow;
      const float la = live && !slow ? lsum : 0.f;
      l_run[vs] += la;
      l_max[vs] = fmaxf(l_max[vs], la);
      if (__builtin_expect(exact, 0)) {
        // A lane without a stabiliser has the offset +FLT_MAX: its hidden keys
        // (score -inf) get probability 0 and a visible key an infinite one.
        // While such a lane sees nothing (a key run that starts past its row's
        // context) the fast step is exact for it (zeros), so a step of a fast
        // tile needs the exact path only where one of them sees a key (sum not
        // 0); that step sets its stabiliser.
        if (!slow_e && !__any(m_run[vs] == -INFINITY && !(lsum == 0.f))) {
          l_run[vs] += lsum;
          l_max[vs] = fmaxf(l_max[vs], lsum);
        } else {
          soft_exact(IC<vs>{}, e, half, s[vs], pk[vs]);
        }
      }
    }
  };

  // ---- one pass over the tile list (MODE: kPassNormal accumulates O and l,
  // kPassMax only the row maxima)
  auto run = [&](auto MODE) __attribute__((always_inline)) {
    // prologue: K(0..3), V(0..2), words of tiles 0, 1 land; scores of step 0 for
    // both streams and stream 0's softmax of step 0; V(0) and the first K(1)
    // chunks into registers
    int e0 = entry(0), e1 = entry(1), e2 = entry(2), e3 = entry(3);   // tiles T .. T+3
    issue_k(lds_k + 0 * kKSlot, key0_of(e0, 0));
    issue_k(lds_k + 1 * kKSlot, key0_of(e0, 1));
    issue_k(lds_k + 2 * kKSlot, key0_of(e1, 0));
    issue_k(lds_k + 3 * kKSlot, key0_of(e1, 1));
    issue_v(lds_v + 0 * kVSlot, key0_of(e0, 0));
    issue_v(lds_v + 1 * kVSlot, key0_of(e0, 1));
    issue_v(lds_v + 2 * kVSlot, key0_of(e1, 0));
    issue_bits(0, e0);
    issue_bits(kBitsSlot, e1);
    wait_vmem<0>();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      first[i] = __any(m_run[i] == -INFINITY);
      cbs[i] = stab_off(m_run[i]);
    }
    {
      const bool bin0 = eclass(e0) == 2;
      const f32x16_t b0 = bin0 ? bias_build(0, bias_word(IC<0>{}, 0)) : f32x16_t{};
      const f32x16_t b1 = bin0 ? bias_build(0, bias_word(IC<1>{}, 0)) : f32x16_t{};
      f32x16_t a0, a1;
      static_for<kDqk / 16>([&](auto C) __attribute__((always_inline)) {
        constexpr int c = decltype(C)::value;
        const bf16x8_t kop = read_k(0, c);
        mfma_s<c == 0 ? 1 : 0>(a0, kop, qf[0][c], b0);
        mfma_s<c == 0 ? 1 : 0>(a1, kop, qf[1][c], b1);
      });
      s_nop_after_mfma(a0);
      s_nop_after_mfma(a1);
      s[0] = a0;
      s[1] = a1;
    }
    if (nsteps > 0) {
      if (decltype(MODE)::value == kPassMax) {
        float x[16];
        masked_scores(IC<0>{}, e0, 0, s[0], x);
        m_run[0] = fmaxf(m_run[0], step_max(x));
      } else {
        soft_exact(IC<0>{}, e0, 0, s[0], pk[0]);
      }
    }
    bias_fix(1, e0, bias_word(IC<0>{}, 0));            // stream 0, step 1 (the first phase A)
#pragma unroll
    for (int op = 0; op < 8; ++op) vf[op] = read_v(0, op);
#pragma unroll
    for (int c = 0; c < kDqk / 16; ++c) kreg[c] = read_k(kKSlot, c);
    __syncthreads();

    // Tile T (entries e0 .. e3 = tiles T .. T+3), steps t = 2T + H (H = 0, 1).
    // K(s) lives in K slot s%4, V(s) in V slot s%3, the words of tile T in word
    // slot T%3; the slots are tracked as byte offsets (kpar = 2*kKSlot*(T&1),
    // vs0..vs2 = V slots of steps t, t+1, t+2, bs0..bs2 = word slots of tiles
    // T, T+1, T+2).  Registers on entry to step t: vf = V(t), kreg = K(t+1),
    // s[1] = stream 1's raw scores of step t, pk[0] = stream 0's P^T of step t.
    //   copies: K(t+4) into K(t)'s slot (read in step t-1), V(t+3) into V(t)'s
    //           slot (read into registers in step t-1) and, at H = 0, the
    //           words of tile T+2
    //   phase A: matrix of stream 0 (scores t+1 from K(t+1), PV t)
    //            || softmax of stream 1, step t
    //   phase B: matrix of stream 1 (scores t+1 from K(t+1), PV t; K(t+2)
    //            replaces kreg and V(t+1) replaces vf, register by register)
    //            || softmax of stream 0, step t+1
    //   then each wave waits for its copies of step t-1 and the workgroup
    //   synchronises: K(t+3), V(t+2) and their words are published, the slots
    //   read in step t are free.
    uint32_t kpar = 0;
    uint32_t vs0 = 0, vs1 = kVSlot, vs2 = 2 * kVSlot;
    uint32_t bs0 = 0, bs1 = kBitsSlot, bs2 = 2 * kBitsSlot;
    for (int T = 0; T < ntiles; ++T) {
      const bool slow0 = slow_tile(e0), slow1 = slow_tile(e1);
      auto step = [&](auto HC) __attribute__((always_inline)) {
        constexpr int H = decltype(HC)::value;
        const uint32_t kcopy = lds_k + kpar + H * kKSlot;               // K slot of steps t and t+4
        const uint32_t kread = (kpar ^ (2 * kKSlot)) + H * kKSlot;      // K slot of step t+2
        const int kkey = key0_of(e2, H);                                 // K(t+4)
        const int vkey = H ? key0_of(e2, 0) : key0_of(e1, 1);            // V(t+3)
        const int es1 = H ? e1 : e0;                                     // tile of step t+1
        const uint32_t vcopy = lds_v + vs0, vread = vs1;
        const uint32_t bcopy = bs2, bnext = H ? bs1 : bs0, bafter = bs1;  // word slots: T+2, tile of t+1, of t+2
        // copies of the step, one per MFMA slot: K(t+4) and (H = 0) the words of
        // tile T+2 in phase A, V(t+3) in phase B
        auto copies_a = [&](auto K) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value;
          if constexpr (k % 3 == 1 && k / 3 < 6) issue_k_piece(IC<k / 3>{}, kcopy, kkey);
          if constexpr (H == 0 && k == 18) issue_bits(bcopy, e2);
        };
        auto copies_b = [&](auto K) __attribute__((always_inline)) {
          constexpr int k = decltype(K)::value;
          if constexpr (k % 4 == 1 && k / 4 < 4) issue_v_piece(IC<k / 4>{}, vcopy, vkey);
        };
        // visibility words prefetched in the phases: stream 1's for step t+1
        // (phase B's scores) in phase A, stream 0's for step t+2 (the next phase
        // A) in phase B
        uint64_t w1, w0;
        auto bias_a = [&](auto K) __attribute__((always_inline)) { bias_slot(IC<1>{}, K, bnext, w1); };
        auto bias_b = [&](auto K) __attribute__((always_inline)) { bias_slot(IC<0>{}, K, bafter, w0); };
        const int cls = eclass(es1);   // class of the tile of step t+1, which both phases score
        // ---- phase A
        phase(IC<0>{}, MODE, std::false_type{}, copies_a, bias_a, kread, 0u, e0, H, true, cls, slow0);
        bias_fix(H ^ 1, es1, w1);
        // ---- phase B
        phase(IC<1>{}, MODE, std::true_type{}, copies_b, bias_b, kread, vread, es1, H ^ 1, H == 0 || T + 1 < ntiles,
              cls, H ? slow1 : slow0);
        bias_fix(H, e1, w0);
        // copies of step t-1 complete (those of step t may still be in flight)
        wait_vmem<H == 0 ? 11 : 10>();
        step_barrier();
        // phase B's operand reads (the next step's K and V) have landed by now;
        // one wait here replaces the compiler's countdown of a dozen waits in
        // front of phase A's MFMAs
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt / expcnt not waited
        const uint32_t tv = vs0;
        vs0 = vs1; vs1 = vs2; vs2 = tv;
      };
      step(IC<0>{});
      step(IC<1>{});
      const uint32_t tb = bs0;
      bs0 = bs1; bs1 = bs2; bs2 = tb;
      kpar ^= 2 * kKSlot;
      e0 = e1; e1 = e2; e2 = e3;
      e3 = entry(T + 4);
    }
    wait_vmem<0>();
  };

  run(IC<kPassNormal>{});
  // fast steps beyond the headroom, or non-finite sums (NaN and inf fail both tests)
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (!(l_max[i] <= kSumLimit) || !(l_run[i] <= 3.0e38f)) over = true;
  // Some row of the item rose more than the headroom above its stabiliser: both
  // waves take the second pass (row maxima, then the accumulation again with the
  // exact maxima as stabilisers, which no probability can exceed).
  {
    __syncthreads();
    int* const flag = reinterpret_cast<int*>(smem);
    if (threadIdx.x == 0) *flag = 0;
    __syncthreads();
    if (lane == 0 && __any(over)) *flag = 1;
    __syncthreads();
    const bool redo = *flag != 0;
    __syncthreads();
    if (__builtin_expect(redo, 0)) {
      m_run[0] = m_run[1] = -INFINITY;
      run(IC<kPassMax>{});
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        l_run[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][j][r] = 0.f;
      }
      run(IC<kPassNormal>{});
    }
  }

  // ---- normalise and store
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float l = halves_sum(l_run[i]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse_row = l > 0.f ? m_run[i] + __logf(l) : -INFINITY;
    if (a.part_o) {            // one run of a split row: bf16 partials for the combine
      const size_t prow = (static_cast<size_t>(sp) * a.B * a.H + bh) * a.Lq + q_row[i];
      if (q_ok[i] && hi == 0) a.part_lse[prow] = lse_row;
      if (q_ok[i]) {
        uint16_t* pp = a.part_o + prow * kDv;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2_t w2 = {pack_bf16x2(o[i][j][4 * g] * inv, o[i][j][4 * g + 1] * inv),
                                pack_bf16x2(o[i][j][4 * g + 2] * inv, o[i][j][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2_t*>(pp + 32 * j + 8 * g + 4 * hi) = w2;
          }
      }
      continue;
    }
    if (a.lse && q_ok[i] && hi == 0) a.lse[bh * a.Lq + q_row[i]] = lse_row;
    if (q_ok[i]) {
      uint16_t* op = a.out + (bh * a.Lq + q_row[i]) * kDv;
      // o[i][j][r] holds dv = 32*j + 8*(r>>2) + 4*hi + (r&3)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2_t w2 = {pack_bf16x2(o[i][j][4 * g] * inv, o[i][j][4 * g + 1] * inv),
                              pack_bf16x2(o[i][j][4 * g + 2] * inv, o[i][j][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(op + 32 * j + 8 * g + 4 * hi) = w2;
        }
    }
  }
}

// Merge of the split runs of every row: with w_s = exp(lse_s - max lse),
// out = sum_s w_s o_s / sum_s w_s and lse = max + log(sum_s w_s), summed in split
// order (deterministic).  A row whose runs are all empty gives 0 and -inf.
// One thread per 4 output columns, 32 threads per row.
constexpr int kMaxRuns = 8;          // key runs per row (the split heuristic's cap)

__global__ void __launch_bounds__(256) attn_combine(AttnCombineArgs a) {
  // 16 lanes per row, 8 dims (16 bytes) per lane.  Every run's normaliser and
  // partial are loaded up front (one memory round trip), then merged in run
  // order.
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (row >= a.rows) return;
  const int d = (threadIdx.x & 15) * 8;
  float ls[kMaxRuns];
  u32x4_t ob[kMaxRuns];
#pragma unroll
  for (int sp = 0; sp < kMaxRuns; ++sp) {
    ls[sp] = -INFINITY;
    ob[sp] = u32x4_t{0u, 0u, 0u, 0u};
    if (sp < a.nsplit) {
      ls[sp] = a.part_lse[sp * a.rows + row];
      ob[sp] = *reinterpret_cast<const u32x4_t*>(a.part_o + (sp * a.rows + row) * kDv + d);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxRuns; ++sp) mx = fmaxf(mx, ls[sp]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxRuns; ++sp) {
      if (ls[sp] == -INFINITY) continue;              // also every run past nsplit
      const float w = __builtin_amdgcn_exp2f((ls[sp] - mx) * kLog2e);
      wsum += w;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = __builtin_fmaf(w, __uint_as_float(ob[sp][c] << 16), acc[2 * c]);
        acc[2 * c + 1] = __builtin_fmaf(w, __uint_as_float(ob[sp][c] & 0xFFFF0000u), acc[2 * c + 1]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const u32x4_t w4 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                      pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4_t*>(a.out + row * kDv + d) = w4;
  if (a.lse && d == 0) a.lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_combine(const AttnCombineArgs& a, hipStream_t s) {
  if (a.nsplit < 1 || a.nsplit > kMaxRuns) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>((a.rows + 15) / 16);
  hipLaunchKernelGGL(attn_combine, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnBf16Args& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.nqt * a.H * a.nsplit;
  if (!a.counts)
    hipLaunchKernelGGL((attn_fwd_bf16<false, false>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.mask && a.mask_bf16)
    hipLaunchKernelGGL((attn_fwd_bf16<true, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16<false, true>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
