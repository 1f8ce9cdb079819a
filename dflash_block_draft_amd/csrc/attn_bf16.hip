// Fused non-causal draft MLA attention forward, bf16 MFMA on gfx950.
//
// What it computes (NeMo AutoModel DFlash page, KimiK3DFlashAttention.forward;
// DSpark page, KimiK3DSparkAttention): for every (batch, head, noise query)
//   s_j = scale * (q_nope . k_nope[h][j] + q_rope . k_rope[j]) + mask[i][j]
//   out = softmax_j(s) @ v[h]
// over the keys [context | noise block], with no materialised score matrix.
//
// Decomposition (one workgroup = one (batch, head, 128-query tile)):
//  * 8 waves, two per SIMD: wave w owns queries 32*(w&3) .. +31 of the tile
//    and keys 32*(w>>2) .. +31 of every 64-key tile; the two key-half waves of
//    a query group keep separate (m, l, O) and merge them once at the end.
//  * Ping-pong: each wave alternates a matrix phase (score MFMAs of the next
//    tile + PV MFMAs of the current one) and a vector phase (softmax of the
//    next tile), with a workgroup barrier after every phase.  The key-half-1
//    waves run one phase behind the key-half-0 waves, so on every SIMD (waves
//    w and w+4) one wave feeds the matrix core while the other does its
//    exponentials.
//  * Scores are computed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16:
//    a lane holds one query and 16 of its keys, so row sums are in-lane, and
//    the packed bf16 P^T values are directly the B operand of O^T = V^T P^T
//    (the key order of the contraction is free, so keys are relabelled to
//    match the accumulator layout).  V^T operands come from the V tile with
//    the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//  * K = [k_nope | head-shared k_rope], V and the visibility words go global ->
//    LDS with buffer_load ... lds (no VGPR staging; out-of-range reads give
//    zeros) into three-slot rings; every copy has two phases of slack before
//    the barrier that publishes it.  The key loop is unrolled by the ring
//    length so every LDS address and copy destination is a constant.  LDS
//    tiles are 16-row x 64 B blocks with XOR-swizzled K chunks: conflict-free
//    operand reads, 64-byte coalesced loads.
//  * Q (32 x 192 bf16 per wave) stays in registers for the whole key loop; the
//    K operands of the next score tile are read into registers at the end of
//    the vector phase, so the matrix phase starts on data already there.
//  * Binary-mask tiles (only 0 / -inf) initialise the score accumulator to
//    0 / -inf from a 64-bit visibility word per query, so the MFMA applies the
//    mask; general masks add their values to the scaled scores.
//  * Online softmax in fp32 with the hardware exp2 and a stabiliser m that is
//    only raised when needed: the probabilities of a tile are first formed
//    with the current m; if some lane's tile sum exceeds 2^8 (or m is still
//    -inf) the wave takes the exact path (tile max, rescale of O and l by
//    exp(m_old - m_new), recompute).  Any stabiliser gives the same result in
//    exact arithmetic because it scales O and l alike.
#include "common.h"
#include "dma.h"
#include "launch.h"

#include <type_traits>

namespace dflash {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKBytes = kTileN * kDqk * 2;          // 24 KiB: 4 row blocks x 6 chunk quads x 1 KiB
constexpr int kVBytes = kTileN * kDv * 2;           // 16 KiB: 4 row blocks x 4 chunk quads x 1 KiB
constexpr int kBitsBytes = kTileM * 8;              // 1 KiB: one visibility word per query
constexpr int kKRingN = 4;                           // K and visibility-word rings: copies lead by 2.5 tiles
constexpr int kVRingN = 3;                           // V ring: copies lead by 2 tiles
constexpr int kKRing = 0;
constexpr int kVRing = kKRing + kKRingN * kKBytes;
constexpr int kBitsRing = kVRing + kVRingN * kVBytes;
constexpr int kRingBytes = kBitsRing + kKRingN * kBitsBytes;
static_assert(kRingBytes <= 160 * 1024, "LDS budget");
constexpr int kPrefetchK = 8;                        // K operand chunks read before the matrix phase
constexpr float kSumLimit = 256.0f;                  // fast path keeps every probability <= 2^8
constexpr uint32_t kNegInfBits = 0xFF800000u;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
typedef __attribute__((address_space(3))) char lds_char_t;

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

// LDS tile layout (K and V): row block rb (16 rows) x chunk quad cq (4 x 16 B
// chunks) -> 1 KiB block (rb * nq + cq); inside it row r%16 takes 64 B and the
// 16-byte chunk c%4 of that row sits at slot (c%4) ^ swz(r), swz(r) = (r>>2)&3
// for K and 0 for V.  Wave w copies, of each tile, row block w/2 of K: the
// k_nope quads 2(w%2), 2(w%2)+1 (adjacent blocks) and the k_rope quad 4 + w%2,
// and V blocks 2w, 2w+1; lane l of a block covers row rb*16 + l/4, slot l%4.
struct TileCopy {
  u32x4_t kn, kr, v, bits;     // descriptors: this (b, h)'s k_nope, the shared k_rope, v, visibility words
  uint32_t voff[4];            // per-lane byte offset inside the source rows (tile start excluded)
  uint32_t kn_lds, kr_lds, v_lds;   // LDS address of this wave's k_nope pair / k_rope / V pair in slot 0
};

__device__ __forceinline__ u32x4_t uniform4(u32x4_t d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_amdgcn_readfirstlane(d[i]);
  return d;
}

template <bool MASK_BF16>
__device__ __forceinline__ float load_mask(const void* mask, size_t idx) {
  if (MASK_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(mask)[idx]);
  return static_cast<const float*>(mask)[idx];
}

template <int N>
using IC = std::integral_constant<int, N>;

template <bool MASK_BF16>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_bf16(AttnBf16Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[kRingBytes];
  lds_char_t* const lds = (lds_char_t*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: keeps descriptors scalar
  const int qg = wave & 3;      // query group: 32 queries
  const int kh = wave >> 2;     // key half of each 64-key tile; also the ping-pong group
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
  const int n_all = a.counts ? a.counts[bq] : a.nkt;
  const int t_begin = static_cast<int>(static_cast<int64_t>(n_all) * sp / a.nsplit);
  const int ntiles = static_cast<int>(static_cast<int64_t>(n_all) * (sp + 1) / a.nsplit) - t_begin;

  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int q_local = qg * 32 + li;               // this lane's query within the tile
  const int q_row = qt * kTileM + q_local;
  const bool q_ok = q_row < a.Lq;
  const size_t tile_row0 = static_cast<size_t>(bq) * a.nkt;

  // ---- tile list of this q-tile (entry: k-tile | class << 24), read with scalar
  // loads; past the end an entry is 0 (no tile); without a mask every k-tile is class 1
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const int32_t* list = a.counts ? a.lists + tile_row0 + t_begin : nullptr;
  const const_i32* clist = (const const_i32*)(uintptr_t)(list);
  auto entry = [&](int i) __attribute__((always_inline)) -> int {
    if (i >= ntiles) return 0;
    if (!list) return (t_begin + i) | (1 << 24);
    return clist[i];
  };

  // ---- global -> LDS copy plan of this wave
  TileCopy tc;
  tc.kn = buffer_desc(a.kn + bh * a.Lk * kDn, a.Lk * kDn * 2);
  tc.kr = buffer_desc(a.kr + static_cast<size_t>(b) * a.Lk * kDr, a.Lk * kDr * 2);
  tc.v = buffer_desc(a.v + bh * a.Lk * kDv, a.Lk * kDv * 2);
  tc.bits = buffer_desc(a.bits ? a.bits + tile_row0 * kTileM : nullptr, a.bits ? a.nkt * kBitsBytes : 0);
  {
    const int r16 = lane >> 2, s4 = lane & 3;
    const int krb = wave >> 1;                                   // K row block of this wave
    const int krow = krb * 16 + r16;
    const int kslot = s4 ^ ((r16 >> 2) & 3);                     // swizzled 16-byte chunk in the quad
#pragma unroll
    for (int i = 0; i < 2; ++i)                                  // k_nope quads 2(w%2) + i: dims 64(w%2) + 32i ..
      tc.voff[i] = krow * (kDn * 2) + ((2 * (wave & 1) + i) * 4 + kslot) * 16;
    tc.voff[2] = krow * (kDr * 2) + ((wave & 1) * 4 + kslot) * 16;   // k_rope quad 4 + w%2
    tc.kn_lds = lds0 + kKRing + (krb * 6 + 2 * (wave & 1)) * 1024;
    tc.kr_lds = lds0 + kKRing + (krb * 6 + 4 + (wave & 1)) * 1024;
    // V blocks 2w, 2w+1 of 16 (4 row blocks x 4 quads): row block w/2, quads 2(w%2) + i
    const int vrow0 = (wave >> 1) * 16 + r16;
    tc.voff[3] = vrow0 * (kDv * 2) + (2 * (wave & 1) * 4 + s4) * 16;   // second block is +64 B in the row
    tc.v_lds = lds0 + kVRing + 2 * wave * 1024;
  }
  // Tiles past the end use k0 = Lk: every lane's read is out of range (zeros, no
  // traffic), so every wave always issues the same number of copies and the
  // wait counts are constants.
  auto k0_of = [&](int e) __attribute__((always_inline)) -> int { return (e >> 24) ? (e & 0xFFFFFF) * kTileN : a.Lk; };
  auto bits_kt = [&](int e) __attribute__((always_inline)) -> int { return (e >> 24) == 2 ? (e & 0xFFFFFF) : a.nkt; };
  auto issue_k = [&](uint32_t slot_off, int k0) __attribute__((always_inline)) {
    dma16<0>(tc.kn, tc.kn_lds + slot_off, tc.voff[0], k0 * (kDn * 2));
    dma16<1024>(tc.kn, tc.kn_lds + slot_off, tc.voff[1], k0 * (kDn * 2));
    dma16<0>(tc.kr, tc.kr_lds + slot_off, tc.voff[2], k0 * (kDr * 2));
  };
  auto issue_v = [&](uint32_t slot_off, int k0) __attribute__((always_inline)) {
    dma16<0>(tc.v, tc.v_lds + slot_off, tc.voff[3], k0 * (kDv * 2));
    dma16<1024>(tc.v, tc.v_lds + slot_off, tc.voff[3] + 64, k0 * (kDv * 2));
  };
  // visibility words of a class-2 tile (1 KiB, copied by wave 0); kt = nkt reads zeros
  auto issue_bits = [&](uint32_t slot_off, int kt) __attribute__((always_inline)) {
    if (wave == 0) dma16<kBitsRing>(tc.bits, lds0 + slot_off, lane * 16, kt * kBitsBytes);
  };

  // ---- per-lane LDS read offsets (bytes inside a slot)
  // K operand of chunk c (dims 16c .. 16c+15): 16-byte chunk 2c+hi of row kh*32+li
  // -> block (rb*6 + c/2), slot (2*(c&1) + hi) ^ swz(row).
  const int krow = kh * 32 + li;
  const int kq = (li >> 2) & 3;
  const int k_even = ((krow >> 4) * 6) * 1024 + (krow & 15) * 64 + (hi ^ kq) * 16;
  const int k_odd = ((krow >> 4) * 6) * 1024 + (krow & 15) * 64 + ((2 + hi) ^ kq) * 16;
  // V^T operand (transposing read): lane i of 16-lane group G addresses row
  // kh*32 + 16*step + 4*hi + i/4 (+8), dims 32*j + 16*(G&1) + 4*(i&3).
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vrow = kh * 32 + 4 * hi + (i16 >> 2);
  const int v_base = ((vrow >> 4) * 4) * 1024 + (vrow & 15) * 64 + (2 * (g16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8;
  const lds_char_t* const ke_ptr = lds + kKRing + k_even;
  const lds_char_t* const ko_ptr = lds + kKRing + k_odd;
  const lds_char_t* const v_ptr = lds + kVRing + v_base;
  const lds_u64_t* const bits_ptr = reinterpret_cast<const lds_u64_t*>(lds + kBitsRing + q_local * 8);

  // ---- Q fragments (B operand of S^T = K Q^T): 12 chunks of 16 dims
  bf16x8_t qf[kDqk / 16];
  {
    const uint16_t* qp = a.q + (bh * a.Lq + (q_ok ? q_row : 0)) * kDqk + 8 * hi;
#pragma unroll
    for (int c = 0; c < kDqk / 16; ++c) {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      qf[c] = as_bf16x8(q_ok ? ldg16(qp + 16 * c) : z);
    }
  }

  f32x16_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m_run = -INFINITY;   // stabiliser (natural units), same in both lane halves
  float l_run = 0.f;         // this lane's partial row sum

  const float scale = a.scale;
  const float scale_log2 = a.scale * kLog2e;
  const size_t mask_row = (static_cast<size_t>(b) * a.Lq + (q_ok ? q_row : 0)) * a.Lk;

  f32x16_t s;                    // scores of the tile between its matrix and vector phases
  bf16x8_t kf[kDqk / 16];        // K operands of the next score tile
  uint32_t pk[8];                // P^T of the tile awaiting PV, bf16 pairs

  // K operand chunks [C0, C1) of ring slot SL into registers
  auto read_k = [&](uint32_t slot_off, auto C0, auto C1) __attribute__((always_inline)) {
#pragma unroll
    for (int c = decltype(C0)::value; c < decltype(C1)::value; ++c) {
      const lds_char_t* kp = ((c & 1) ? ko_ptr : ke_ptr) + slot_off + (c >> 1) * 1024;
      kf[c] = as_bf16x8(*reinterpret_cast<const lds_u32x4_t*>(kp));
    }
  };
  // First K operands of ring slot SL (the rest are read in the matrix phase, behind
  // the first MFMAs); for a binary tile also its hidden-key word, applied to the
  // scores in the vector phase.
  uint32_t hid_next = 0, hid = 0;   // bit 8g+c <-> key kh*32+8g+4hi+c of the tile is hidden
  auto load_k = [&](int slot, int e) __attribute__((always_inline)) {
    read_k(slot * kKBytes, IC<0>{}, IC<kPrefetchK>{});
    if ((e >> 24) == 2) {
      const uint64_t w64 = bits_ptr[slot * (kBitsBytes / 8)];
      hid_next = ~static_cast<uint32_t>(w64 >> (kh * 32 + 4 * hi));
    }
  };
  auto score_mfma = [&]() __attribute__((always_inline)) {
    const f32x16_t z = {};
    s = mfma32(kf[0], qf[0], z);
#pragma unroll
    for (int c = 1; c < kDqk / 16; ++c) s = mfma32(kf[c], qf[c], s);
  };
  // O^T += V^T P^T over this wave's 32 keys (two 16-key MFMA steps).  B operand
  // element e of lane (li, hi) is key 8*(e>>2) + 4*hi + (e&3) of the step; the
  // transposing reads deliver V[that key][32*j + li] as A operand.
  s16x8_t av[2][4];              // V^T operands of the tile awaiting PV
  auto read_v = [&](uint32_t slot_off) __attribute__((always_inline)) {
#pragma unroll
    for (int step = 0; step < 2; ++step)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const lds_char_t* vp = v_ptr + slot_off + step * 4096 + j * 1024;
        const s16x4_t lo = ds_read_tr(vp);
        const s16x4_t hi4 = ds_read_tr(vp + 512);
        av[step][j] = s16x8_t{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
  };
  auto pv_mfma = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const u32x4_t pb = {pk[4 * step + 0], pk[4 * step + 1], pk[4 * step + 2], pk[4 * step + 3]};
      const bf16x8_t bfr = as_bf16x8(pb);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = mfma32(__builtin_bit_cast(bf16x8_t, av[step][j]), bfr, o[j]);
    }
  };
  // p = exp2(fma(x, ca, cb)) -> pk (bf16 pairs); returns the lane's sum of p.  The sum
  // uses plain fp32 adds: v_dot2 would wait for the matrix core, which the other
  // wave of the SIMD keeps busy during this phase.
  auto probs = [&](const float* x, float ca, float cb) __attribute__((always_inline)) -> float {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], ca, cb));
#pragma unroll
    for (int u = 0; u < 8; ++u) pk[u] = pack_bf16x2(p[2 * u], p[2 * u + 1]);
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      l0 += p[r];
      l1 += p[r + 1];
    }
    return l0 + l1;
  };
  // Vector phase: softmax of the raw scores in s (tile entry e) -> pk, m_run, l_run, o.
  // Fast path (zero or binary tile, no ragged end): probabilities with the
  // current stabiliser, hidden keys set to -inf first.  Exact path (general mask,
  // ragged end, no stabiliser yet, or a probability that may exceed 2^8): masked
  // natural-unit scores, tile max, rescale of O and l when the stabiliser rises,
  // probabilities.
  auto softmax = [&](int e) __attribute__((always_inline)) {
    const int cls = e >> 24;
    const int k0 = (e & 0xFFFFFF) * kTileN;
    const bool ragged = k0 + kTileN > a.Lk;
    float lsum = 0.f;
    bool exact = true;
    // (a lane with no stabiliser yet takes the exact path: skip the fast attempt)
    if ((cls == 1 || cls == 2) && !ragged && !__any(m_run == -INFINITY)) {
      // hidden keys of a binary tile become -inf, whose probability is exactly 0
      float x[16];
      if (cls == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int h1 = __builtin_amdgcn_sbfe(static_cast<int>(hid), 8 * (r >> 2) + (r & 3), 1);   // -1: hidden
          x[r] = __int_as_float((h1 & static_cast<int>(kNegInfBits)) | (~h1 & __float_as_int(s[r])));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = s[r];
      }
      lsum = probs(x, scale_log2, -(m_run == -INFINITY ? 0.f : m_run) * kLog2e);
      exact = __any(!(lsum <= kSumLimit));   // NaN sums too
    }
    if (__builtin_expect(exact, 0)) {
      // accumulator r <-> key k0 + kh*32 + 8*(r>>2) + 4*hi + (r&3)
      const int kbase = k0 + kh * 32 + 4 * hi;
      float x[16];
      if (cls == 3 && a.mask) {   // (a reused map without its mask: no values to add)
        // general mask values: x = scale*qk + mask
        float mv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {   // all 16 loads in flight together (clamped index, fixed below)
          const int kk = kbase + 8 * (r >> 2) + (r & 3);
          mv[r] = load_mask<MASK_BF16>(a.mask, mask_row + min(kk, a.Lk - 1));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], scale, q_ok ? mv[r] : 0.f);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = s[r] * scale;
        if (cls == 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int h1 = __builtin_amdgcn_sbfe(static_cast<int>(hid), 8 * (r >> 2) + (r & 3), 1);   // -1: hidden
            x[r] = __int_as_float((h1 & static_cast<int>(kNegInfBits)) | (~h1 & __float_as_int(x[r])));
          }
        }
      }
      if (ragged) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 8 * (r >> 2) + (r & 3) >= a.Lk) x[r] = -INFINITY;
      }
      float tmax = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, x[r]);
      const float m_new = fmaxf(m_run, halves_max(tmax));
      if (__any(m_new != m_run)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
        l_run *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
        m_run = m_new;
      }
      // subtract before scaling: m * log2e can overflow where x - m does not (mask values near -FLT_MAX)
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] -= m_use;
      lsum = probs(x, kLog2e, 0.f);
    }
    l_run += lsum;
  };

  // ---- prologue: K(0..3), bits(0..3), V(0..1) land before anyone reads
  int e0 = entry(0), e1 = entry(1), e2 = entry(2), e3 = entry(3), e4 = entry(4);   // tiles t .. t+4
  int e5 = entry(5);
  issue_k(0 * kKBytes, k0_of(e0));
  issue_k(1 * kKBytes, k0_of(e1));
  issue_k(2 * kKBytes, k0_of(e2));
  issue_k(3 * kKBytes, k0_of(e3));
  issue_v(0 * kVBytes, k0_of(e0));
  issue_v(1 * kVBytes, k0_of(e1));
  issue_bits(0 * kBitsBytes, bits_kt(e0));
  issue_bits(1 * kBitsBytes, bits_kt(e1));
  issue_bits(2 * kBitsBytes, bits_kt(e2));
  issue_bits(3 * kBitsBytes, bits_kt(e3));
  wait_vmem<0>();
  __syncthreads();

  // Phase schedule (every phase ends with a workgroup barrier):
  //   key half 0:  S(0) | V(0) | M(0) | V(1) | M(1) | ... | M(T-1) | idle
  //   key half 1:  idle | S(0) | V(0) | M(0) | V(1) | ... | V(T-1) | M(T-1)
  // M(t) = scores of tile t+1 and PV of tile t; V(t) = softmax of tile t.
  // Tile u lives in K / bits slot u%4 and V slot u%3.  Copies of K(t+4),
  // bits(t+4) and V(t+2) are issued at the start of the phase both halves run
  // in slot 2t+2 (half 0: M(t), half 1: V(t)): the slots they overwrite were
  // last read in slot 2t+1.  Each wave waits for its own copies before the
  // barrier that precedes their first read: K(t+2), bits(t+2) at the end of
  // slot 2t+2 (first read in slot 2t+3), V(t+1) at the end of slot 2t+3.
  if (kh == 1) __syncthreads();
  load_k(0, e0);
  read_k(0, IC<kPrefetchK>{}, IC<kDqk / 16>{});
  score_mfma();
  hid = hid_next;
  __syncthreads();

  int v3 = 0;                                      // t % 3
  for (int it = 0; it < ntiles; ++it) {
    const int k4 = it & 3;                         // K / bits slot of tile it (and it+4)
    const int k4n = (it + 1) & 3;                  // K / bits slot of tile it+1
    const int v3n2 = v3 == 0 ? 2 : v3 - 1;         // V slot of tile it+2
    const int e_next = e5;
    e5 = entry(it + 6);
    auto issue_copies = [&]() __attribute__((always_inline)) {
      issue_k(k4 * kKBytes, k0_of(e4));
      issue_bits(k4 * kBitsBytes, bits_kt(e4));
      issue_v(v3n2 * kVBytes, k0_of(e2));
    };
    // ---- vector phase: K operands of tile it+1, softmax of tile it
    if (it + 1 < ntiles) load_k(k4n, e1);
    if (kh == 1) issue_copies();
    softmax(e0);
    if (kh == 0) {            // V(it): issued three phases ago, five (six) copies since
      if (wave == 0) wait_vmem<6>(); else wait_vmem<5>();
    } else {                  // K(it+2): twelve copies since
      wait_vmem<12>();
    }
    __syncthreads();
    // ---- matrix phase: scores of tile it+1 (after the last tile they score stale
    // data and are never used), PV of tile it.  The remaining K operands and all V
    // operands are requested before the first MFMA; the first eight score MFMAs run
    // on operands already in registers while they arrive.
    if (kh == 0) issue_copies();
    read_k(k4n * kKBytes, IC<kPrefetchK>{}, IC<kDqk / 16>{});
    read_v(v3 * kVBytes);
    __builtin_amdgcn_sched_barrier(0);
    score_mfma();
    pv_mfma();
    if (kh == 0) {            // K(it+2), bits(it+2): twelve (fourteen) copies since
      if (wave == 0) wait_vmem<14>(); else wait_vmem<12>();
    } else {                  // V(it+1): five copies since
      wait_vmem<5>();
    }
    __syncthreads();
    e0 = e1; e1 = e2; e2 = e3; e3 = e4; e4 = e_next;
    hid = hid_next;
    v3 = v3 == 2 ? 0 : v3 + 1;
  }
  if (kh == 0) __syncthreads();
  wait_vmem<0>();

  // ---- merge the two key halves of each query group, normalise, store
  l_run = halves_sum(l_run);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + qg * (64 * 66);   // O[16][4][64] + m[64] + l[64]
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[(r * 4 + j) * 64 + lane] = o[j][r];
    red[64 * 64 + lane] = m_run;
    red[65 * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = red[64 * 64 + lane];
    const float l1 = red[65 * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m) * kLog2e);
    const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * kLog2e);
    const float l = l_run * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse_row = l > 0.f ? m + __logf(l) : -INFINITY;
    if (a.part_o) {            // one run of a split row: fp32 partials for the combine
      const size_t prow = (static_cast<size_t>(sp) * a.B * a.H + bh) * a.Lq + q_row;
      if (q_ok && hi == 0) a.part_lse[prow] = lse_row;
      if (q_ok) {
        float* pp = a.part_o + prow * kDv;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4_t x;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int r = 4 * g + c;
              x[c] = (o[j][r] * a0 + red[(r * 4 + j) * 64 + lane] * a1) * inv;
            }
            *reinterpret_cast<f32x4_t*>(pp + 32 * j + 8 * g + 4 * hi) = x;
          }
      }
      return;
    }
    if (a.lse && q_ok && hi == 0) a.lse[bh * a.Lq + q_row] = lse_row;
    if (q_ok) {
      uint16_t* op = a.out + (bh * a.Lq + q_row) * kDv;
      // o[j][r] holds dv = 32*j + 8*(r>>2) + 4*hi + (r&3)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float x[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * g + c;
            x[c] = (o[j][r] * a0 + red[(r * 4 + j) * 64 + lane] * a1) * inv;
          }
          const u32x2_t w2 = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          *reinterpret_cast<u32x2_t*>(op + 32 * j + 8 * g + 4 * hi) = w2;
        }
    }
  }
}

// Merge of the split runs of every row: with w_s = exp(lse_s - max lse),
// out = sum_s w_s o_s / sum_s w_s and lse = max + log(sum_s w_s), summed in split
// order (deterministic).  A row whose runs are all empty gives 0 and -inf.
// One thread per 4 output columns, 32 threads per row.
__global__ void __launch_bounds__(256) attn_combine(AttnCombineArgs a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (row >= a.rows) return;
  const int d = (threadIdx.x & 31) * 4;
  float mx = -INFINITY;
  for (int sp = 0; sp < a.nsplit; ++sp) mx = fmaxf(mx, a.part_lse[sp * a.rows + row]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float ls = a.part_lse[sp * a.rows + row];
      if (ls == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((ls - mx) * kLog2e);
      const f32x4_t o = *reinterpret_cast<const f32x4_t*>(a.part_o + (sp * a.rows + row) * kDv + d);
      wsum += w;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(w, o[c], acc[c]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const u32x2_t w2 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2_t*>(a.out + row * kDv + d) = w2;
  if (a.lse && d == 0) a.lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_combine(const AttnCombineArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.rows + 7) / 8);
  hipLaunchKernelGGL(attn_combine, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnBf16Args& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.nqt * a.H * a.nsplit;
  if (a.mask && a.mask_bf16)
    hipLaunchKernelGGL(attn_fwd_bf16<true>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16<false>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
