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
//    and keys 32*(w>>2) .. +31 of every 64-key tile; the two waves of a query
//    group merge (m, l, O) once at the end.
//  * Each wave is software-pipelined: in iteration i it runs the score MFMAs of
//    tile i+1 in the same basic block as the softmax and PV of tile i, so the
//    MFMA pipe and the VALU work at the same time within a wave (and across
//    the two waves of a SIMD).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane holds one query and 16 of its keys, so row max / row sum are
//    in-lane (plus one v_permlane32_swap), and the lane's P^T values are
//    already the B operand of O^T = V^T P^T for the same key order (the order
//    of the key contraction is free, so keys are relabelled to match the
//    accumulator layout).  V^T operands come straight from the V tile with the
//    gfx950 transposing LDS read (ds_read_b64_tr_b16).
//  * K = [k_nope | head-shared k_rope], V and the visibility words go global ->
//    LDS with buffer_load ... lds (no VGPR staging; out-of-range reads give
//    zeros).  K and V have separate three-slot rings: K of tile i+1 is read in
//    iteration i, V of tile i too, so issuing K(i+3) and V(i+2) in iteration i
//    gives every copy two iterations to land, with one barrier per tile.  LDS
//    tiles are 16-row x 64 B blocks with XOR-swizzled K chunks: conflict-free
//    operand reads, 64-byte coalesced loads, immediate offsets.
//  * Q (32 x 192 bf16 per wave) stays in registers for the whole key loop.
//  * Binary-mask tiles (only 0 / -inf) initialise the score accumulator to
//    0 / -inf from a 64-bit visibility word per query, so the MFMA applies the
//    mask; general masks add their values to the scaled scores.
//  * Online softmax in fp32 with the hardware exp2; the running max is only
//    raised when a new score exceeds it by more than 2^8 in probability space
//    ("lazy rescale"), exact because the same max scales both O and l.  The
//    row sum adds the bf16-rounded probabilities (v_dot2), the same values the
//    PV MFMA consumes.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKBytes = kTileN * kDqk * 2;          // 24 KiB: 4 row blocks x 6 chunk quads x 1 KiB
constexpr int kVBytes = kTileN * kDv * 2;           // 16 KiB: 4 row blocks x 4 chunk quads x 1 KiB
constexpr int kBitsBytes = kTileM * 8;              // 1 KiB: one visibility word per query
constexpr int kRing = 3;
constexpr int kKRing = 0;
constexpr int kVRing = kKRing + kRing * kKBytes;
constexpr int kBitsRing = kVRing + kRing * kVBytes;
constexpr int kRingBytes = kBitsRing + kRing * kBitsBytes;
static_assert(kRingBytes + 4 * kLdsListMax <= 160 * 1024, "LDS budget");
constexpr float kLazyTau = 8.0f / kLog2e;            // natural-units slack before a rescale
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

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt left at their no-wait maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16*lane; reads past
// the descriptor's num_records return zeros.  Issued as inline asm so the compiler
// does not treat the in-flight LDS write as a dependency of unrelated LDS reads
// (it would otherwise wait for it before every ds_read); completion is awaited
// explicitly (wait_vmem) before the barrier that publishes the slot.  No memory
// clobber: the slot it writes is not read before that barrier.
__device__ __forceinline__ void dma16(u32x4_t rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr));
}

__device__ __forceinline__ u32x4_t buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4_t d = {static_cast<uint32_t>(p), static_cast<uint32_t>(p >> 32) & 0xFFFFu, bytes, 0x00020000u};
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_amdgcn_readfirstlane(d[i]);
  return d;
}

// LDS tile layout (K and V): row block rb (16 rows) x chunk quad cq (4 x 16 B
// chunks) -> 1 KiB block (rb * nq + cq); inside it row r%16 takes 64 B and the
// 16-byte chunk c%4 of that row sits at slot (c%4) ^ swz(r), swz(r) = (r>>2)&3
// for K and 0 for V.  A wave copies 3 K blocks and 2 V blocks of each tile;
// lane l of a block covers row rb*16 + l/4 and slot l%4.
struct TileCopy {
  u32x4_t kdesc[3], v, bits;   // descriptors (k_nope or k_rope slice per K block)
  uint32_t voff[5];            // per-lane byte offset inside the source slice (tile start excluded)
  uint32_t lds_off[5];         // block offset inside a K / V slot
  int krow_bytes[3];           // source row pitch of each K block (k_nope 256 B, k_rope 128 B)
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

template <bool MASK_BF16>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_bf16(AttnBf16Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[kRingBytes];
  __shared__ int s_list[kLdsListMax];
  lds_char_t* const lds = (lds_char_t*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: keeps descriptors scalar
  const int qg = wave & 3;      // query group: 32 queries
  const int kh = wave >> 2;     // key half of each 64-key tile
  const int li = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: heads of one (batch, q-tile) are adjacent in launch order
  const int h = blockIdx.x % a.H;
  const int rank = blockIdx.x / a.H;
  const int bq = a.order ? a.order[rank] : rank;
  const int b = bq / a.nqt;
  const int qt = bq % a.nqt;
  const int ntiles = a.counts ? a.counts[bq] : a.nkt;

  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int q_local = qg * 32 + li;               // this lane's query within the tile
  const int q_row = qt * kTileM + q_local;
  const bool q_ok = q_row < a.Lq;
  const size_t tile_row0 = static_cast<size_t>(bq) * a.nkt;

  // ---- tile list of this q-tile -> LDS (entry: k-tile | class << 24); host caps ntiles
  const int32_t* list = a.counts ? a.lists + tile_row0 : nullptr;
  if (list)
    for (int i = t; i < ntiles; i += kThreads) s_list[i] = list[i];

  // ---- global -> LDS copy plan of this wave
  TileCopy tc;
  const u32x4_t kn_desc = buffer_desc(a.kn + bh * a.Lk * kDn, a.Lk * kDn * 2);
  const u32x4_t kr_desc = buffer_desc(a.kr + static_cast<size_t>(b) * a.Lk * kDr, a.Lk * kDr * 2);
  tc.v = buffer_desc(a.v + bh * a.Lk * kDv, a.Lk * kDv * 2);
  tc.bits = buffer_desc(a.bits ? a.bits + tile_row0 * kTileM : nullptr, a.bits ? a.nkt * kBitsBytes : 0);
  {
    const int r16 = lane >> 2, s4 = lane & 3;
#pragma unroll
    for (int i = 0; i < 3; ++i) {            // K blocks 3w .. 3w+2 of 24 (4 row blocks x 6 quads)
      const int blk = 3 * wave + i, rb = blk / 6, cq = blk % 6;
      const int row = rb * 16 + r16;
      const int chunk = cq * 4 + (s4 ^ ((r16 >> 2) & 3));
      const bool rope = cq >= 4;                                  // chunks 16..23: k_rope dims
      tc.lds_off[i] = blk * 1024;
      tc.kdesc[i] = uniform4(rope ? kr_desc : kn_desc);
      tc.krow_bytes[i] = rope ? kDr * 2 : kDn * 2;
      tc.voff[i] = rope ? row * (kDr * 2) + (chunk - 16) * 16 : row * (kDn * 2) + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {            // V blocks 2w, 2w+1 of 16 (4 row blocks x 4 quads)
      const int blk = 2 * wave + i, rb = blk / 4, cq = blk % 4;
      const int row = rb * 16 + r16;
      tc.lds_off[3 + i] = blk * 1024;
      tc.voff[3 + i] = row * (kDv * 2) + (cq * 4 + s4) * 16;
    }
  }
  // k0 = Lk makes every lane's read out of range (zeros, no traffic): used for
  // ring slots whose tile does not exist, so every wave always issues the same
  // number of copies and the wait count is a constant.
  auto issue_k = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      dma16(tc.kdesc[i], lds0 + kKRing + slot * kKBytes + tc.lds_off[i], tc.voff[i], k0 * tc.krow_bytes[i]);
  };
  auto issue_v = [&](int slot, int k0) {
#pragma unroll
    for (int i = 3; i < 5; ++i) dma16(tc.v, lds0 + kVRing + slot * kVBytes + tc.lds_off[i], tc.voff[i], k0 * (kDv * 2));
  };
  // visibility words of a class-2 tile (1 KiB, copied by wave 0); kt = nkt reads zeros
  auto issue_bits = [&](int slot, int kt) {
    if (wave == 0) dma16(tc.bits, lds0 + kBitsRing + slot * kBitsBytes, lane * 16, kt * kBitsBytes);
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
  float m_run = -INFINITY;   // running max (natural units), same in both halves
  float l_run = 0.f;         // this lane's partial row sum

  const float scale = a.scale;
  const float scale_log2 = a.scale * kLog2e;
  const size_t mask_row = (static_cast<size_t>(b) * a.Lq + (q_ok ? q_row : 0)) * a.Lk;

  auto entry = [&](int i) -> int {
    if (i >= ntiles) return 0;
    if (!list) return i | (1 << 24);
    return __builtin_amdgcn_readfirstlane(s_list[i]);
  };
  auto k0_of = [&](int i, int e) -> int { return i < ntiles ? (e & 0xFFFFFF) * kTileN : a.Lk; };
  auto bits_kt = [&](int i, int e) -> int { return (i < ntiles && (e >> 24) == 2) ? (e & 0xFFFFFF) : a.nkt; };

  // Scores of the tile in ring slot `slot`: S^T = K Q^T over the 12 16-dim chunks.
  // A binary-mask tile starts the accumulator at 0 / -inf for visible / hidden keys
  // (the MFMA then applies the mask); other tiles start from an inline zero.
  auto scores = [&](int e, int slot) {
    const lds_char_t* ke = lds + kKRing + slot * kKBytes + k_even;
    const lds_char_t* ko = lds + kKRing + slot * kKBytes + k_odd;
    const bf16x8_t k_first = as_bf16x8(*reinterpret_cast<const lds_u32x4_t*>(ke));
    f32x16_t s;
    if ((e >> 24) == 2) {
      const uint64_t w64 = *reinterpret_cast<const lds_u64_t*>(lds + kBitsRing + slot * kBitsBytes + q_local * 8);
      const uint32_t w = static_cast<uint32_t>(w64 >> (kh * 32 + 4 * hi));   // bit 8g+c <-> key kh*32+8g+4hi+c
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(w), 8 * (r >> 2) + (r & 3), 1));
        s[r] = __uint_as_float(kNegInfBits & ~keep);
      }
      s = mfma32(k_first, qf[0], s);
    } else {
      const f32x16_t z = {};
      s = mfma32(k_first, qf[0], z);
    }
#pragma unroll
    for (int c = 1; c < kDqk / 16; ++c) {
      const lds_char_t* kp = ((c & 1) ? ko : ke) + (c >> 1) * 1024;
      const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const lds_u32x4_t*>(kp));
      s = mfma32(kf, qf[c], s);
    }
    return s;
  };

  // ---- prologue: K(0..2), bits(0..2), V(0..1) in flight; everyone scores tile 0
  __syncthreads();                                              // s_list visible
  int e0 = entry(0), e1 = entry(1), e2 = entry(2);
  issue_k(0, k0_of(0, e0));
  issue_k(1, k0_of(1, e1));
  issue_k(2, k0_of(2, e2));
  issue_v(0, k0_of(0, e0));
  issue_v(1, k0_of(1, e1));
  issue_bits(0, bits_kt(0, e0));
  issue_bits(1, bits_kt(1, e1));
  issue_bits(2, bits_kt(2, e2));
  wait_vmem<0>();
  __syncthreads();
  f32x16_t s = scores(e0, 0);                  // S(0)

  int e_cur = e0, e_nxt = e1, e_nxt2 = e2;     // tiles it, it+1, it+2
  int slot = 0;                                // ring slot of tile it
  for (int it = 0; it < ntiles; ++it) {
    const int slot1 = slot == 2 ? 0 : slot + 1;        // tile it+1
    const int slot2 = slot1 == 2 ? 0 : slot1 + 1;      // tile it+2 (and it-1)
    const int e_nxt3 = entry(it + 3);
    const int cls = e_cur >> 24;
    const int k0 = (e_cur & 0xFFFFFF) * kTileN;
    // accumulator r <-> key k0 + kh*32 + 8*(r>>2) + 4*hi + (r&3)
    const int kbase = k0 + kh * 32 + 4 * hi;

    // ---- part 1: tile max of S(it)
    float tile_max;
    if (cls == 3) {
      // general mask values: s <- scale*qk + mask (natural units)
      float mv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {   // all 16 loads in flight together (clamped index, fixed below)
        const int kk = kbase + 8 * (r >> 2) + (r & 3);
        mv[r] = load_mask<MASK_BF16>(a.mask, mask_row + min(kk, a.Lk - 1));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kbase + 8 * (r >> 2) + (r & 3);
        const float m = kk < a.Lk ? (q_ok ? mv[r] : 0.f) : -INFINITY;
        s[r] = __builtin_fmaf(s[r], scale, m);
      }
      tile_max = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tile_max = fmaxf(tile_max, s[r]);
    } else {
      if (k0 + kTileN > a.Lk) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 8 * (r >> 2) + (r & 3) >= a.Lk) s[r] = -INFINITY;
      }
      tile_max = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tile_max = fmaxf(tile_max, s[r]);
      tile_max *= scale;
    }
    tile_max = halves_max(tile_max);

    // ---- lazy rescale (wave-uniform decision)
    const bool need = (tile_max > m_run + kLazyTau) || (m_run == -INFINITY && tile_max > -INFINITY);
    if (__any(need)) {
      const float m_new = fmaxf(m_run, tile_max);
      const float alpha = (m_run == -INFINITY || m_new == -INFINITY) ? (m_run == m_new ? 1.f : 0.f)
                                                                     : __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    // p = exp2(fma(x, ca, cb)): raw scores for zero/binary tiles, s - m for general ones
    float ca = scale_log2, cb = -m_use * kLog2e;
    if (cls == 3) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] -= m_use;
      ca = kLog2e;
      cb = 0.f;
    }
    // ---- copies for later tiles: K(it+3) and bits(it+3) into the slots of tile it,
    // V(it+2) into the V slot of tile it-1 (all last read before the previous barrier).
    // Issued here so their scalar work overlaps the MFMAs below.
    issue_k(slot, k0_of(it + 3, e_nxt3));
    issue_bits(slot, bits_kt(it + 3, e_nxt3));
    issue_v(slot2, k0_of(it + 2, e_nxt2));

    // ---- part 2: S(it+1) MFMAs interleaved with the probabilities of tile it, then
    // PV(it).  The sched barrier keeps the score chain ahead of the PV MFMAs, so the
    // next iteration's tile max does not wait behind them.
    const f32x16_t s_next = scores(e_nxt, slot1);
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], ca, cb));
    uint32_t pk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pk[u] = pack_bf16x2(p[2 * u], p[2 * u + 1]);
    __builtin_amdgcn_sched_barrier(0);
    // row sum of the rounded probabilities, the values the PV MFMA consumes
    {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[u]), one2, l0, false);
        l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[u + 1]), one2, l1, false);
      }
      l_run += l0 + l1;
    }
    // O^T += V^T P^T over this wave's 32 keys (two 16-key MFMA steps).  B operand
    // element e of lane (li, hi) is key 8*(e>>2) + 4*hi + (e&3) of the step; the
    // transposing reads deliver V[that key][32*j + li] as A operand.
    const lds_char_t* vs = lds + kVRing + slot * kVBytes + v_base;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const u32x4_t pb = {pk[4 * step + 0], pk[4 * step + 1], pk[4 * step + 2], pk[4 * step + 3]};
      const bf16x8_t bfr = as_bf16x8(pb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const lds_char_t* vp = vs + step * 4096 + j * 1024;
        const s16x4_t lo = ds_read_tr(vp);
        const s16x4_t hi4 = ds_read_tr(vp + 512);
        const s16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[j] = mfma32(__builtin_bit_cast(bf16x8_t, av), bfr, o[j]);
      }
    }

    s = s_next;
    e_cur = e_nxt;
    e_nxt = e_nxt2;
    e_nxt2 = e_nxt3;
    slot = slot1;
    // copies issued one iteration ago (K(it+2), bits(it+2), V(it+1)) must have
    // landed; this iteration's (5 per wave, 6 for wave 0) stay in flight.
    if (wave == 0) wait_vmem<6>();
    else wait_vmem<5>();
    __syncthreads();
  }
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

}  // namespace

hipError_t launch_attn_bf16(const AttnBf16Args& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.nqt * a.H;
  if (a.mask && a.mask_bf16)
    hipLaunchKernelGGL(attn_fwd_bf16<true>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16<false>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
