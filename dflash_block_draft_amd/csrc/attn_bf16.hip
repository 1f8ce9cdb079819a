// Fused non-causal draft MLA attention forward, bf16 MFMA on gfx950.
//
// What it computes (NeMo AutoModel DFlash page, KimiK3DFlashAttention.forward;
// DSpark page, KimiK3DSparkAttention): for every (batch, head, noise query)
//   s_j = scale * (q_nope . k_nope[h][j] + q_rope . k_rope[j]) + mask[i][j]
//   out = softmax_j(s) @ v[h]
// over the keys [context | noise block], with no materialised score matrix.
//
// Decomposition (one workgroup = one (batch, head, 128-query tile)):
//  * 8 waves: wave w owns queries 32*(w&3) .. +31 of the tile and keys
//    32*(w>>2) .. +31 of every 64-key tile; the two waves of a query group
//    merge (m, l, O) once at the end.  Two waves per SIMD, so one wave's
//    softmax overlaps the other's MFMAs.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds one query and 16 of its keys, so row max / row sum are
//    in-lane (plus one v_permlane32_swap), and the lane's P^T values are
//    already the B operand of O^T = V^T P^T for the same key order (the order
//    of the key contraction is free, so keys are relabelled to match the
//    accumulator layout).
//  * V^T operands come straight from the row-major V tile with the gfx950
//    transposing LDS read (ds_read_b64_tr_b16); V rows are padded to 320 B so
//    those reads are bank-conflict free, K rows to 400 B for the b128 reads.
//  * Q (32 x 192 bf16 per wave) stays in registers for the whole key loop.
//  * K = [k_nope | k_rope] and V tiles are staged in LDS, double-buffered,
//    with 16-byte coalesced loads; the head-shared k_rope tile is stored next
//    to this head's k_nope so one LDS row feeds the whole 192-wide contraction.
//  * Online softmax in fp32 with the hardware exp2; the running max is only
//    raised when a new score exceeds it by more than 2^8 in probability space
//    ("lazy rescale"), exact because the same max scales both O and l.
//  * Tiles come from the occupancy lists: empty tiles are never visited, zero
//    tiles skip the mask entirely, binary tiles apply a prefetched 64-bit
//    visibility word per query, general tiles add the mask values.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKsStride = kDqk + 8;               // bf16 per LDS K row (400 B)
constexpr int kVsStride = kDv + 32;               // bf16 per LDS V row (320 B)
constexpr int kKsTile = kTileN * kKsStride;
constexpr int kVsTile = kTileN * kVsStride;
constexpr int kStageElems = kKsTile + kVsTile;     // one buffer
constexpr float kLazyTau = 8.0f / kLog2e;          // natural-units slack before a rescale
constexpr uint32_t kNegInfBits = 0xFF800000u;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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
__device__ __forceinline__ s16x4_t ds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

struct Stage {
  u32x4_t kn0, kn1, kr, v0, v1;
};

// Global -> registers for the key tile starting at k0 (zero rows past Lk).
__device__ __forceinline__ void load_stage(Stage& st, const uint16_t* kn_bh, const uint16_t* kr_b,
                                           const uint16_t* v_bh, int k0, int Lk, int t) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  {
    const int row = t >> 4, c = t & 15;
    const bool ok = k0 + row < Lk;
    st.kn0 = ok ? ldg16(kn_bh + static_cast<size_t>(k0 + row) * kDn + c * 8) : z;
    st.v0 = ok ? ldg16(v_bh + static_cast<size_t>(k0 + row) * kDv + c * 8) : z;
  }
  {
    const int row = 32 + (t >> 4), c = t & 15;
    const bool ok = k0 + row < Lk;
    st.kn1 = ok ? ldg16(kn_bh + static_cast<size_t>(k0 + row) * kDn + c * 8) : z;
    st.v1 = ok ? ldg16(v_bh + static_cast<size_t>(k0 + row) * kDv + c * 8) : z;
  }
  {
    const int row = t >> 3, c = t & 7;
    st.kr = (k0 + row < Lk) ? ldg16(kr_b + static_cast<size_t>(k0 + row) * kDr + c * 8) : z;
  }
}

__device__ __forceinline__ void store_stage(const Stage& st, uint16_t* buf, int t) {
  uint16_t* Ks = buf;
  uint16_t* Vs = buf + kKsTile;
  {
    const int row = t >> 4, c = t & 15;
    stg16(Ks + row * kKsStride + c * 8, st.kn0);
    stg16(Vs + row * kVsStride + c * 8, st.v0);
  }
  {
    const int row = 32 + (t >> 4), c = t & 15;
    stg16(Ks + row * kKsStride + c * 8, st.kn1);
    stg16(Vs + row * kVsStride + c * 8, st.v1);
  }
  {
    const int row = t >> 3, c = t & 7;
    stg16(Ks + row * kKsStride + kDn + c * 8, st.kr);
  }
}

template <bool MASK_BF16>
__device__ __forceinline__ float load_mask(const void* mask, size_t idx) {
  if (MASK_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(mask)[idx]);
  return static_cast<const float*>(mask)[idx];
}

template <bool MASK_BF16>
__global__ void __launch_bounds__(kThreads, 1) attn_fwd_bf16(AttnBf16Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStageElems];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
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
  const int ntiles = a.counts ? (a.no_skip ? a.nkt : a.counts[bq]) : a.nkt;

  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const uint16_t* kn_bh = a.kn + bh * a.Lk * kDn;
  const uint16_t* v_bh = a.v + bh * a.Lk * kDv;
  const uint16_t* kr_b = a.kr + static_cast<size_t>(b) * a.Lk * kDr;

  const int q_local = qg * 32 + li;               // this lane's query within the tile
  const int q_row = qt * kTileM + q_local;
  const bool q_ok = q_row < a.Lq;

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
  const size_t tile_row0 = static_cast<size_t>(bq) * a.nkt;

  auto tile_at = [&](int i, int& kt, int& cls) {
    if (!a.counts) { kt = i; cls = 1; return; }
    if (a.no_skip) {
      kt = i;
      const int c = a.classes[tile_row0 + i];
      cls = c == 0 ? 3 : c;
      return;
    }
    const int e = a.lists[tile_row0 + i];
    kt = e & 0xFFFFFF;
    cls = e >> 24;
  };
  auto load_bits = [&](int kt, int cls) -> uint32_t {
    if (cls != 2) return 0u;
    const uint64_t w = a.bits[(tile_row0 + kt) * kTileM + q_local];
    return static_cast<uint32_t>(w >> (kh * 32 + 4 * hi));   // bit 8g+c <-> key kh*32 + 8g + 4hi + c
  };

  // per-lane LDS offsets (elements)
  const int k_off = (kh * 32 + li) * kKsStride + 8 * hi;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_off = (kh * 32 + 4 * hi + (i16 >> 2)) * kVsStride + 16 * (g16 & 1) + 4 * (i16 & 3);

  Stage st;
  int kt_cur = 0, cls_cur = 1;
  uint32_t bits_cur = 0u;
  if (ntiles > 0) {
    tile_at(0, kt_cur, cls_cur);
    load_stage(st, kn_bh, kr_b, v_bh, kt_cur * kTileN, a.Lk, t);
    bits_cur = load_bits(kt_cur, cls_cur);
    store_stage(st, smem, t);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = kt_cur * kTileN;
    const bool has_next = it + 1 < ntiles;
    int kt_nxt = 0, cls_nxt = 1;
    uint32_t bits_nxt = 0u;
    if (has_next) {
      tile_at(it + 1, kt_nxt, cls_nxt);
      load_stage(st, kn_bh, kr_b, v_bh, kt_nxt * kTileN, a.Lk, t);
      bits_nxt = load_bits(kt_nxt, cls_nxt);
    }
    const uint16_t* Ks = smem + (it & 1) * kStageElems;
    const uint16_t* Vs = Ks + kKsTile;

    // ---- S^T block: keys kh*32 + (rows), queries qg*32 + li
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < kDqk / 16; ++c) {
      const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Ks + k_off + 16 * c));
      s = mfma32(kf, qf[c], s);
    }

    // accumulator r <-> key k0 + kh*32 + 8*(r>>2) + 4*hi + (r&3)
    const int kbase = k0 + kh * 32 + 4 * hi;
    float tile_max;
    if (cls_cur == 3) {
      // general mask values: s <- scale*qk + mask (natural units)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kbase + 8 * (r >> 2) + (r & 3);
        float mv = -INFINITY;
        if (kk < a.Lk) mv = q_ok ? load_mask<MASK_BF16>(a.mask, mask_row + kk) : 0.f;
        s[r] = __builtin_fmaf(s[r], scale, mv);
      }
      tile_max = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tile_max = fmaxf(tile_max, s[r]);
    } else {
      if (cls_cur == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = 8 * (r >> 2) + (r & 3);
          const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(bits_cur), bit, 1));
          s[r] = __uint_as_float((__float_as_uint(s[r]) & keep) | (kNegInfBits & ~keep));
        }
      }
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

    // ---- probabilities (hardware exp2; results below 2^-126 flush to 0)
    float p[16];
    if (cls_cur == 3) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f((s[r] - m_use) * kLog2e);
    } else {
      const float nm = -m_use * kLog2e;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, nm));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) l_run += p[r];
    uint32_t pk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pk[u] = pack_bf16x2(p[2 * u], p[2 * u + 1]);

    // ---- O^T += V^T P^T over this wave's 32 keys (two 16-key MFMA steps).
    // B operand element e of lane (li, hi) is key 8*(e>>2) + 4*hi + (e&3) of the
    // step; the transposing reads deliver V[that key][32*j + li] as A operand.
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const u32x4_t pb = {pk[4 * step + 0], pk[4 * step + 1], pk[4 * step + 2], pk[4 * step + 3]};
      const bf16x8_t bfr = as_bf16x8(pb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t* vp = Vs + v_off + 16 * step * kVsStride + 32 * j;
        const s16x4_t lo = ds_read_tr(vp);
        const s16x4_t hi4 = ds_read_tr(vp + 8 * kVsStride);
        typedef short s16x8_t __attribute__((ext_vector_type(8)));
        const s16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[j] = mfma32(__builtin_bit_cast(bf16x8_t, av), bfr, o[j]);
      }
    }

    if (has_next) store_stage(st, smem + ((it + 1) & 1) * kStageElems, t);
    kt_cur = kt_nxt;
    cls_cur = cls_nxt;
    bits_cur = bits_nxt;
    __syncthreads();
  }

  // ---- merge the two key halves of each query group, normalise, store
  l_run = halves_sum(l_run);
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
