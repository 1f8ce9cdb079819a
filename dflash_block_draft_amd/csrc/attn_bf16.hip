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
//    32*(w>>2) .. +31 of every 64-key tile, so the two waves of a query group
//    split each key tile and merge (m, l, O) once at the end.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds one query and 16 of its keys, so row max / row sum are
//    in-lane, and the lane's P^T values are already the B operand of
//    O^T = V^T P^T for the same key order (the contraction order over keys is
//    free, so keys are simply relabelled to match the accumulator layout).
//  * Q (32 x 192 bf16 per wave) stays in registers for the whole key loop.
//  * K = [k_nope | k_rope] and V tiles are staged in LDS, double-buffered,
//    with 16-byte coalesced loads; the head-shared k_rope tile is stored next
//    to this head's k_nope so one LDS row feeds the whole 192-wide contraction.
//  * Online softmax in fp32 with exp2; the running max is only raised when a
//    new score exceeds it by more than 2^8 in probability space ("lazy
//    rescale"), which is exact because the same max scales both O and l.
//  * Tiles come from the occupancy lists: empty tiles are never visited, zero
//    tiles skip the mask entirely, mixed tiles add it from global memory.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKsStride = kDqk + 8;               // bf16 per LDS K row (400 B: conflict-free b128 reads)
constexpr int kVsStride = kDv;                     // bf16 per LDS V row
constexpr int kKsTile = kTileN * kKsStride;
constexpr int kVsTile = kTileN * kVsStride;
constexpr int kStageElems = kKsTile + kVsTile;     // one buffer
constexpr float kLazyTau = 8.0f / kLog2e;          // natural-units slack before a rescale

// Cross-half exchange (lane l <-> lane l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

struct Stage {
  u32x4_t kn0, kn1, kr, v0, v1;
};

// Global -> registers for key tile starting at k0 (zero rows past Lk).
__device__ __forceinline__ void load_stage(Stage& st, const uint16_t* kn_bh, const uint16_t* kr_b,
                                           const uint16_t* v_bh, int k0, int Lk, int t) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  {
    const int ci = t, row = ci >> 4, c = ci & 15;
    st.kn0 = (k0 + row < Lk) ? ldg16(kn_bh + static_cast<size_t>(k0 + row) * kDn + c * 8) : z;
    st.v0 = (k0 + row < Lk) ? ldg16(v_bh + static_cast<size_t>(k0 + row) * kDv + c * 8) : z;
  }
  {
    const int ci = t + kThreads, row = ci >> 4, c = ci & 15;
    st.kn1 = (k0 + row < Lk) ? ldg16(kn_bh + static_cast<size_t>(k0 + row) * kDn + c * 8) : z;
    st.v1 = (k0 + row < Lk) ? ldg16(v_bh + static_cast<size_t>(k0 + row) * kDv + c * 8) : z;
  }
  {
    const int ci = t, row = ci >> 3, c = ci & 7;
    st.kr = (k0 + row < Lk) ? ldg16(kr_b + static_cast<size_t>(k0 + row) * kDr + c * 8) : z;
  }
}

__device__ __forceinline__ void store_stage(const Stage& st, uint16_t* buf, int t) {
  uint16_t* Ks = buf;
  uint16_t* Vs = buf + kKsTile;
  {
    const int ci = t, row = ci >> 4, c = ci & 15;
    stg16(Ks + row * kKsStride + c * 8, st.kn0);
    stg16(Vs + row * kVsStride + c * 8, st.v0);
  }
  {
    const int ci = t + kThreads, row = ci >> 4, c = ci & 15;
    stg16(Ks + row * kKsStride + c * 8, st.kn1);
    stg16(Vs + row * kVsStride + c * 8, st.v1);
  }
  {
    const int ci = t, row = ci >> 3, c = ci & 7;
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

  const int q_row = qt * kTileM + qg * 32 + li;   // this lane's query
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

  auto tile_at = [&](int i, int& kt, int& cls) {
    if (!a.counts) { kt = i; cls = 1; return; }
    if (a.no_skip) {
      kt = i;
      const int c = a.classes[static_cast<size_t>(bq) * a.nkt + i];
      cls = c == 0 ? 2 : c;
      return;
    }
    const int e = a.lists[static_cast<size_t>(bq) * a.nkt + i];
    kt = e & 0xFFFFFF;
    cls = e >> 24;
  };

  Stage st;
  if (ntiles > 0) {
    int kt0, c0;
    tile_at(0, kt0, c0);
    load_stage(st, kn_bh, kr_b, v_bh, kt0 * kTileN, a.Lk, t);
    store_stage(st, smem, t);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    int kt, cls;
    tile_at(it, kt, cls);
    const int k0 = kt * kTileN;
    const bool has_next = it + 1 < ntiles;
    if (has_next) {
      int ktn, cn;
      tile_at(it + 1, ktn, cn);
      load_stage(st, kn_bh, kr_b, v_bh, ktn * kTileN, a.Lk, t);
    }
    const uint16_t* Ks = smem + (it & 1) * kStageElems;
    const uint16_t* Vs = Ks + kKsTile;

    // ---- S^T block: keys kh*32 + (rows), queries qg*32 + li
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    {
      const uint16_t* kp = Ks + (kh * 32 + li) * kKsStride + 8 * hi;
#pragma unroll
      for (int c = 0; c < kDqk / 16; ++c) {
        const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + 16 * c));
        s = mfma32(kf, qf[c], s);
      }
    }

    // key of accumulator r: k0 + kh*32 + 8*(r>>2) + 4*hi + (r&3)
    const int kbase = k0 + kh * 32 + 4 * hi;
    const bool partial = k0 + kTileN > a.Lk;
    float tile_max;
    if (cls == 2) {
      // mixed: s <- scale*qk + mask (natural units)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int key = kbase + 8 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int kk = key + c;
          float mv;
          if (kk < a.Lk) mv = q_ok ? load_mask<MASK_BF16>(a.mask, mask_row + kk) : 0.f;
          else mv = -INFINITY;
          s[4 * g + c] = __builtin_fmaf(s[4 * g + c], scale, mv);
        }
      }
      tile_max = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tile_max = fmaxf(tile_max, s[r]);
    } else {
      if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 8 * (r >> 2) + (r & 3) >= a.Lk) s[r] = -INFINITY;
      }
      tile_max = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tile_max = fmaxf(tile_max, s[r]);
      tile_max *= scale;
    }
    tile_max = fmaxf(tile_max, swap_halves(tile_max));

    // ---- lazy rescale (wave-uniform decision)
    const bool need = (tile_max > m_run + kLazyTau) || (m_run == -INFINITY && tile_max > -INFINITY);
    if (__any(need)) {
      const float m_new = fmaxf(m_run, tile_max);
      const float alpha = (m_run == -INFINITY || m_new == -INFINITY) ? (m_run == m_new ? 1.f : 0.f)
                                                                     : exp2f((m_run - m_new) * kLog2e);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // ---- probabilities
    float p[16];
    if (cls == 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = exp2f((s[r] - m_use) * kLog2e);
    } else {
      const float nm = -m_use * kLog2e;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = exp2f(__builtin_fmaf(s[r], scale_log2, nm));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) l_run += p[r];
    uint32_t pk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pk[u] = pack_bf16x2(p[2 * u], p[2 * u + 1]);

    // ---- O^T += V^T P^T over this wave's 32 keys (two 16-key MFMA steps).
    // B operand element e of lane (li, hi) is key 8*(e>>2) + 4*hi + (e&3) of the
    // step; the A operand (V^T) is loaded for exactly those keys.  Output row i of
    // block j is dv = 4*i + j, so one 8-byte LDS read per key serves all 4 blocks.
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      u32x4_t pb = {pk[4 * step + 0], pk[4 * step + 1], pk[4 * step + 2], pk[4 * step + 3]};
      const bf16x8_t bfr = as_bf16x8(pb);
      u32x2_t vr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kh * 32 + 16 * step + 8 * (e >> 2) + 4 * hi + (e & 3);
        vr[e] = *reinterpret_cast<const u32x2_t*>(Vs + key * kVsStride + 4 * li);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t av;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t x = vr[2 * u][j >> 1];
          const uint32_t y = vr[2 * u + 1][j >> 1];
          av[u] = (j & 1) ? hi16_pair(x, y) : lo16_pair(x, y);
        }
        o[j] = mfma32(as_bf16x8(av), bfr, o[j]);
      }
    }

    if (has_next) store_stage(st, smem + ((it + 1) & 1) * kStageElems, t);
    __syncthreads();
  }

  // ---- merge the two key halves of each query group, normalise, store
  l_run += swap_halves(l_run);
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
    const float a0 = (m_run == -INFINITY) ? 0.f : exp2f((m_run - m) * kLog2e);
    const float a1 = (m1 == -INFINITY) ? 0.f : exp2f((m1 - m) * kLog2e);
    const float l = l_run * a0 + l1 * a1;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (q_ok) {
      uint16_t* op = a.out + (bh * a.Lq + q_row) * kDv;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // dv = 32*g + 16*hi + 4*c + j  <-  o[j][4*g + c]
        uint32_t w[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            x[j] = (o[j][4 * g + c] * a0 + red[((4 * g + c) * 4 + j) * 64 + lane] * a1) * inv;
          w[2 * c] = pack_bf16x2(x[0], x[1]);
          w[2 * c + 1] = pack_bf16x2(x[2], x[3]);
        }
        uint16_t* dst = op + 32 * g + 16 * hi;
        stg16(dst, u32x4_t{w[0], w[1], w[2], w[3]});
        stg16(dst + 8, u32x4_t{w[4], w[5], w[6], w[7]});
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
