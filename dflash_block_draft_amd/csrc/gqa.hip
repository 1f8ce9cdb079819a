// The MHA/GQA DFlash draft's attention path (Modular MAX page,
// pipelines.architectures.dflash_kimi_k25): qk-norm + yarn RoPE applied in
// place to head-major rows, and block attention of the draft's queries over the
// bf16 KV cache that holds the materialised context plus the block itself.
//
// norm_rope: one workgroup per 4 tokens of a batch row, one wave per head row of
// 128: lane l holds entries l and l + 64, which are exactly a rotate-half pair, so
// the RMSNorm reduction is one wave sum and the rotation needs no data movement.
// The yarn frequencies are formed once per workgroup in fp64, each angle
// (position times frequency) is reduced modulo 2 pi in fp64 and only then taken
// through fp32 sin / cos, so large positions lose no accuracy.
//
// gqa_attn: the cache is read once per KV head for its whole query group (g heads
// x bs block tokens <= 64 query rows), so each key byte feeds 64 rows: the
// kernel streams K and V at HBM rate and is bound by HBM, not by the matrix
// cores.  Keys are split across workgroups (split-K, flash-decoding style) so
// B * Hkv * splits workgroups cover the chip; each keeps fp32 (O, m, l) partials
// and a combine kernel merges the splits in order.  Inside a workgroup, four
// waves = 2 query blocks of 32 x 2 key halves of each 64-key tile; scores are
// computed transposed (S^T = K Q^T, one query per lane) so P^T feeds
// O^T += V^T P^T straight from the accumulator, with V^T read from the cache's
// transposed V (keys contiguous per dimension) -- no transposing LDS reads.
#include "common.h"
#include "launch.h"

#include <math.h>

#include <type_traits>

namespace dflash {
namespace {

constexpr int kD = 128;                       // head_dim this file is built for
constexpr int kKT = 64;                       // keys per tile
constexpr int kSK = kD * 2 + 16;              // K tile row stride (bytes): 272
constexpr int kSV = kKT * 2 + 16;             // V^T tile row stride (bytes): 144
constexpr int kStageK = kKT * kSK;
constexpr int kStage = kStageK + kD * kSV;    // 35840 bytes
constexpr int kDepth = 3;                      // tiles in flight: register sets = LDS stages

__device__ __forceinline__ float bf16r(float x) { return bf16_bits_to_f32(pack_bf16x2(x, 0.f) & 0xFFFFu); }

__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kRopeTok = 4;                    // tokens per norm/rope workgroup

constexpr int kRopeBatch = 8;                  // (token, head) rows a wave loads before it computes

__global__ void __launch_bounds__(256) norm_rope_bf16(NormRopeArgs a) {
  __shared__ float s_cos[kRopeTok][kD / 2], s_sin[kRopeTok][kD / 2];
  const int b = blockIdx.y;
  const int tbase = blockIdx.x * kRopeTok;
  const int t0 = a.row_off ? min(max(a.row_off[b], 0), a.off_max) : 0;
  {  // one angle per thread: the product and its reduction modulo 2 pi in fp64, sin / cos in fp32
    const int tk = threadIdx.x / (kD / 2), i = threadIdx.x % (kD / 2);
    const double two_pi = 6.283185307179586;
    const double ang = static_cast<double>(t0 + tbase + tk) * a.inv_freq[i];
    const float red = static_cast<float>(ang - floor(ang / two_pi) * two_pi);
    float sn, cs;
    sincosf(red, &sn, &cs);
    s_cos[tk][i] = cs * a.mscale;
    s_sin[tk][i] = sn * a.mscale;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float g0 = bf16_bits_to_f32(a.gamma[lane]), g1 = bf16_bits_to_f32(a.gamma[lane + 64]);
  const int njobs = min(kRopeTok, a.T - tbase) * a.H;   // token-major (token, head) rows of this workgroup
  // each wave takes jobs wave, wave + 4, ...; the rows of a batch are all loaded
  // before any is normalised, so their latencies overlap
  for (int base = wave; base < njobs; base += 4 * kRopeBatch) {
    float x0[kRopeBatch], x1[kRopeBatch];
    uint16_t* rows[kRopeBatch];
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u) {
      const int job = min(base + 4 * u, njobs - 1);      // past the end: a repeat of the last row, not stored
      const int tk = job / a.H, h = job % a.H;
      const int t = tbase + tk;
      const int row_t = a.rows_local ? t : t0 + t;
      rows[u] = a.x + ((static_cast<size_t>(b) * a.H + h) * a.Lt + row_t) * kD;
      x0[u] = bf16_bits_to_f32(rows[u][lane]);
      x1[u] = bf16_bits_to_f32(rows[u][lane + 64]);
    }
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u) {
      const int job = base + 4 * u;
      float ss = x0[u] * x0[u] + x1[u] * x1[u];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
      if (job >= njobs) continue;
      const int tk = job / a.H;
      const float r = rsqrtf(ss / kD + a.eps);
      const float n0 = bf16r(bf16r(x0[u] * r) * g0), n1 = bf16r(bf16r(x1[u] * r) * g1);
      const float c = s_cos[tk][lane], sn = s_sin[tk][lane];
      const uint32_t w = pack_bf16x2(n0 * c - n1 * sn, n1 * c + n0 * sn);
      rows[u][lane] = static_cast<uint16_t>(w & 0xFFFFu);
      rows[u][lane + 64] = static_cast<uint16_t>(w >> 16);
    }
  }
}

template <int N>
using IC = std::integral_constant<int, N>;

__global__ void __launch_bounds__(256) gqa_attn_bf16(GqaAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kDepth * kStage];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 31, hi = lane >> 5;
  const int qb = w & 1, kh = w >> 1;
  const int sp = blockIdx.x, bk = blockIdx.y;
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int g = a.Hq / a.Hkv, Qg = g * a.bs;
  const int L = min(max(a.ctx_len[b], 0), a.Lmax - a.bs) + a.bs;
  const int ntiles = (L + kKT - 1) / kKT;
  const int tile0 = sp * a.tiles_per_split, tile1 = min(tile0 + a.tiles_per_split, ntiles);

  // this lane's query row of the group
  const int r = 32 * qb + li;
  const bool r_ok = r < Qg;
  const int h = hk * g + (r_ok ? r / a.bs : 0), i = r_ok ? r % a.bs : 0;
  bf16x8_t qreg[kD / 16];
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    qreg[s] = as_bf16x8(r_ok ? ldg16(a.q + ((static_cast<size_t>(b) * a.Hq + h) * a.bs + i) * kD + 16 * s + 8 * hi) : z);
  }
  const uint16_t* kbase = a.k + static_cast<size_t>(bk) * a.Lmax * kD;
  const uint16_t* vbase = a.vt + static_cast<size_t>(bk) * kD * a.Lmax;

  f32x16_t o[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
  float m = -INFINITY, l = 0.f;                       // log2 units

  // Tile i of the split goes global -> registers set i % kDepth (issued kDepth - 1
  // tiles ahead) -> LDS stage i % kDepth: while tile i is computed, the loads of
  // tiles i+1 .. i+kDepth are in flight (the register sets come from the file this
  // one-wave-per-SIMD kernel has to spare).  The loads go through buffer resources
  // and are issued unconditionally, so the compiler can count them (a wait for one
  // set leaves the younger sets in flight): K rows past L read as zeros (the
  // resource ends at row L), a tile past the split uses an offset beyond both
  // resources (zeros, no traffic), and V^T keys past L are zeroed when the tail
  // tile is committed (they are inside the resource: the cache there is unset).
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), 0, L * kD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase), 0, kD * a.Lmax * 2, 0x00020000);
  constexpr uint32_t kPastEnd = 0x80000000u;   // > every resource size (the host bounds a slice by 2^31 bytes)
  uint32_t kvo[4], vvo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ci = t + 256 * c;
    kvo[c] = static_cast<uint32_t>((ci >> 4) * kD * 2 + (ci & 15) * 16);        // K: 64 rows x 16 chunks
    vvo[c] = static_cast<uint32_t>((ci >> 3) * a.Lmax * 2 + (ci & 7) * 16);     // V^T: 128 rows x 8 chunks of 8 keys
  }
  u32x4_t pre[kDepth][8];
  auto prefetch = [&](auto S, int tile) __attribute__((always_inline)) {
    constexpr int set = decltype(S)::value;
    const bool real = tile < tile1;
    const uint32_t ks = real ? static_cast<uint32_t>(tile) * kKT * kD * 2 : kPastEnd;
    const uint32_t vs = real ? static_cast<uint32_t>(tile) * kKT * 2 : kPastEnd;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pre[set][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, kvo[c], ks, 0));
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pre[set][4 + c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, vvo[c], vs, 0));
  };
  auto commit = [&](auto S, int tile) __attribute__((always_inline)) {
    constexpr int set = decltype(S)::value;
    char* st = smem + set * kStage;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ci = t + 256 * c;
      *reinterpret_cast<u32x4_t*>(st + (ci >> 4) * kSK + (ci & 15) * 16) = pre[set][c];
    }
    if ((tile + 1) * kKT > L) {                     // the tail tile: zero V^T keys >= L
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int key = tile * kKT + 8 * ((t + 256 * c) & 7);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k2 = key + 2 * e;
          const uint32_t keep = (k2 < L ? 0x0000FFFFu : 0u) | (k2 + 1 < L ? 0xFFFF0000u : 0u);
          pre[set][4 + c][e] &= keep;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ci = t + 256 * c;
      *reinterpret_cast<u32x4_t*>(st + kStageK + (ci >> 3) * kSV + (ci & 7) * 16) = pre[set][4 + c];
    }
  };

  const float c2 = a.scale * kLog2e;
  auto compute = [&](const char* st, int tile) __attribute__((always_inline)) {
    f32x16_t s = {};
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int k = 0; k < kD / 16; ++k)
      s = mfma32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(st + (32 * kh + li) * kSK + (16 * k + 8 * hi) * 2)),
                 qreg[k], s);
    float x[16], tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = tile * kKT + 32 * kh + 8 * (e >> 2) + 4 * hi + (e & 3);
      x[e] = key < L ? s[e] * c2 : -INFINITY;
      tmax = fmaxf(tmax, x[e]);
    }
    // a key half can lie wholly past L (the tail tile): m_new stays -inf there, and a
    // finite stabiliser keeps exp2(-inf - m) = 0 instead of exp2(-inf + inf) = NaN
    const float m_new = fmaxf(m, halves_max(tmax));
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    if (__any(m_new != m)) {          // rescale only when some row's maximum rose (alpha = 1 elsewhere)
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < kD / 32; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
      m = m_new;
    }
    float p[16], sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = bf16r(__builtin_amdgcn_exp2f(x[e] - m_sub));
      sum += p[e];
    }
    l += halves_sum(sum);
    bf16x8_t pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4_t wv = {pack_bf16x2(p[8 * kk], p[8 * kk + 1]), pack_bf16x2(p[8 * kk + 2], p[8 * kk + 3]),
                          pack_bf16x2(p[8 * kk + 4], p[8 * kk + 5]), pack_bf16x2(p[8 * kk + 6], p[8 * kk + 7])};
      pb[kk] = as_bf16x8(wv);
    }
#pragma unroll
    for (int j = 0; j < kD / 32; ++j) {
      const char* rowp = st + kStageK + (32 * j + li) * kSV;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // keys 32kh + 16kk + {4hi .. 4hi+3} and {8 + 4hi .. 8 + 4hi + 3}: the accumulator's row order
        const int kb = 32 * kh + 16 * kk + 4 * hi;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(rowp + kb * 2);
        const u32x2_t up = *reinterpret_cast<const u32x2_t*>(rowp + (kb + 8) * 2);
        const u32x4_t av = {lo[0], lo[1], up[0], up[1]};
        o[j] = mfma32(as_bf16x8(av), pb[kk], o[j]);
      }
    }
  };

  // One step on tile `tile` (set / stage S = its index % kDepth): start the loads of
  // tile + kDepth - 1 (past the split: a no-traffic zero read) into the set tile - 1
  // used (committed one step ago), compute,
  // then commit tile + 1 into its stage (last read by the step before this one,
  // which every wave has left: the barrier that ended it).  Returns false after the
  // split's last tile.
  auto step = [&](auto S, int tile) __attribute__((always_inline)) -> bool {
    constexpr int set = decltype(S)::value;
    constexpr int prev = (set + kDepth - 1) % kDepth, next = (set + 1) % kDepth;
    prefetch(IC<prev>{}, tile + kDepth - 1);
    compute(smem + set * kStage, tile);
    if (tile + 1 >= tile1) return false;
    commit(IC<next>{}, tile + 1);
    __syncthreads();
    return true;
  };
  if (tile0 < tile1) {
    static_assert(kDepth == 3, "the prologue and the unrolled loop below are written for three sets");
    prefetch(IC<0>{}, tile0);
    prefetch(IC<1>{}, tile0 + 1);
    commit(IC<0>{}, tile0);
    __syncthreads();
    for (int tile = tile0;; tile += kDepth) {
      if (!step(IC<0>{}, tile)) break;
      if (!step(IC<1>{}, tile + 1)) break;
      if (!step(IC<2>{}, tile + 2)) break;
    }
  }
  __syncthreads();

  // merge the two key halves of each query block, write the split's partial
  float* red = reinterpret_cast<float*>(smem) + qb * (64 * (16 * kD / 32 + 2));
  if (kh == 1) {
#pragma unroll
    for (int j = 0; j < kD / 32; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(j * 16 + e) * 64 + lane] = o[j][e];
    red[(kD / 2) * 64 + lane] = m;
    red[(kD / 2 + 1) * 64 + lane] = l;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = red[(kD / 2) * 64 + lane], l1 = red[(kD / 2 + 1) * 64 + lane];
    const float mm = fmaxf(m, m1);
    const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    const size_t prow = (static_cast<size_t>(bk) * a.splits + sp) * 64 + r;
    if (r_ok) {
      float* po = a.part_o + prow * kD;
      // o[j][e] holds dim 32 j + 8 (e / 4) + 4 hi + e % 4
#pragma unroll
      for (int j = 0; j < kD / 32; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4_t v;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * gq + c;
            v[c] = o[j][e] * a0 + red[(j * 16 + e) * 64 + lane] * a1;
          }
          *reinterpret_cast<f32x4_t*>(po + 32 * j + 8 * gq + 4 * hi) = v;
        }
      if (hi == 0) {
        a.part_ml[prow * 2] = mm;
        a.part_ml[prow * 2 + 1] = l * a0 + l1 * a1;
      }
    }
  }
}

// out[b, h, i, :] = sum over splits of the partials, merged in split order.
__global__ void __launch_bounds__(kD) gqa_combine_bf16(GqaAttnArgs a) {
  const int r = blockIdx.x, bk = blockIdx.y;
  const int b = bk / a.Hkv, hk = bk % a.Hkv, g = a.Hq / a.Hkv;
  const int d = threadIdx.x;
  const size_t base = static_cast<size_t>(bk) * a.splits * 64 + r;
  float mm = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mm = fmaxf(mm, a.part_ml[(base + static_cast<size_t>(s) * 64) * 2]);
  float lsum = 0.f, acc = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const size_t row = base + static_cast<size_t>(s) * 64;
    const float ms = a.part_ml[row * 2];
    if (ms == -INFINITY) continue;
    const float wgt = __builtin_amdgcn_exp2f(ms - mm);
    lsum += wgt * a.part_ml[row * 2 + 1];
    acc += wgt * a.part_o[row * kD + d];
  }
  const int h = hk * g + r / a.bs, i = r % a.bs;
  const float v = lsum > 0.f ? acc / lsum : 0.f;
  a.out[((static_cast<size_t>(b) * a.Hq + h) * a.bs + i) * kD + d] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFFu);
}

}  // namespace

hipError_t launch_norm_rope_bf16(const NormRopeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(norm_rope_bf16, dim3((a.T + kRopeTok - 1) / kRopeTok, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gqa_attn_bf16(const GqaAttnArgs& a, hipStream_t s) {
  const unsigned bk = static_cast<unsigned>(a.B) * a.Hkv;
  hipLaunchKernelGGL(gqa_attn_bf16, dim3(a.splits, bk), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gqa_combine_bf16, dim3((a.Hq / a.Hkv) * a.bs, bk), dim3(kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
