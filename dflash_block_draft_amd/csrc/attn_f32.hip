// fp32 draft MLA attention (same definition as the bf16 kernel; NeMo AutoModel
// DFlash page, KimiK3DFlashAttention.forward), computed entirely in fp32 with
// FMA dot products and an exact per-tile online softmax.  It exists so fp32
// inputs get an fp32 result; it is a correctness path, not a fast one.
//
// One wave per (batch, head, 64 queries); each lane owns one query row.  Key
// tiles of 32 keys are staged in LDS and read as broadcasts (every lane reads
// the same key), so there are no bank conflicts.
#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kQ = 64;      // queries per workgroup (one per lane)
constexpr int kKT = 32;     // keys per LDS tile

__global__ void __launch_bounds__(64) attn_fwd_f32(AttnF32Args a) {
  __shared__ float Ks[kKT][kDqk];
  __shared__ float Vs[kKT][kDv];
  const int lane = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int qi = qt * kQ + lane;
  const bool q_ok = qi < a.Lq;
  const size_t bh = static_cast<size_t>(b) * a.H + h;

  float qv[kDqk];
  {
    const float* qp = a.q + (bh * a.Lq + (q_ok ? qi : 0)) * kDqk;
#pragma unroll
    for (int d = 0; d < kDqk; ++d) qv[d] = q_ok ? qp[d] : 0.f;
  }
  float o[kDv];
#pragma unroll
  for (int d = 0; d < kDv; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kn = a.kn + bh * a.Lk * kDn;
  const float* kr = a.kr + static_cast<size_t>(b) * a.Lk * kDr;
  const float* vv = a.v + bh * a.Lk * kDv;
  const float* mrow = a.mask ? a.mask + (static_cast<size_t>(b) * a.Lq + (q_ok ? qi : 0)) * a.Lk : nullptr;

  for (int k0 = 0; k0 < a.Lk; k0 += kKT) {
    const int nk = min(kKT, a.Lk - k0);
    __syncthreads();
    for (int e = lane; e < kKT * kDqk; e += 64) {
      const int r = e / kDqk, d = e % kDqk;
      float x = 0.f;
      if (r < nk) x = d < kDn ? kn[static_cast<size_t>(k0 + r) * kDn + d] : kr[static_cast<size_t>(k0 + r) * kDr + d - kDn];
      Ks[r][d] = x;
    }
    for (int e = lane; e < kKT * kDv; e += 64) {
      const int r = e / kDv, d = e % kDv;
      Vs[r][d] = r < nk ? vv[static_cast<size_t>(k0 + r) * kDv + d] : 0.f;
    }
    __syncthreads();

    float s[kKT];
    float tmax = -INFINITY;
    for (int j = 0; j < kKT; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < kDqk; ++d) acc = __builtin_fmaf(qv[d], Ks[j][d], acc);
      float sj = acc * a.scale;
      if (j >= nk) sj = -INFINITY;
      else if (mrow) sj += mrow[k0 + j];
      s[j] = sj;
      tmax = fmaxf(tmax, sj);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new != -INFINITY) {                  // else nothing visible yet for this row
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < kDv; ++d) o[d] *= alpha;
      m = m_new;
      for (int j = 0; j < kKT; ++j) {
        const float p = expf(s[j] - m);        // exp(-inf) = 0
        l += p;
#pragma unroll
        for (int d = 0; d < kDv; ++d) o[d] = __builtin_fmaf(p, Vs[j][d], o[d]);
      }
    }
  }
  if (!q_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse) a.lse[bh * a.Lq + qi] = l > 0.f ? m + logf(l) : -INFINITY;
  float* op = a.out + (bh * a.Lq + qi) * kDv;
#pragma unroll
  for (int d = 0; d < kDv; ++d) op[d] = o[d] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const AttnF32Args& a, hipStream_t s) {
  dim3 grid((a.Lq + kQ - 1) / kQ, a.H, a.B);
  hipLaunchKernelGGL(attn_fwd_f32, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
