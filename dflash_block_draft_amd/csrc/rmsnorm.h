// RMSNorm pieces shared by the kernels that apply a norm to their operands as
// they load them (Kimi RMSNorm: fp32 variance of the bf16 input, the normalised
// value returned in the input dtype, then multiplied by the bf16 weight;
// DFlash page, module text).
#pragma once

#include "common.h"

namespace dflash {

// 8 bf16 entries x of one row -> bf16(bf16(x * r) * gamma)
__device__ __forceinline__ u32x4_t rms_norm_chunk(u32x4_t x, float r, u32x4_t g) {
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t xn = pack_bf16x2(bf16_bits_to_f32(x[j] & 0xFFFFu) * r, bf16_bits_to_f32(x[j] >> 16) * r);
    o[j] = pack_bf16x2(bf16_bits_to_f32(xn & 0xFFFFu) * bf16_bits_to_f32(g[j] & 0xFFFFu),
                       bf16_bits_to_f32(xn >> 16) * bf16_bits_to_f32(g[j] >> 16));
  }
  return o;
}

// r = rsqrt(mean of squares + eps) of row m from its partial sums of squares
// (stats[m * parts + p], summed in p order) over K entries.
__device__ __forceinline__ float rms_row_scale(const float* stats, int parts, int64_t m, int K, float eps) {
  float s = 0.f;
  for (int p = 0; p < parts; ++p) s += stats[m * parts + p];
  return rsqrtf(s / static_cast<float>(K) + eps);
}

}  // namespace dflash
