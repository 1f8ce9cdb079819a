// Device-side building blocks shared by the gfx950 kernels of the draft MLA attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dims.h"

namespace dflash {


constexpr float kLog2e = 1.4426950408889634f;

// A tile-list entry packs the k-tile index in its low 24 bits and the class above.
constexpr int kMaxKeyTiles = (1 << 24) - 1;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 32x32x16 bf16 MFMA, fp32 accumulate: C[32x32] += A[32x16] * B[16x32].
// Lane l supplies A row (l % 32), B column (l % 32), and k = 8*(l / 32) + 0..7.
// Result: lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even; lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Byte select: result = { lo16(x), lo16(y) } and { hi16(x), hi16(y) }.
__device__ __forceinline__ uint32_t lo16_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void stg16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

}  // namespace dflash
