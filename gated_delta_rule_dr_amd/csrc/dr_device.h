// Device-side helpers shared by the libdr kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Element i of a q/k/v array that is either fp32 or bf16.
__device__ __forceinline__ float load_qkv(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_o(void* p, int64_t i, float x, bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  else
    static_cast<float*>(p)[i] = x;
}

// 16x16x32 fp16 matrix-core product with fp32 accumulation (CDNA4).
// Lane l supplies A[row = l % 16][k = 8 * (l / 16) + 0..7] and B[k = 8 * (l / 16) + 0..7]
// [col = l % 16]; it receives D[row = 4 * (l / 16) + 0..3][col = l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace dr
