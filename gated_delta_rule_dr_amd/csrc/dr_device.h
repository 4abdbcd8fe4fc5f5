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

// Four consecutive outputs (16-byte aligned for fp32, 8-byte for bf16).
__device__ __forceinline__ void store_o4(void* p, int64_t i, f32x4 x, bool bf16) {
  if (bf16) {
    uint2 w;
    w.x = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
    w.y = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = x;
  }
}

// Loads n = RPL contiguous q/k elements starting at element `i` into `out` (vector loads:
// the ABI guarantees 16-byte aligned bases, and i is a multiple of RPL >= 4).
template <int RPL>
__device__ __forceinline__ void load_rows(const void* base, int64_t i, bool bf16, float* out) {
  if (bf16) {
    const uint2* p = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int r = 0; r < RPL / 4; ++r) {
      uint2 x = p[r];
      out[4 * r + 0] = __uint_as_float(x.x << 16);
      out[4 * r + 1] = __uint_as_float(x.x & 0xffff0000u);
      out[4 * r + 2] = __uint_as_float(x.y << 16);
      out[4 * r + 3] = __uint_as_float(x.y & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
#pragma unroll
    for (int r = 0; r < RPL / 4; ++r) {
      float4 x = p[r];
      out[4 * r + 0] = x.x;
      out[4 * r + 1] = x.y;
      out[4 * r + 2] = x.z;
      out[4 * r + 3] = x.w;
    }
  }
}

template <int RPL>
__device__ __forceinline__ void load_f32_rows(const float* base, int64_t i, float* out) {
  const float4* p = reinterpret_cast<const float4*>(base + i);
#pragma unroll
  for (int r = 0; r < RPL / 4; ++r) {
    float4 x = p[r];
    out[4 * r + 0] = x.x;
    out[4 * r + 1] = x.y;
    out[4 * r + 2] = x.z;
    out[4 * r + 3] = x.w;
  }
}

// 16x16x32 fp16 matrix-core product with fp32 accumulation (CDNA4).
// Lane l supplies A[row = l % 16][k = 8 * (l / 16) + 0..7] and B[k = 8 * (l / 16) + 0..7]
// [col = l % 16]; it receives D[row = 4 * (l / 16) + 0..3][col = l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations and meets the
// other waves, but leaves global loads in flight (a __syncthreads() fence would also wait for
// every outstanding global load, which defeats prefetching the next chunk across stages).  The
// memory clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Global-address-space pointer.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

// Returns `p` as a global pointer passed through an empty asm, so the compiler no longer knows
// the pointee is read-only for the whole kernel.  Loads through the result are then ordinary
// global loads that lds_barrier() keeps in place, instead of invariant loads the compiler may
// sink to their first use (which would turn a next-chunk prefetch into a stall).
template <typename T>
__device__ __forceinline__ gptr<T> opaque_gptr(T* p) {
  gptr<T> g = (gptr<T>)p;
  asm volatile("" : "+s"(g));
  return g;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Vector loads from global element `i` of `base` (16 or 8 bytes, element type T).
template <typename T>
__device__ __forceinline__ uint4 gload_u4(gptr<const T> base, int64_t i) {
  const u32x4 x = *(gptr<const u32x4>)(base + i);
  return make_uint4(x.x, x.y, x.z, x.w);
}
template <typename T>
__device__ __forceinline__ uint2 gload_u2(gptr<const T> base, int64_t i) {
  const u32x2 x = *(gptr<const u32x2>)(base + i);
  return make_uint2(x.x, x.y);
}
__device__ __forceinline__ float4 gload_f4(gptr<const float> base, int64_t i) {
  const f32x4 x = *(gptr<const f32x4>)(base + i);
  return make_float4(x.x, x.y, x.z, x.w);
}

}  // namespace dr
