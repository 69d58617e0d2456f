// Device-side helpers shared by the gfx950 kernels of libcsa2fp4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Order-preserving map of a float score to an unsigned key (larger float ->
// larger key). -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Lane shuffles inside a wave (ds_bpermute based).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, WAVE); }
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T bitcast_u32(uint32_t v) { T r; __builtin_memcpy(&r, &v, 4); return r; }

}  // namespace csa2
