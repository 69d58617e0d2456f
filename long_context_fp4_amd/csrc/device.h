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
typedef int i32x8_t __attribute__((ext_vector_type(8)));

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

// Wave-wide primitives on VALU lane movement (DPP within rows of 16 lanes,
// v_readlane for the four row results) instead of LDS-routed shuffles.
// DPP controls: row_shr:n = 0x110 + n, quad_perm [1,0,3,2] = 0xB1,
// [2,3,0,1] = 0x4E, row_mirror = 0x140, row_half_mirror = 0x141.
#define CSA2_DPP(old, v, ctrl, rm, bm, bz) \
  ((uint32_t)__builtin_amdgcn_update_dpp((int)(old), (int)(v), (ctrl), (rm), (bm), (bz)))

// Inclusive prefix sum of v over the lanes of the wave.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  uint32_t x = v;
  x += CSA2_DPP(0u, v, 0x111, 0xf, 0xf, true);    // + v[i-1] (0 at a row start)
  x += CSA2_DPP(0u, v, 0x112, 0xf, 0xf, true);    // + v[i-2]
  x += CSA2_DPP(0u, v, 0x113, 0xf, 0xf, true);    // + v[i-3]
  x += CSA2_DPP(0u, x, 0x114, 0xf, 0xe, false);   // lanes 4..15 of a row: + x[i-4]
  x += CSA2_DPP(0u, x, 0x118, 0xf, 0xc, false);   // lanes 8..15 of a row: + x[i-8]
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Reductions over the 16 lanes of each row (every lane of the row gets it).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, CSA2_DPP(0u, v, 0xB1, 0xf, 0xf, false));
  v = max(v, CSA2_DPP(0u, v, 0x4E, 0xf, 0xf, false));
  v = max(v, CSA2_DPP(0u, v, 0x141, 0xf, 0xf, false));
  return max(v, CSA2_DPP(0u, v, 0x140, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t row_or_u32(uint32_t v) {
  v |= CSA2_DPP(0u, v, 0xB1, 0xf, 0xf, false);
  v |= CSA2_DPP(0u, v, 0x4E, 0xf, 0xf, false);
  v |= CSA2_DPP(0u, v, 0x141, 0xf, 0xf, false);
  return v | CSA2_DPP(0u, v, 0x140, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row_and_u32(uint32_t v) {
  v &= CSA2_DPP(0u, v, 0xB1, 0xf, 0xf, false);
  v &= CSA2_DPP(0u, v, 0x4E, 0xf, 0xf, false);
  v &= CSA2_DPP(0u, v, 0x141, 0xf, 0xf, false);
  return v & CSA2_DPP(0u, v, 0x140, 0xf, 0xf, false);
}
__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(CSA2_DPP(0u, __float_as_uint(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __uint_as_float(CSA2_DPP(0u, __float_as_uint(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __uint_as_float(CSA2_DPP(0u, __float_as_uint(v), 0x141, 0xf, 0xf, false)));
  return fmaxf(v, __uint_as_float(CSA2_DPP(0u, __float_as_uint(v), 0x140, 0xf, 0xf, false)));
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
// Wave-uniform max / or / and of v.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max_u32(v);
  return max(max(readlane_u32(v, 0), readlane_u32(v, 16)), max(readlane_u32(v, 32), readlane_u32(v, 48)));
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v = row_or_u32(v);
  return readlane_u32(v, 0) | readlane_u32(v, 16) | readlane_u32(v, 32) | readlane_u32(v, 48);
}
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v) {
  v = row_and_u32(v);
  return readlane_u32(v, 0) & readlane_u32(v, 16) & readlane_u32(v, 32) & readlane_u32(v, 48);
}

template <typename T>
__device__ __forceinline__ T bitcast_u32(uint32_t v) { T r; __builtin_memcpy(&r, &v, 4); return r; }

}  // namespace csa2
