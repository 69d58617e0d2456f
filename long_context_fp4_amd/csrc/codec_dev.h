// Scalar codec helpers shared by the cache writers (device code, gfx950).
#pragma once
#include "device.h"
#include <math.h>

namespace csa2 {

// Nearest-even E4M3FN of a finite v >= 0, saturating at 448. Returns the byte
// and the exact value in *val.
__device__ __forceinline__ uint32_t e4m3fn_rne(float v, float* val) {
  if (v >= 448.0f) { *val = 448.0f; return 0x7Eu; }
  if (v < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    float k = rintf(v * 512.0f);             // exact scaling, round half to even
    *val = k * (1.0f / 512.0f);
    return (uint32_t)k;                      // k == 8 is the byte of 2^-6
  }
  uint32_t b = __float_as_uint(v);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;   // keep 3 mantissa bits
  float rv = __uint_as_float(r);
  if (rv > 448.0f) { *val = 448.0f; return 0x7Eu; }
  *val = rv;
  int e = (int)(r >> 23) - 127;
  return ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
}

// floor(log2(a)) of a finite a > 0, exact (handles float32 subnormals).
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t b = __float_as_uint(a);
  int e = (int)(b >> 23);
  if (e > 0) return e - 127;
  return 31 - __clz(b) - 149;
}

}  // namespace csa2
