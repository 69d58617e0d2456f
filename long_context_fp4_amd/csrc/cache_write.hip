// Fused ratio-m merge + FP4 quantization + packing of the compressed global
// KV cache, for gfx950.
//
// What is computed ("Le cache KV en FP4 — les 890 octets, vérifiés", sections
// "Le coût d'une entrée" and "Le compte par couche"; "DeepSeek-V4.1 Flash
// compresse le KV-Cache de 4 fois", section "Mécanismes de compression du
// KV-Cache", item 2): every m consecutive hidden rows are merged channel by
// channel with learned weights into one entry; the 512-channel latent is
// packed as E2M1 codes with one E4M3FN scale per 16 channels (288 B), the
// 128-channel indexer key as E2M1 codes with one E8M0 scale per 32 channels
// (64 B of codes + 4 B of scales).
//
// Work layout: one workgroup of 320 lanes packs 16 entries. Waves 0-3 own the
// latent (16 lanes per entry, 32 channels = two scale blocks per lane), wave 4
// owns the indexer key (4 lanes per entry, 32 channels = one MX block per
// lane). Every lane therefore merges 32 channels of m rows: m x 64 B of
// contiguous bf16 loads and one 16 B store of codes, so the reads of a row and
// the writes of the code bytes are fully coalesced 128-bit accesses.
//
// Bit-exactness: the merge is evaluated with separate float32 roundings
// (contraction is switched off for this file), the scale division is the
// correctly rounded float32 division, and the E2M1 code of x/s is decided by
// exact comparisons of |x| against t*s for the seven rounding thresholds t of
// the E2M1 grid. t*s is exact in float32 (t has at most 3 significant bits,
// an E4M3 scale at most 4), and for |x| and s in float32 no quotient |x|/s can
// lie strictly between a threshold and the float32 rounding boundary next to
// it (the smallest gap |x|/s - t is ulp(|x|)/s, which exceeds half an ulp of t
// because the scale's significand is below 2), so these comparisons give the
// same code as rounding the float32 quotient. Thresholds where the tie goes
// down use '>', those where it goes up use '>='.
#include "device.h"
#include <math.h>

#pragma clang fp contract(off)

namespace csa2 {

constexpr int CW_ENTRIES = 16;
constexpr int CW_THREADS = 320;

// E2M1 magnitude code of |x| for block scale s (s > 0), via the thresholds
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times s.
struct Thresholds {
  float t0, t1, t2, t3, t4, t5, t6;
  __device__ __forceinline__ explicit Thresholds(float s)
      : t0(0.25f * s), t1(0.75f * s), t2(1.25f * s), t3(1.75f * s),
        t4(2.5f * s), t5(3.5f * s), t6(5.0f * s) {}
  __device__ __forceinline__ uint32_t mag(float a) const {
    return (uint32_t)(a > t0) + (uint32_t)(a >= t1) + (uint32_t)(a > t2) + (uint32_t)(a >= t3) +
           (uint32_t)(a > t4) + (uint32_t)(a >= t5) + (uint32_t)(a > t6);
  }
};

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

template <int M>
__global__ __launch_bounds__(CW_THREADS) void cache_write_kernel(
    const uint16_t* __restrict__ x_lat, const uint16_t* __restrict__ x_idx,
    const float* __restrict__ w_lat, const float* __restrict__ w_idx,
    int64_t n_total, int64_t E, int64_t T, int m_rt,
    uint8_t* __restrict__ kv, uint8_t* __restrict__ ik, uint8_t* __restrict__ iks) {
  const int m = M > 0 ? M : m_rt;
  __shared__ uint32_t lds_scale[CW_ENTRIES][8];   // 32 latent scale bytes per entry

  const int tid = threadIdx.x;
  const bool latent = tid < 256;
  const int el = latent ? (tid >> 4) : ((tid - 256) >> 2);
  const int part = latent ? (tid & 15) : ((tid - 256) & 3);
  const int C = latent ? 512 : 128;
  const int64_t e = (int64_t)blockIdx.x * CW_ENTRIES + el;
  const bool valid = e < n_total;

  float acc[32];
  if (valid) {
    const int64_t b = e / E, i = e - b * E;
    const int64_t row0 = b * T + i * (int64_t)m;
    const uint16_t* xb = latent ? x_lat : x_idx;
    const float* wb = latent ? w_lat : w_idx;
#pragma unroll
    for (int j = 0; j < m; ++j) {
      const u32x4_t* src = (const u32x4_t*)(xb + (row0 + j) * C + part * 32);
      const float4* wp = (const float4*)(wb + (int64_t)j * C + part * 32);
      u32x4_t xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[q] = __builtin_nontemporal_load(src + q);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float4 wv = wp[q];
        uint32_t d0 = xv[q >> 1][(q & 1) * 2], d1 = xv[q >> 1][(q & 1) * 2 + 1];
        float x0 = bf16_to_f32(d0 & 0xFFFFu), x1 = bf16_to_f32(d0 >> 16);
        float x2 = bf16_to_f32(d1 & 0xFFFFu), x3 = bf16_to_f32(d1 >> 16);
        if (j == 0) {
          acc[4 * q + 0] = wv.x * x0; acc[4 * q + 1] = wv.y * x1;
          acc[4 * q + 2] = wv.z * x2; acc[4 * q + 3] = wv.w * x3;
        } else {
          acc[4 * q + 0] = acc[4 * q + 0] + wv.x * x0; acc[4 * q + 1] = acc[4 * q + 1] + wv.y * x1;
          acc[4 * q + 2] = acc[4 * q + 2] + wv.z * x2; acc[4 * q + 3] = acc[4 * q + 3] + wv.w * x3;
        }
      }
    }
  }

  if (latent) {
    uint32_t codes[4];
    uint32_t sbytes = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(acc[16 * blk + c]));
      float s;
      uint32_t sb = e4m3fn_rne(amax / 6.0f, &s);
      sbytes |= sb << (8 * blk);
      Thresholds th(s);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float x = acc[16 * blk + 8 * d + c];
          uint32_t code = th.mag(fabsf(x)) | ((__float_as_uint(x) >> 28) & 8u);
          word |= code << (4 * c);
        }
        codes[2 * blk + d] = (s > 0.0f) ? word : 0u;
      }
    }
    if (valid) {
      u32x4_t out = {codes[0], codes[1], codes[2], codes[3]};
      *(u32x4_t*)(kv + e * 288 + part * 16) = out;
      ((uint16_t*)&lds_scale[el][0])[part] = (uint16_t)sbytes;
    }
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(acc[c]));
    uint32_t xbyte = 0;
    float s = 0.0f;
    if (amax > 0.0f) {
      int X = floor_log2(amax) - 2;
      int bb = X + 127;
      bb = bb < 0 ? 0 : (bb > 254 ? 254 : bb);
      xbyte = (uint32_t)bb;
      s = ldexpf(1.0f, bb - 127);
    }
    Thresholds th(s);
    uint32_t codes[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float x = acc[8 * d + c];
        uint32_t code = th.mag(fabsf(x)) | ((__float_as_uint(x) >> 28) & 8u);
        word |= code << (4 * c);
      }
      codes[d] = (amax > 0.0f) ? word : 0u;
    }
    if (valid) {
      u32x4_t out = {codes[0], codes[1], codes[2], codes[3]};
      *(u32x4_t*)(ik + e * 64 + part * 16) = out;
      iks[e * 4 + part] = (uint8_t)xbyte;
    }
  }

  __syncthreads();
  // 16 entries x 32 scale bytes = 32 stores of 16 B
  if (tid < 32) {
    const int ent = tid >> 1, half = tid & 1;
    const int64_t e2 = (int64_t)blockIdx.x * CW_ENTRIES + ent;
    if (e2 < n_total) {
      u32x4_t v = {lds_scale[ent][4 * half + 0], lds_scale[ent][4 * half + 1],
                   lds_scale[ent][4 * half + 2], lds_scale[ent][4 * half + 3]};
      *(u32x4_t*)(kv + e2 * 288 + 256 + 16 * half) = v;
    }
  }
}

hipError_t launch_cache_write(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                              const float* w_idx, int B, int64_t T, int m, uint8_t* kv, uint8_t* ik,
                              uint8_t* iks, hipStream_t stream) {
  const int64_t E = T / m;
  const int64_t n_total = (int64_t)B * E;
  if (n_total == 0) return hipSuccess;
  const int64_t blocks = (n_total + CW_ENTRIES - 1) / CW_ENTRIES;
  dim3 grid((unsigned)blocks), block(CW_THREADS);
  switch (m) {
    case 1: hipLaunchKernelGGL(cache_write_kernel<1>, grid, block, 0, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    case 2: hipLaunchKernelGGL(cache_write_kernel<2>, grid, block, 0, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    case 4: hipLaunchKernelGGL(cache_write_kernel<4>, grid, block, 0, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    default: hipLaunchKernelGGL(cache_write_kernel<0>, grid, block, 0, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
  }
  return hipGetLastError();
}

}  // namespace csa2
