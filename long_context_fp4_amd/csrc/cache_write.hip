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
// latent (16 lanes per entry), wave 4 owns the indexer key (4 lanes per
// entry). Every lane merges 32 channels of m rows with 16-byte loads laid out
// so that each load instruction covers whole contiguous stretches of the rows
// (a streaming load never leaves a line half read), and writes its codes as
// 4-byte words that are contiguous across the lanes of an entry.
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
#include "codec_dev.h"
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

// Lane mapping. Latent (waves 0-3): 16 lanes per entry; lane p takes the 8
// channels 128q + 8p .. +7 for q = 0..3, so each 16-byte load instruction of
// the 16 lanes reads 256 contiguous bytes of a row, and a 16-channel scale
// block (channels 16b .. 16b+15, b = 8q + p/2) is split over the lane pair
// p, p^1. Indexer (wave 4): 4 lanes per entry; lane p takes channels
// 32q + 8p .. +7, so a 32-channel MX block q is split over the lane quad.
// Block maxima are combined across lanes with DPP swaps (max is exact, so
// the result does not depend on the split).
struct LaneMap {
  bool latent;
  int el, p, C, qstride;
  __device__ explicit LaneMap(int tid)
      : latent(tid < 256), el(tid < 256 ? (tid >> 4) : ((tid - 256) >> 2)),
        p(tid < 256 ? (tid & 15) : ((tid - 256) & 3)), C(tid < 256 ? 512 : 128), qstride(tid < 256 ? 128 : 32) {}
};

// Stages the merge weights ([m][512] latent then [m][128] indexer) in LDS;
// every thread of the workgroup calls it (the caller's barrier follows).
__device__ __forceinline__ void stage_weights(float* lds_w, const float* w_lat, const float* w_idx, int m) {
  for (int k = threadIdx.x; k < m * 128; k += CW_THREADS) {
    ((float4*)lds_w)[k] = ((const float4*)w_lat)[k];
    if (k < m * 32) ((float4*)(lds_w + m * 512))[k] = ((const float4*)w_idx)[k];
  }
}

// This lane's share of one entry, one 8-channel group q at a time (channels
// qstride*q + 8p .. +7): merge the m rows (rowq(j, q): the 8 bf16 of group q
// of row j), take the block maximum across the lanes of the block, pack.
// Working group by group keeps few values live, so more waves fit a SIMD.
// With `store` unset the lane still takes part in the lane exchanges. Codes go
// to the entry's rows kv_e / ik_e / iks_e, latent scale bytes to scale_e (LDS,
// 32 bytes per entry, stored by the caller).
template <int M, typename RowQ>
__device__ __forceinline__ void merge_pack(const LaneMap& L, bool store, int m, const float* lds_w, RowQ rowq,
                                           uint8_t* kv_e, uint8_t* ik_e, uint8_t* iks_e, uint8_t* scale_e) {
  const float* wb = L.latent ? lds_w : lds_w + m * 512;
  const int p = L.p;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    if (store) {
#pragma unroll
      for (int j = 0; j < m; ++j) {
        const u32x4_t xv = rowq(j, q);
        const float4* wp = (const float4*)(wb + (int64_t)j * L.C + L.qstride * q + 8 * p);
        const float4 wa = wp[0], wc = wp[1];
        const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wc.x, wc.y, wc.z, wc.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t d = xv[h];
          const float x0 = bf16_to_f32(d & 0xFFFFu), x1 = bf16_to_f32(d >> 16);
          if (j == 0) {
            acc[2 * h] = wv[2 * h] * x0;
            acc[2 * h + 1] = wv[2 * h + 1] * x1;
          } else {
            acc[2 * h] = acc[2 * h] + wv[2 * h] * x0;
            acc[2 * h + 1] = acc[2 * h + 1] + wv[2 * h + 1] * x1;
          }
        }
      }
    }
    // the lane's amax, combined over the lanes of its block
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaxf(a, fabsf(acc[c]));
    uint32_t ab = __float_as_uint(a);                 // a >= 0: the bits order like the values
    ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp((int)ab, (int)ab, 0xB1, 0xf, 0xf, false));   // lane ^ 1
    if (!L.latent) ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp((int)ab, (int)ab, 0x4E, 0xf, 0xf, false));   // lane ^ 2
    const float amax = __uint_as_float(ab);
    if (L.latent) {
      float s;
      const uint32_t sb = e4m3fn_rne(amax / 6.0f, &s);
      Thresholds th(s);
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float x = acc[c];
        const uint32_t code = th.mag(fabsf(x)) | ((__float_as_uint(x) >> 28) & 8u);
        word |= code << (4 * c);
      }
      if (!(s > 0.0f)) word = 0u;
      if (store) {
        *(uint32_t*)(kv_e + 64 * q + 4 * p) = word;
        if ((p & 1) == 0) scale_e[8 * q + (p >> 1)] = (uint8_t)sb;
      }
    } else {
      uint32_t xbyte = 0;
      float s = 0.0f;
      if (amax > 0.0f) {
        const int X = floor_log2(amax) - 2;
        int bb = X + 127;
        bb = bb < 0 ? 0 : (bb > 254 ? 254 : bb);
        xbyte = (uint32_t)bb;
        s = ldexpf(1.0f, bb - 127);
      }
      Thresholds th(s);
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float x = acc[c];
        const uint32_t code = th.mag(fabsf(x)) | ((__float_as_uint(x) >> 28) & 8u);
        word |= code << (4 * c);
      }
      if (!(amax > 0.0f)) word = 0u;
      if (store) {
        *(uint32_t*)(ik_e + 16 * q + 4 * p) = word;
        if (p == 0) iks_e[q] = (uint8_t)xbyte;
      }
    }
  }
}

// 16 entries x 32 scale bytes from LDS = 32 stores of 16 B (threads 0..31);
// row_of(ent) gives the cache row of entry slot ent, or -1 to skip it.
template <typename RowOf>
__device__ __forceinline__ void store_scales(const uint32_t (*lds_scale)[8], uint8_t* kv, RowOf row_of) {
  if (threadIdx.x < 2 * CW_ENTRIES) {
    const int ent = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t r = row_of(ent);
    if (r >= 0) {
      u32x4_t v = {lds_scale[ent][4 * half + 0], lds_scale[ent][4 * half + 1], lds_scale[ent][4 * half + 2],
                   lds_scale[ent][4 * half + 3]};
      *(u32x4_t*)(kv + r * 288 + 256 + 16 * half) = v;
    }
  }
}

template <int M>
__global__ __launch_bounds__(CW_THREADS) void cache_write_kernel(
    const uint16_t* __restrict__ x_lat, const uint16_t* __restrict__ x_idx,
    const float* __restrict__ w_lat, const float* __restrict__ w_idx,
    int64_t n_total, int64_t E, int64_t T, int m_rt,
    uint8_t* __restrict__ kv, uint8_t* __restrict__ ik, uint8_t* __restrict__ iks) {
  const int m = M > 0 ? M : m_rt;
  __shared__ uint32_t lds_scale[CW_ENTRIES][8];   // 32 latent scale bytes per entry
  // the merge weights, staged once per workgroup (every entry uses the same ones)
  extern __shared__ __attribute__((aligned(16))) float lds_w[];

  const LaneMap L(threadIdx.x);
  const int64_t e = (int64_t)blockIdx.x * CW_ENTRIES + L.el;
  const bool valid = e < n_total;
  const int64_t eb = valid ? e / E : 0, ei = valid ? e - eb * E : 0;
  const int64_t row0 = eb * T + ei * (int64_t)m;
  const uint16_t* xb = (L.latent ? x_lat : x_idx) + row0 * L.C + 8 * L.p;

  // with m fixed at compile time, the rows are requested before the weights
  // are staged, so their latency overlaps the staging
  constexpr int MR = M > 0 ? M : 1;
  u32x4_t xr[MR][4];
  if (M > 0 && valid) {
#pragma unroll
    for (int j = 0; j < MR; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xr[j][q] = __builtin_nontemporal_load((const u32x4_t*)(xb + (int64_t)j * L.C + L.qstride * q));
  }
  stage_weights(lds_w, w_lat, w_idx, m);
  __syncthreads();

  merge_pack<M>(
      L, valid, m, lds_w,
      [&](int j, int q) -> u32x4_t {
        return M > 0 ? xr[j < MR ? j : 0][q]
                     : __builtin_nontemporal_load((const u32x4_t*)(xb + (int64_t)j * L.C + L.qstride * q));
      },
      kv + e * 288, ik + e * 64, iks + e * 4, (uint8_t*)&lds_scale[L.el][0]);

  __syncthreads();
  store_scales(lds_scale, kv, [&](int ent) -> int64_t {
    const int64_t e2 = (int64_t)blockIdx.x * CW_ENTRIES + ent;
    return e2 < n_total ? e2 : -1;
  });
}

// Decode-time append ([FP4] section "Le compte par couche": one entry per m
// tokens; a trailing partial group waits): one token per sequence. Workgroup =
// 16 sequences, lanes as in cache_write_kernel. A sequence whose staged count
// plus this token reaches m merges its m - 1 staged rows and the token into
// the entry at row entry_offset[b] + n_entries[b] (when that is below
// `capacity`; otherwise the group is dropped and dropped[b] is set) and
// clears its stage; any other sequence copies the token into stage row
// stage_count[b]. The counters are updated after the workgroup's barrier, by
// one lane per sequence, once every lane has read them. With m == 1 there is
// no stage: every token is an entry.
template <int M>
__global__ __launch_bounds__(CW_THREADS) void cache_append_kernel(
    const uint16_t* __restrict__ x_lat, const uint16_t* __restrict__ x_idx,
    const float* __restrict__ w_lat, const float* __restrict__ w_idx, int B, int m_rt,
    uint16_t* __restrict__ st_lat, uint16_t* __restrict__ st_idx, int32_t* __restrict__ st_count,
    const int64_t* __restrict__ entry_offset, int32_t* __restrict__ n_entries, int64_t capacity,
    uint8_t* __restrict__ kv, uint8_t* __restrict__ ik, uint8_t* __restrict__ iks, int32_t* __restrict__ dropped) {
  const int m = M > 0 ? M : m_rt;
  __shared__ uint32_t lds_scale[CW_ENTRIES][8];
  __shared__ int64_t lds_row[CW_ENTRIES];        // cache row written for each sequence slot, or -1
  extern __shared__ __attribute__((aligned(16))) float lds_w[];

  const LaneMap L(threadIdx.x);
  const int b = blockIdx.x * CW_ENTRIES + L.el;
  const bool seq = b < B;
  const int bs = seq ? b : 0;
  // Every load is issued first (the counters, this token's rows, the staged
  // rows, the weights), so the call waits for one round trip.
  const int32_t cnt_raw = st_count[bs];
  const int32_t ne = n_entries[bs];
  const int64_t eoff = entry_offset[bs];
  const uint16_t* tok = (L.latent ? x_lat : x_idx) + (int64_t)bs * L.C + 8 * L.p;
  uint16_t* stg = (L.latent ? st_lat : st_idx) + (int64_t)bs * (m - 1) * L.C + 8 * L.p;
  u32x4_t tk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) tk[q] = *(const u32x4_t*)(tok + L.qstride * q);
  constexpr int MS = M > 1 ? M - 1 : 1;
  u32x4_t sr[MS][4];
  if (M > 1) {
#pragma unroll
    for (int j = 0; j < MS; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sr[j][q] = *(const u32x4_t*)(stg + (int64_t)j * L.C + L.qstride * q);
  }
  stage_weights(lds_w, w_lat, w_idx, m);
  // (a count outside [0, m-1] is taken as m-1, so no access leaves the stage)
  const int cnt = seq ? min(max((int)cnt_raw, 0), m - 1) : 0;
  const bool complete = seq && cnt + 1 >= m;
  const bool write = complete && ne >= 0 && (int64_t)ne < capacity;
  const int64_t row = write ? eoff + ne : -1;
  if (seq && !complete) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4_t*)(stg + (int64_t)cnt * L.C + L.qstride * q) = tk[q];
  }
  if (L.latent && L.p == 0) lds_row[L.el] = row;
  __syncthreads();

  const int64_t r = write ? row : 0;
  merge_pack<M>(
      L, write, m, lds_w,
      [&](int j, int q) -> u32x4_t {
        if (j == m - 1) return tk[q];
        if (M > 1) return sr[j < MS ? j : 0][q];
        return *(const u32x4_t*)(stg + (int64_t)j * L.C + L.qstride * q);
      },
      kv + r * 288, ik + r * 64, iks + r * 4, (uint8_t*)&lds_scale[L.el][0]);

  __syncthreads();
  store_scales(lds_scale, kv, [&](int ent) -> int64_t { return lds_row[ent]; });
  if (seq && L.latent && L.p == 0) {
    st_count[b] = complete ? 0 : cnt + 1;
    if (write) n_entries[b] = ne + 1;
    if (dropped) dropped[b] = complete && !write ? 1 : 0;
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
  const size_t lds = (size_t)m * 640 * sizeof(float);   // the staged merge weights
  switch (m) {
    case 1: hipLaunchKernelGGL(cache_write_kernel<1>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    case 2: hipLaunchKernelGGL(cache_write_kernel<2>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    case 4: hipLaunchKernelGGL(cache_write_kernel<4>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
    default: hipLaunchKernelGGL(cache_write_kernel<0>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, n_total, E, T, m, kv, ik, iks); break;
  }
  return hipGetLastError();
}

hipError_t launch_cache_append(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                               const float* w_idx, int B, int m, uint16_t* st_lat, uint16_t* st_idx,
                               int32_t* st_count, const int64_t* entry_offset, int32_t* n_entries,
                               int64_t capacity, uint8_t* kv, uint8_t* ik, uint8_t* iks, int32_t* dropped,
                               hipStream_t stream) {
  dim3 grid((unsigned)((B + CW_ENTRIES - 1) / CW_ENTRIES)), block(CW_THREADS);
  const size_t lds = (size_t)m * 640 * sizeof(float);
#define CSA2_APPEND(Mv)                                                                                  \
  hipLaunchKernelGGL(cache_append_kernel<Mv>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, B, m, \
                     st_lat, st_idx, st_count, entry_offset, n_entries, capacity, kv, ik, iks, dropped)
  switch (m) {
    case 1: CSA2_APPEND(1); break;
    case 2: CSA2_APPEND(2); break;
    case 4: CSA2_APPEND(4); break;
    default: CSA2_APPEND(0); break;
  }
#undef CSA2_APPEND
  return hipGetLastError();
}

}  // namespace csa2
