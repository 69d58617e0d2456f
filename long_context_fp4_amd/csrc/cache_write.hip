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
// Work layout: one workgroup of 320 lanes packs 16 consecutive entries of one
// sequence. Waves 0-3 own the latent (16 lanes per entry), wave 4 owns the
// indexer key (4 lanes per entry). Every lane merges 32 channels of m rows with
// 16-byte loads laid out so that each load instruction covers whole contiguous
// stretches of the rows (a streaming load never leaves a line half read), and
// puts its codes into the entry's row assembled in LDS; the workgroup then
// writes its 16 rows (4608 + 1024 contiguous bytes) with 16-byte stores.
//
// Bit-exactness: the merge is evaluated with separate float32 roundings
// (contraction is switched off for this file). The E2M1 code of a latent
// value x is the nearest-even E2M1 value (saturating at 6) of the correctly
// rounded float32 quotient x / s: the quotient comes from one multiply by the
// correctly rounded reciprocal of s and Markstein's correction step (two fused
// multiply-adds), and gfx950's f32 -> FP4 conversion (nearest even, ties to
// even, saturating, sign kept also for zero; checked against the rounding
// thresholds of every E4M3 scale) turns two quotients into one code byte. An
// indexer value is scaled by 2^-X exactly (ldexp) and converted the same way.
#include "device.h"
#include "codec_dev.h"
#include <math.h>

#pragma clang fp contract(off)

namespace csa2 {

constexpr int CW_ENTRIES = 16;
constexpr int CW_THREADS = 320;

// The correctly rounded quotient x / s for an E4M3 scale s > 0, given
// y = 1 / s correctly rounded: q = x y; t = q s - x (exact, one fused
// multiply-add); q - t y is then the correctly rounded quotient (Markstein's
// correction step; it holds whenever no intermediate underflows, and an
// underflow only touches quotients far below the first rounding threshold).
// The order of the two fused operations keeps the sign of a zero quotient.
// No overflow: |x| is at most the block maximum, so |x| y stays below 2^128
// for every scale the block maximum can round to.
__device__ __forceinline__ float quotient(float x, float s, float y) {
  const float q = x * y;
  const float t = fmaf(q, s, -x);
  return fmaf(-t, y, q);
}

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

// The packed rows of a workgroup's 16 entries are assembled in LDS and then
// written with 16-byte stores. Row pitches are chosen so that the 4-byte code
// words of the lanes of one wave fall on distinct banks (latent: 80 words,
// four entries per wave 16 banks apart; indexer: 20 words, the 64 lanes of
// wave 4 on 64 distinct banks).
constexpr int CW_LAT_PITCH = 320;   // bytes per staged latent row (288 used)
constexpr int CW_IDX_PITCH = 80;    // bytes per staged indexer row (64 used)
struct alignas(16) Staging {
  uint8_t lat[CW_ENTRIES * CW_LAT_PITCH];
  uint8_t idx[CW_ENTRIES * CW_IDX_PITCH];
  uint32_t iks[CW_ENTRIES];
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
// With `store` unset the lane still takes part in the lane exchanges. The
// codes and scale bytes go to the entry's staged rows in LDS.
template <int M, typename RowQ>
__device__ __forceinline__ void merge_pack(const LaneMap& L, bool store, int m, const float* lds_w, RowQ rowq,
                                           Staging& st) {
  const float* wb = L.latent ? lds_w : lds_w + m * 512;
  const int p = L.p;
  uint8_t* lat_e = st.lat + L.el * CW_LAT_PITCH;
  uint8_t* idx_e = st.idx + L.el * CW_IDX_PITCH;
  uint32_t xbytes = 0;                                  // indexer: the 4 E8M0 bytes of the entry
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
      // codes of the correctly rounded quotients x / s (two channels per conversion)
      const float y = 1.0f / s;
      uint32_t word = 0;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, quotient(acc[0], s, y), quotient(acc[1], s, y), 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, quotient(acc[2], s, y), quotient(acc[3], s, y), 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, quotient(acc[4], s, y), quotient(acc[5], s, y), 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, quotient(acc[6], s, y), quotient(acc[7], s, y), 1.0f, 3);
      if (!(s > 0.0f)) word = 0u;
      // the scale bytes of blocks 8q + 2k and 8q + 2k + 1 (lanes 4k and
      // 4k + 2) meet in lane 4k, which stores them as one 16-bit word
      const uint32_t sb2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x4E, 0xf, 0xf, false);   // lane ^ 2
      if (store) {
        *(uint32_t*)(lat_e + 64 * q + 4 * p) = word;
        if ((p & 3) == 0) *(uint16_t*)(lat_e + 256 + 8 * q + (p >> 1)) = (uint16_t)(sb | (sb2 << 8));
      }
    } else {
      uint32_t xbyte = 0;
      if (amax > 0.0f) {
        const int X = floor_log2(amax) - 2;
        int bb = X + 127;
        bb = bb < 0 ? 0 : (bb > 254 ? 254 : bb);
        xbyte = (uint32_t)bb;
      }
      // x * 2^-X is exact (the values lie below 8: no overflow; an underflow
      // only touches values far below the first rounding threshold)
      const int nx = 127 - (int)xbyte;
      uint32_t word = 0;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(acc[0], nx), ldexpf(acc[1], nx), 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(acc[2], nx), ldexpf(acc[3], nx), 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(acc[4], nx), ldexpf(acc[5], nx), 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(acc[6], nx), ldexpf(acc[7], nx), 1.0f, 3);
      if (!(amax > 0.0f)) word = 0u;
      xbytes |= xbyte << (8 * q);
      if (store) *(uint32_t*)(idx_e + 16 * q + 4 * p) = word;
    }
  }
  if (!L.latent && store && p == 0) st.iks[L.el] = xbytes;
}

// Writes the staged rows of the workgroup's entries with 16-byte non-temporal
// stores (the written cache is not read back by this launch; plain stores
// made the write128k launch ~4 % slower), the E8M0 bytes with one 4-byte store
// per entry. row_of(ent) gives the cache row
// of entry slot ent, or -1 to skip it. Every thread calls it after a barrier.
template <typename RowOf>
__device__ __forceinline__ void store_staged(const Staging& st, uint8_t* kv, uint8_t* ik, uint8_t* iks,
                                             RowOf row_of) {
  constexpr int LAT_CHUNKS = CW_ENTRIES * 18;         // 288 B = 18 x 16 B per latent row
  constexpr int IDX_CHUNKS = CW_ENTRIES * 4;          // 64 B = 4 x 16 B per indexer row
  constexpr int TASKS = LAT_CHUNKS + IDX_CHUNKS + CW_ENTRIES;
  for (int t = threadIdx.x; t < TASKS; t += CW_THREADS) {
    if (t < LAT_CHUNKS) {
      const int ent = t / 18, c = t - 18 * (t / 18);
      const int64_t r = row_of(ent);
      if (r >= 0)
        __builtin_nontemporal_store(*(const u32x4_t*)(st.lat + ent * CW_LAT_PITCH + 16 * c), (u32x4_t*)(kv + r * 288 + 16 * c));
    } else if (t < LAT_CHUNKS + IDX_CHUNKS) {
      const int u = t - LAT_CHUNKS, ent = u >> 2, c = u & 3;
      const int64_t r = row_of(ent);
      if (r >= 0)
        __builtin_nontemporal_store(*(const u32x4_t*)(st.idx + ent * CW_IDX_PITCH + 16 * c), (u32x4_t*)(ik + r * 64 + 16 * c));
    } else {
      const int ent = t - LAT_CHUNKS - IDX_CHUNKS;
      const int64_t r = row_of(ent);
      if (r >= 0) *(uint32_t*)(iks + r * 4) = st.iks[ent];
    }
  }
}

// Grid (entry blocks of 16, sequences). Sequence b's rows are x[b*T ..
// b*T + n_b - 1] with n_b = n_tokens[b] clamped to [0, T] (T when n_tokens is
// NULL); it gets floor(n_b / m) entries, written at cache rows row0_b + i with
// row0_b = out_off[b] (b * floor(T / m) when out_off is NULL).
template <int M>
__global__ __launch_bounds__(CW_THREADS) void cache_write_kernel(
    const uint16_t* __restrict__ x_lat, const uint16_t* __restrict__ x_idx,
    const float* __restrict__ w_lat, const float* __restrict__ w_idx, int64_t T, int m_rt,
    const int64_t* __restrict__ n_tokens, const int64_t* __restrict__ out_off,
    uint8_t* __restrict__ kv, uint8_t* __restrict__ ik, uint8_t* __restrict__ iks) {
  const int m = M > 0 ? M : m_rt;
  __shared__ Staging st;
  // the merge weights, staged once per workgroup (every entry uses the same ones)
  extern __shared__ __attribute__((aligned(16))) float lds_w[];

  const int b = blockIdx.y;
  int64_t nb = T;
  if (n_tokens) nb = min(max(n_tokens[b], (int64_t)0), T);
  const int64_t Eb = nb / m;
  const int64_t e0 = (int64_t)blockIdx.x * CW_ENTRIES;
  if (e0 >= Eb) return;                                // uniform over the workgroup
  const int64_t row0 = (out_off ? out_off[b] : (int64_t)b * (T / m)) + e0;
  const int cnt = (int)min((int64_t)CW_ENTRIES, Eb - e0);

  const LaneMap L(threadIdx.x);
  const bool valid = L.el < cnt;
  const int64_t ei = valid ? e0 + L.el : 0;
  const uint16_t* xb = (L.latent ? x_lat : x_idx) + ((int64_t)b * T + ei * m) * L.C + 8 * L.p;

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
      st);

  __syncthreads();
  store_staged(st, kv, ik, iks, [&](int ent) -> int64_t { return ent < cnt ? row0 + ent : -1; });
}

// Decode-time append ([FP4] section "Le compte par couche": one entry per m
// tokens; a trailing partial group waits): one token per sequence. Workgroup =
// 16 sequences, lanes as in cache_write_kernel. A sequence whose staged count
// plus this token reaches m merges its m - 1 staged rows and the token into
// the entry at row entry_offset[b] + n_entries[b] (when n_entries[b] is below
// its capacity[b]; otherwise the group is dropped and dropped[b] is set) and
// clears its stage; any other sequence copies the token into stage row
// stage_count[b]. The counters are updated after the workgroup's barrier, by
// one lane per sequence, once every lane has read them. With m == 1 there is
// no stage: every token is an entry.
template <int M>
__global__ __launch_bounds__(CW_THREADS) void cache_append_kernel(
    const uint16_t* __restrict__ x_lat, const uint16_t* __restrict__ x_idx,
    const float* __restrict__ w_lat, const float* __restrict__ w_idx, int B, int m_rt,
    uint16_t* __restrict__ st_lat, uint16_t* __restrict__ st_idx, int32_t* __restrict__ st_count,
    const int64_t* __restrict__ entry_offset, int32_t* __restrict__ n_entries, const int64_t* __restrict__ capacity,
    uint8_t* __restrict__ kv, uint8_t* __restrict__ ik, uint8_t* __restrict__ iks, int32_t* __restrict__ dropped) {
  const int m = M > 0 ? M : m_rt;
  __shared__ Staging st;
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
  const int64_t cap = capacity[bs];
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
  const bool write = complete && ne >= 0 && (int64_t)ne < cap;
  const int64_t row = write ? eoff + ne : -1;
  if (seq && !complete) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4_t*)(stg + (int64_t)cnt * L.C + L.qstride * q) = tk[q];
  }
  if (L.latent && L.p == 0) lds_row[L.el] = row;
  __syncthreads();

  merge_pack<M>(
      L, write, m, lds_w,
      [&](int j, int q) -> u32x4_t {
        if (j == m - 1) return tk[q];
        if (M > 1) return sr[j < MS ? j : 0][q];
        return *(const u32x4_t*)(stg + (int64_t)j * L.C + L.qstride * q);
      },
      st);

  __syncthreads();
  store_staged(st, kv, ik, iks, [&](int ent) -> int64_t { return lds_row[ent]; });
  if (seq && L.latent && L.p == 0) {
    st_count[b] = complete ? 0 : cnt + 1;
    if (write) n_entries[b] = ne + 1;
    if (dropped) dropped[b] = complete && !write ? 1 : 0;
  }
}

hipError_t launch_cache_write(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                              const float* w_idx, int B, int64_t T, int m, const int64_t* n_tokens,
                              const int64_t* out_entry_offset, uint8_t* kv, uint8_t* ik, uint8_t* iks,
                              hipStream_t stream) {
  const int64_t E = T / m;                             // entries of the longest possible sequence
  if (E == 0) return hipSuccess;
  dim3 grid((unsigned)((E + CW_ENTRIES - 1) / CW_ENTRIES), (unsigned)B), block(CW_THREADS);
  const size_t lds = (size_t)m * 640 * sizeof(float);   // the staged merge weights
#define CSA2_WRITE(Mv)                                                                                     \
  hipLaunchKernelGGL(cache_write_kernel<Mv>, grid, block, lds, stream, x_lat, x_idx, w_lat, w_idx, T, m, \
                     n_tokens, out_entry_offset, kv, ik, iks)
  switch (m) {
    case 1: CSA2_WRITE(1); break;
    case 2: CSA2_WRITE(2); break;
    case 4: CSA2_WRITE(4); break;
    default: CSA2_WRITE(0); break;
  }
#undef CSA2_WRITE
  return hipGetLastError();
}

hipError_t launch_cache_append(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                               const float* w_idx, int B, int m, uint16_t* st_lat, uint16_t* st_idx,
                               int32_t* st_count, const int64_t* entry_offset, int32_t* n_entries,
                               const int64_t* capacity, uint8_t* kv, uint8_t* ik, uint8_t* iks, int32_t* dropped,
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
