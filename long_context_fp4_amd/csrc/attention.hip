// Gather-dequant sparse decode attention over the FP4 latent cache, for gfx950.
//
// What is computed ("DeepSeek-V4.1 Flash compresse le KV-Cache de 4 fois",
// section "Mécanismes de compression du KV-Cache", item 1: one 512-d latent
// shared by keys and values across heads; "Le cache KV en FP4 — les 890
// octets, vérifiés", section "Les ingrédients": the latent serves attention;
// "DeepSeek V4.1 Flash : 890 octets de cache KV par token", section
// "L'architecture : trois leviers contre le cache": attention reads the top-512
// positions): for each head h, logit_i = tau * (q_h . c_i) over the selected
// positions i, o_h = softmax-weighted sum of c_i, lse_h = log sum exp(logit).
//
// Design
// ------
// Workgroup = (sequence, group of 16 heads, split of the index list; a last
// group with fewer heads runs with zero queries in the missing columns); its 4
// waves take 16-entry tiles in turn. Per tile a lane gathers 64 code bytes and
// 8 scale bytes of one entry (a quarter of its 288-byte row) and dequantizes
// them to fp16: the gfx950 scaled FP4->fp16 conversion (which applies a power
// of two exactly) gives 256 * E2M1, and one packed fp16 multiply by the E4M3
// scale / 256 (the E4M3 bit pattern shifted into fp16 position) gives the exact
// latent value (an E2M1 x E4M3 product has at most 6 significant bits and lies
// in [2^-10, 2688], so fp16 holds it exactly).
//   QK^T: v_mfma_f32_16x16x32_f16 with the dequantized tile as the A operand
//   straight from registers and the queries as B. Queries are bf16; each head
//   is multiplied by a power of two that puts its largest magnitude in
//   [2^14, 2^15) before rounding to fp16, so only values below 2^-16 of the
//   head's maximum can lose bits; the power is divided out of the logit.
//   Softmax: online, in fp32, with the running reference maximum raised only
//   when a tile's maximum exceeds it by more than 8 (so P <= e^8 fits fp16 and
//   the 128 accumulators are rescaled rarely).
//   PV: O^T += C^T P^T with v_mfma_f32_16x16x16_f16; P^T comes straight from
//   the QK output registers, C^T is read back from the wave's LDS copy of the
//   tile with gfx950's transposing LDS read (ds_read_b64_tr_b16), which hands
//   every lane 4 entries of one dimension; rows are 1056 B apart so the 16 rows
//   of a read fall on distinct banks.
// The 4 waves' partial states are merged through LDS; with several splits the
// workgroup writes an unnormalised partial that a small kernel combines.
#include "device.h"
#include "kernels.h"
#include <math.h>
#include <atomic>

namespace csa2 {

constexpr int AT_WAVES = 8;                    // two waves per SIMD
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_PITCH = 1056;                 // bytes per entry row of the fp16 tile (rows 8 banks apart)
constexpr int AT_WAVE_LDS = 16 * AT_PITCH;     // 16896
constexpr int AT_LDS = AT_WAVES * AT_WAVE_LDS; // 135168 (>= 4 x 32 KiB for the merge; the queries first)
constexpr float AT_RESCALE = 8.0f;
constexpr int AT_QPITCH = 1040;                // bytes per head row of the fp16 queries
constexpr int AT_MAX_CHUNK = 2048;             // positions of one split (k <= CSA2_MAX_K)

__device__ __forceinline__ f16x8_t dequant_latent8(uint32_t dw, uint32_t spair) {
  const f16x2_t sp = bitcast_u32<f16x2_t>(spair);
  f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 256.0f, 0) * sp;
  f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 256.0f, 1) * sp;
  f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 256.0f, 2) * sp;
  f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 256.0f, 3) * sp;
  return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// fp16 pair (s/256, s/256) for an E4M3FN scale byte (scales are non-negative)
__device__ __forceinline__ uint32_t scale_pair(uint32_t sbyte) {
  const uint32_t h = (sbyte & 0x7Fu) << 7;
  return h | (h << 16);
}

// max / sum over the four lanes l, l^16, l^32, l^48 (VALU lane swaps)
__device__ __forceinline__ float max_lane_groups(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float t = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float sum_lane_groups_a(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float t = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

__global__ __launch_bounds__(AT_THREADS) void attention_kernel(
    const uint8_t* __restrict__ kv, const int64_t* __restrict__ entry_offset,
    const int32_t* __restrict__ n_entries, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ q, int B, int H, float tau, int S,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // tile slots; the queries first
  __shared__ float4 pbuf[AT_WAVES][64];        // softmax weights of each slot, lane layout of the producer
  __shared__ float mref[AT_WAVES][16];         // producer reference maximum per head
  __shared__ float sm_lscale[16];
  __shared__ int32_t sidx[AT_MAX_CHUNK];       // the split's positions (-1 = skip)

  const int HG = (H + 15) / 16;
  const int wg = blockIdx.x;
  const int s = wg % S;
  const int hg = (wg / S) % HG;
  const int b = wg / (S * HG);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int head = 16 * hg + r;
  const bool head_ok = head < H;

  // --- entry range of this split, in tiles of 16
  const int chunk = ((k + S - 1) / S + 15) & ~15;
  const int e_lo = s * chunk;
  const int e_hi = min(k, e_lo + chunk);
  const int nent = max(e_hi - e_lo, 0);
  const int ntiles = (nent + 15) / 16;
  const int nrounds = (ntiles + AT_WAVES - 1) / AT_WAVES;
  const int64_t nb = n_entries[b];
  const int64_t row_base = entry_offset[b];
  const int32_t* ib = idx + (int64_t)b * k + e_lo;
  const bool any_rows = nb > 0;

  // --- early loads: this thread's query slice, and the first rows of this wave
  // (tile `wave`, position read straight from the index list)
  const int qh = tid >> 5, qc = tid & 31;
  const int hq = 16 * hg + qh;
  u32x4_t raw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (hq < H) {
    const uint16_t* src = q + ((int64_t)b * H + hq) * 512 + 16 * qc;
    raw[0] = *(const u32x4_t*)src;
    raw[1] = *(const u32x4_t*)(src + 8);
  }
  // A lane holds a quarter row (64 code bytes, 8 scale bytes) of one entry of
  // the wave's current tile; each part is reloaded with the next tile's row as
  // soon as it has been consumed. Skipped entries read row 0 of the sequence.
  u32x4_t cw[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  u32x2_t sw = {0, 0};
  if (any_rows && wave < ntiles) {
    const int e = 16 * wave + r;
    int p = e < nent ? ib[e] : -1;
    p = (p >= 0 && p < nb) ? p : 0;
    const uint8_t* row = kv + (row_base + p) * 288;
#pragma unroll
    for (int c = 0; c < 4; ++c) cw[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
    sw = *(const u32x2_t*)(row + 256 + 8 * kg);
  }
  for (int i = tid; i < nrounds * AT_WAVES * 16; i += AT_THREADS) {
    const int p = i < nent ? ib[i] : -1;
    sidx[i] = (p >= 0 && p < nb) ? p : -1;
  }

  // --- queries to fp16 in LDS. Each head is scaled by a power of two that puts
  // its largest magnitude in [2^14, 2^15) before rounding; the logit divides it
  // out again.
  uint8_t* qlds = smem;
  {
    uint32_t qmax = 0;                       // |bf16| bit patterns order like their values
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        qmax = max(qmax, raw[j][t] & 0x7FFFu);
        qmax = max(qmax, (raw[j][t] >> 16) & 0x7FFFu);
      }
    qmax = row_max_u32(qmax);                // 16 lanes, then the other half of the head's 32
    {
      const auto rr = __builtin_amdgcn_permlane16_swap(qmax, qmax, false, false);
      qmax = max((uint32_t)rr[0], (uint32_t)rr[1]);
    }
    const float qmaxf = bf16_to_f32(qmax);
    int sigma = 0;
    if (qmaxf > 0.0f) {
      int e;
      frexpf(qmaxf, &e);         // qmax in [2^(e-1), 2^e)
      sigma = 15 - e;            // qmax * 2^sigma in [2^14, 2^15)
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f16x8_t v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[2 * t] = (_Float16)ldexpf(bf16_to_f32(raw[j][t] & 0xFFFFu), sigma);
        v[2 * t + 1] = (_Float16)ldexpf(bf16_to_f32(raw[j][t] >> 16), sigma);
      }
      *(f16x8_t*)(qlds + qh * AT_QPITCH + 32 * qc + 16 * j) = v;
    }
    if (qc == 0) sm_lscale[qh] = ldexpf(tau, -sigma);
  }
  __syncthreads();
  // B operand of QK: column = head r, K-slice = dims 128kg + 8j .. +7
  f16x8_t qb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) qb[j] = *(const f16x8_t*)(qlds + r * AT_QPITCH + 256 * kg + 16 * j);
  const float lscale = sm_lscale[r];
  uint8_t* wlds = smem + wave * AT_WAVE_LDS;
  __syncthreads();                           // the queries' LDS becomes tile space

  // Producer state (this wave's tiles): reference maximum and partial sum for
  // head r. Consumer state (dims 64 wave .. 64 wave + 63 of every head): the
  // common reference M_c and O^T[dims][heads] in four 16-dim M-tiles.
  float m_w = -INFINITY, l_w = 0.0f, M_c = -INFINITY;
  f32x4_t O[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int last = ntiles - 1 - ((ntiles - 1 - wave) & (AT_WAVES - 1));   // this wave's last tile

  for (int rd = 0; any_rows && rd < nrounds; ++rd) {
    // ---- produce: tile t of this wave -> fp16 slot, logits, weights
    const int t = rd * AT_WAVES + wave;
    const bool t_ok = t < ntiles;
    const uint64_t vmask = t_ok ? __ballot(sidx[16 * t + r] >= 0) : 0ull;
    {
      const int next = t_ok ? min(t + AT_WAVES, last) : last;
      const int pn = last >= 0 ? sidx[16 * next + r] : -1;
      const uint8_t* rown = kv + (row_base + (pn >= 0 ? pn : 0)) * 288;
      f32x4_t lg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t sbyte = (sw[j >> 3] >> (8 * ((j >> 1) & 3))) & 0xFFu;
        const f16x8_t ca = dequant_latent8(cw[j >> 2][j & 3], scale_pair(sbyte));
        lg = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qb[j], lg, 0, 0, 0);
        *(f16x8_t*)(wlds + r * AT_PITCH + 256 * kg + 16 * j) = ca;
        if ((j & 3) == 3) cw[j >> 2] = *(const u32x4_t*)(rown + 64 * kg + 16 * (j >> 2));
      }
      sw = *(const u32x2_t*)(rown + 256 + 8 * kg);

      // this lane: entries 4kg + i of the tile, head r
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (vmask >> (4 * kg + i)) & 1ull;
        x[i] = v ? lg[i] * lscale : -INFINITY;
        tmax = fmaxf(tmax, x[i]);
      }
      tmax = max_lane_groups(tmax);
      // the reference rises only when a tile exceeds it by more than AT_RESCALE,
      // so the weights stay below e^AT_RESCALE
      if (tmax > m_w + AT_RESCALE || (m_w == -INFINITY && tmax > -INFINITY)) {
        const float m_new = fmaxf(m_w, tmax);
        l_w *= (m_w == -INFINITY) ? 0.0f : __expf(m_w - m_new);
        m_w = m_new;
      }
      float4 pv;
      pv.x = (m_w == -INFINITY) ? 0.0f : __expf(x[0] - m_w);
      pv.y = (m_w == -INFINITY) ? 0.0f : __expf(x[1] - m_w);
      pv.z = (m_w == -INFINITY) ? 0.0f : __expf(x[2] - m_w);
      pv.w = (m_w == -INFINITY) ? 0.0f : __expf(x[3] - m_w);
      l_w += (pv.x + pv.y) + (pv.z + pv.w);
      pbuf[wave][lane] = pv;
      if (kg == 0) mref[wave][r] = m_w;
    }
    __syncthreads();

    // ---- consume: O^T[64 dims of this wave] += C^T P^T over the round's 8 slots
    {
      float mw[AT_WAVES];
      float mr = M_c;
#pragma unroll
      for (int w = 0; w < AT_WAVES; ++w) { mw[w] = mref[w][r]; mr = fmaxf(mr, mw[w]); }
      if (mr > M_c) {
        const float alpha = (M_c == -INFINITY) ? 0.0f : __expf(M_c - mr);
#pragma unroll
        for (int u = 0; u < 4; ++u) O[u] *= alpha;
        M_c = mr;
      }
      typedef short i16x4_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
      const int j = lane & 15;
      // lane 4m + a of lane group kg points at entry 4kg + m, dims 16u + 4a .. +3;
      // after the transposing read, lane i of the group holds dim 16u + i of entries 4kg .. 4kg+3
      const int toff = (4 * kg + (j >> 2)) * AT_PITCH + 8 * (j & 3) + 32 * (4 * wave);
#pragma unroll
      for (int pr = 0; pr < AT_WAVES / 2; ++pr) {
        const int w0 = 2 * pr, w1 = 2 * pr + 1;
        const float f0 = (mw[w0] == -INFINITY) ? 0.0f : __expf(mw[w0] - M_c);
        const float f1 = (mw[w1] == -INFINITY) ? 0.0f : __expf(mw[w1] - M_c);
        const float4 p0 = pbuf[w0][lane], p1 = pbuf[w1][lane];
        // K-slots 8kg .. 8kg+3: slot w0 entries 4kg .. 4kg+3; 8kg+4 .. 8kg+7: slot w1
        const f16x8_t pb = {(_Float16)(p0.x * f0), (_Float16)(p0.y * f0), (_Float16)(p0.z * f0),
                            (_Float16)(p0.w * f0), (_Float16)(p1.x * f1), (_Float16)(p1.y * f1),
                            (_Float16)(p1.z * f1), (_Float16)(p1.w * f1)};
        __attribute__((address_space(3))) uint8_t* t0 =
            (__attribute__((address_space(3))) uint8_t*)smem + w0 * AT_WAVE_LDS + toff;
        __attribute__((address_space(3))) uint8_t* t1 =
            (__attribute__((address_space(3))) uint8_t*)smem + w1 * AT_WAVE_LDS + toff;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t0 + 32 * u));
          const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t1 + 32 * u));
          f16x8_t a;
          __builtin_memcpy(&a, &a0, 8);
          __builtin_memcpy((uint8_t*)&a + 8, &a1, 8);
          O[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, O[u], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // --- the sum of the weights: per wave (its own reference), then over waves
  float* lsum = (float*)pbuf;                // [AT_WAVES][16], after the last barrier
  float* mfin = lsum + AT_WAVES * 16;
  l_w = sum_lane_groups_a(l_w);
  if (lane < 16) { lsum[wave * 16 + lane] = l_w; mfin[wave * 16 + lane] = m_w; }
  __syncthreads();
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) {
    const float mw = mfin[w * 16 + r];
    if (mw != -INFINITY) L += lsum[w * 16 + r] * __expf(mw - M_c);
  }
  if (!head_ok) return;

  // lane (r, kg) holds dims 64 wave + 16u + 4kg + i of head r in O[u][i]
  if (S == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float* ob = out + ((int64_t)b * H + head) * 512 + 64 * wave + 4 * kg;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4_t x = O[u];
      *(float4*)(ob + 16 * u) = float4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    }
    if (lse && wave == 0 && kg == 0) lse[(int64_t)b * H + head] = L > 0.0f ? M_c + logf(L) : -INFINITY;
  } else {
    // partial: [B][H][S][512 + 2] -> unnormalised O, then (M, L)
    float* pb = part + (((int64_t)b * H + head) * S + s) * 514;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4_t x = O[u];
      float* o = pb + 64 * wave + 16 * u + 4 * kg;
      o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
    }
    if (wave == 0 && kg == 0) { pb[512] = M_c; pb[513] = L; }
  }
}

// out[b][h] = sum_s e^(M_s - M) O_s / sum_s e^(M_s - M) L_s
__global__ __launch_bounds__(128) void attention_combine_kernel(const float* __restrict__ part, int S,
                                                                float* __restrict__ out, float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const float* p = part + bh * S * 514;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p[s * 514 + 512]);
  float L = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float ms = p[s * 514 + 512];
    if (ms != -INFINITY) L += __expf(ms - M) * p[s * 514 + 513];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  for (int d = threadIdx.x; d < 512; d += 128) {
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float ms = p[s * 514 + 512];
      if (ms != -INFINITY) acc += __expf(ms - M) * p[s * 514 + d];
    }
    out[bh * 512 + d] = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[bh] = L > 0.0f ? M + logf(L) : -INFINITY;
}

int attention_splits(int B, int H, int k) {
  const int base = B * ((H + 15) / 16);
  int S = 1;
  // at least 128 workgroups (one per compute unit pair), each split keeping at
  // least one 16-entry tile per wave
  while (base * S < 128 && (k + 2 * S - 1) / (2 * S) >= 16 * AT_WAVES) S *= 2;
  return S;
}

size_t attention_lds_bytes() { return AT_LDS; }

hipError_t launch_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                            const int32_t* idx, int k, const uint16_t* q, int B, int H, float tau,
                            int S, float* out, float* lse, float* part, hipStream_t stream) {
  // the dynamic LDS limit is raised once per device (per-device flags: the
  // attribute belongs to the current device)
  static std::atomic<uint32_t> attr_set[64];
  int dev = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return e0;
  if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)attention_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, AT_LDS);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev].store(1u, std::memory_order_release);
  }
  dim3 grid((unsigned)(B * ((H + 15) / 16) * S)), block(AT_THREADS);
  hipLaunchKernelGGL(attention_kernel, grid, block, AT_LDS, stream, kv, entry_offset, n_entries, idx,
                     k, q, B, H, tau, S, out, lse, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)(B * H)), dim3(128), 0, stream, part, S,
                     out, lse);
  return hipGetLastError();
}

}  // namespace csa2
