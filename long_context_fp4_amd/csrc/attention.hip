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

namespace csa2 {

constexpr int AT_WAVES = 8;                    // two waves per SIMD
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_PITCH = 1056;                 // bytes per entry row of the fp16 tile (rows 8 banks apart)
constexpr int AT_WAVE_LDS = 16 * AT_PITCH;     // 16896
constexpr int AT_LDS = AT_WAVES * AT_WAVE_LDS; // 135168 (>= 4 x 32 KiB for the merge; the queries first)
constexpr float AT_RESCALE = 8.0f;
constexpr int AT_QPITCH = 1040;                // bytes per head row of the fp16 queries
constexpr int AT_QLDS_K = 2;                   // query K-slices read from LDS at every tile
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
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float sm_m[AT_WAVES][16], sm_l[AT_WAVES][16];
  __shared__ float sm_lscale[16];
  __shared__ int32_t sidx[AT_MAX_CHUNK];                                   // the split's positions (-1 = skip)
  __shared__ f16x8_t qtail[AT_QLDS_K][64];                                 // last query slices, per lane
  uint8_t* qlds = smem;                    // fp16 queries (row = head) until the tiles start

  const int HG = (H + 15) / 16;
  const int wg = blockIdx.x;
  const int s = wg % S;
  const int hg = (wg / S) % HG;
  const int b = wg / (S * HG);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int head = 16 * hg + r;
  const bool head_ok = head < H;

  // --- entry range of this split, in tiles of 16; its positions go to LDS
  const int chunk = ((k + S - 1) / S + 15) & ~15;
  const int e_lo = s * chunk;
  const int e_hi = min(k, e_lo + chunk);
  const int nent = max(e_hi - e_lo, 0);
  const int ntiles = (nent + 15) / 16;
  const int64_t nb = n_entries[b];
  const int64_t row_base = entry_offset[b];
  // --- queries: thread (qh = tid/32, c = tid%32) takes dims 16c .. 16c+15 of head 16hg + qh;
  // their loads are issued before the split's positions are read
  const int qh = tid >> 5, qc = tid & 31;
  const int hq = 16 * hg + qh;
  u32x4_t raw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (hq < H) {
    const uint16_t* src = q + ((int64_t)b * H + hq) * 512 + 16 * qc;
    raw[0] = *(const u32x4_t*)src;
    raw[1] = *(const u32x4_t*)(src + 8);
  }
  // --- entry range of this split, in tiles of 16; its positions go to LDS
  {
    const int32_t* ib = idx + (int64_t)b * k + e_lo;
    for (int i = tid; i < ntiles * 16; i += AT_THREADS) {
      int p = i < nent ? ib[i] : -1;
      sidx[i] = (p >= 0 && p < nb) ? p : -1;
    }
  }
  // Each head is scaled by a power of two that puts its largest magnitude in
  // [2^14, 2^15) before rounding to fp16; the logit divides it out again.
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
      const auto r = __builtin_amdgcn_permlane16_swap(qmax, qmax, false, false);
      qmax = max((uint32_t)r[0], (uint32_t)r[1]);
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
  // (the last AT_QLDS_K slices stay in a small LDS copy, read per tile, to keep
  // the wave within 256 registers)
  f16x8_t qb[16 - AT_QLDS_K];
#pragma unroll
  for (int j = 0; j < 16 - AT_QLDS_K; ++j) qb[j] = *(const f16x8_t*)(qlds + r * AT_QPITCH + 256 * kg + 16 * j);
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < AT_QLDS_K; ++j)
      qtail[j][lane] = *(const f16x8_t*)(qlds + r * AT_QPITCH + 256 * kg + 16 * (16 - AT_QLDS_K + j));
  }
  const float lscale = sm_lscale[r];
  uint8_t* wlds = smem + wave * AT_WAVE_LDS;
  __syncthreads();                           // the queries' LDS becomes tile space

  f32x4_t O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY, l_run = 0.0f;

  // Tiles of this wave: wave, wave + 8, ... A lane holds a quarter row (64
  // code bytes, 8 scale bytes) of one entry; each 16-byte part is reloaded
  // with the next tile's row as soon as the current tile has consumed it, so
  // the next rows are in flight during the rest of the tile. Loads are
  // unconditional (a skipped entry reads row 0 of the sequence and is masked).
  const bool any_rows = nb > 0;
  u32x4_t cw[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  u32x2_t sw = {0, 0};
  if (any_rows && wave < ntiles) {
    const int p = sidx[16 * wave + r];
    const uint8_t* row = kv + (row_base + (p >= 0 ? p : 0)) * 288;
#pragma unroll
    for (int c = 0; c < 4; ++c) cw[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
    sw = *(const u32x2_t*)(row + 256 + 8 * kg);
  }
  auto compute_tile = [&](int tile, int next) {
      const uint64_t vmask = __ballot(sidx[16 * tile + r] >= 0);
      const int pn = sidx[16 * next + r];
      const uint8_t* rown = kv + (row_base + (pn >= 0 ? pn : 0)) * 288;

      // dequantize 128 dims (128kg .. 128kg+127) to fp16, feed QK and copy the tile
      // to the wave's LDS area (row = entry r); logits^T: rows = entries, columns = heads
      f32x4_t lg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t sbyte = (sw[j >> 3] >> (8 * ((j >> 1) & 3))) & 0xFFu;
        const f16x8_t ca = dequant_latent8(cw[j >> 2][j & 3], scale_pair(sbyte));
        const f16x8_t qj = j < 16 - AT_QLDS_K ? qb[j < 16 - AT_QLDS_K ? j : 0] : qtail[j - (16 - AT_QLDS_K)][lane];
        lg = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qj, lg, 0, 0, 0);
        *(f16x8_t*)(wlds + r * AT_PITCH + 256 * kg + 16 * j) = ca;
        if ((j & 3) == 3) cw[j >> 2] = *(const u32x4_t*)(rown + 64 * kg + 16 * (j >> 2));
      }
      sw = *(const u32x2_t*)(rown + 256 + 8 * kg);

      // online softmax for head r; this lane holds entries 4kg + i of the tile
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (vmask >> (4 * kg + i)) & 1ull;
        x[i] = v ? lg[i] * lscale : -INFINITY;
        tmax = fmaxf(tmax, x[i]);
      }
      tmax = max_lane_groups(tmax);
      const bool raise = tmax > m_ref + AT_RESCALE || (m_ref == -INFINITY && tmax > -INFINITY);
      if (__any(raise)) {
        const float m_new = raise ? fmaxf(m_ref, tmax) : m_ref;
        const float alpha = (m_ref == -INFINITY) ? 0.0f : __expf(m_ref - m_new);
        if (raise) {
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < 32; ++t) O[t] *= alpha;
          m_ref = m_new;
        }
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (m_ref == -INFINITY) ? 0.0f : expf(x[i] - m_ref);
        l_run += p[i];
      }
      const f16x4_t pb = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};

      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // O^T[dims x heads] += C^T[dims x entries] P^T[entries x heads], one M-tile per 16 dims.
      // A operand by transposing LDS reads: lane 4m + a of lane group kg points at entry
      // 4kg + m, dims 16u + 4a .. +3; lane i of the group then holds dim 16u + i of
      // entries 4kg .. 4kg+3.
      {
        typedef short i16x4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
        const int j = lane & 15;
        __attribute__((address_space(3))) uint8_t* tb =
            (__attribute__((address_space(3))) uint8_t*)wlds + (4 * kg + (j >> 2)) * AT_PITCH + 8 * (j & 3);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const i16x4_t raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + 32 * u));
          f16x4_t a;
          __builtin_memcpy(&a, &raw, 8);
          O[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pb, O[u], 0, 0, 0);
        }
      }
      __builtin_amdgcn_wave_barrier();
  };
  // rounds of up to 8 tiles per wave, unrolled so the load/compute pipeline is
  // straight-line code (the prefetch past the wave's last tile re-reads it)
  const int last = ntiles - 1 - ((ntiles - 1 - wave) & (AT_WAVES - 1));   // this wave's last tile
  for (int tile = wave; any_rows && tile < ntiles; tile += AT_WAVES) compute_tile(tile, min(tile + AT_WAVES, last));

  // --- merge the waves: per head max, weights, then pairwise sums of O in LDS
  l_run = sum_lane_groups_a(l_run);
  if (lane < 16) { sm_m[wave][lane] = m_ref; sm_l[wave][lane] = l_run; }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) M = fmaxf(M, sm_m[w][r]);
  float L = 0.0f, f_own = 0.0f;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) {
    const float mw = sm_m[w][r];
    const float f = (mw == -INFINITY) ? 0.0f : __expf(mw - M);
    L += f * sm_l[w][r];
    if (w == wave) f_own = f;
  }
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] *= f_own;

  // halving rounds: waves [h, 2h) store their O (32 KiB each), waves [0, h) add it
  f32x4_t* obuf = (f32x4_t*)smem;
#pragma unroll
  for (int half = AT_WAVES / 2; half >= 1; half >>= 1) {
    __syncthreads();
    if (wave >= half && wave < 2 * half) {
      f32x4_t* buf = obuf + (wave - half) * 32 * 64;
#pragma unroll
      for (int t = 0; t < 32; ++t) buf[t * 64 + lane] = O[t];
    }
    __syncthreads();
    if (wave < half) {
      const f32x4_t* buf = obuf + wave * 32 * 64;
#pragma unroll
      for (int t = 0; t < 32; ++t) O[t] += buf[t * 64 + lane];
    }
  }
  if (wave != 0) return;
  if (!head_ok) return;

  // lane (r, kg) holds dims 16u + 4kg + i of head r in O[u][i]
  if (S == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float* ob = out + ((int64_t)b * H + head) * 512;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const f32x4_t x = O[u];
      *(float4*)(ob + 16 * u + 4 * kg) = float4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    }
    if (lse && kg == 0) lse[(int64_t)b * H + head] = L > 0.0f ? M + logf(L) : -INFINITY;
  } else {
    // partial: [B][H][S][512 + 2] -> unnormalised O, then (M, L)
    float* pb = part + (((int64_t)b * H + head) * S + s) * 514;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const f32x4_t x = O[u];
      float* o = pb + 16 * u + 4 * kg;
      o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
    }
    if (kg == 0) { pb[512] = M; pb[513] = L; }
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
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attention_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, AT_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
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
