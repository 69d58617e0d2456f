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
//   tile (pitch 1040 B: conflict-free reads) and repacked with v_perm.
// The 4 waves' partial states are merged through LDS; with several splits the
// workgroup writes an unnormalised partial that a small kernel combines.
#include "device.h"
#include "kernels.h"
#include <math.h>

namespace csa2 {

constexpr int AT_THREADS = 256;
constexpr int AT_PITCH = 1040;                 // bytes per entry row of the fp16 tile
constexpr int AT_WAVE_LDS = 16 * AT_PITCH;     // 16640
constexpr int AT_LDS = 4 * AT_WAVE_LDS;        // 66560 (>= 2 x 32 KiB for the merge)
constexpr float AT_RESCALE = 8.0f;

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

__global__ __launch_bounds__(AT_THREADS) void attention_kernel(
    const uint8_t* __restrict__ kv, const int64_t* __restrict__ entry_offset,
    const int32_t* __restrict__ n_entries, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ q, int B, int H, float tau, int S,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float sm_m[4][16], sm_l[4][16];

  const int HG = (H + 15) / 16;
  const int wg = blockIdx.x;
  const int s = wg % S;
  const int hg = (wg / S) % HG;
  const int b = wg / (S * HG);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int head = 16 * hg + r;
  const bool head_ok = head < H;

  // --- queries: B operand of QK (column = head r, K-slice = dims 128kg + 8j .. +7)
  const uint16_t* qh = q + ((int64_t)b * H + (head_ok ? head : 0)) * 512 + 128 * kg;
  u32x4_t qraw[16];
  float qmax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    qraw[j] = head_ok ? *(const u32x4_t*)(qh + 8 * j) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qmax = fmaxf(qmax, fabsf(bf16_to_f32(qraw[j][t] & 0xFFFFu)));
      qmax = fmaxf(qmax, fabsf(bf16_to_f32(qraw[j][t] >> 16)));
    }
  }
  qmax = fmaxf(qmax, shfl_xor_f(qmax, 16));
  qmax = fmaxf(qmax, shfl_xor_f(qmax, 32));
  int sigma = 0;
  if (qmax > 0.0f) {
    int e;
    frexpf(qmax, &e);          // qmax in [2^(e-1), 2^e)
    sigma = 15 - e;            // qmax * 2^sigma in [2^14, 2^15)
  }
  f16x8_t qb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qb[j][2 * t] = (_Float16)ldexpf(bf16_to_f32(qraw[j][t] & 0xFFFFu), sigma);
      qb[j][2 * t + 1] = (_Float16)ldexpf(bf16_to_f32(qraw[j][t] >> 16), sigma);
    }
  }
  const float lscale = ldexpf(tau, -sigma);

  // --- entry range of this split, in tiles of 16
  const int chunk = ((k + S - 1) / S + 15) & ~15;
  const int e_lo = s * chunk;
  const int e_hi = min(k, e_lo + chunk);
  const int ntiles = e_hi > e_lo ? (e_hi - e_lo + 15) / 16 : 0;
  const int64_t nb = n_entries[b];
  const int64_t row_base = entry_offset[b];
  const int32_t* ib = idx + (int64_t)b * k;
  uint8_t* wlds = smem + wave * AT_WAVE_LDS;
  f32x4_t O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY, l_run = 0.0f;

  // Tiles of this wave: wave, wave + 4, ... Software pipeline: the index of the
  // tile two steps ahead and the rows of the next tile are in flight while the
  // current tile is computed. Loads are unconditional (an invalid entry reads
  // row 0 of the sequence and is masked), so they never wait on a branch.
  const bool any_rows = nb > 0;
  auto idx_of = [&](int tile) -> int {
    const int ent = e_lo + 16 * tile + r;
    return (tile < ntiles && ent < e_hi) ? ib[ent] : -1;
  };
  auto rowp = [&](int p) -> const uint8_t* {
    const int64_t pc = (p >= 0 && p < nb) ? p : 0;
    return kv + (row_base + pc) * 288;
  };
  int pA = idx_of(wave), pB = idx_of(wave + 4);
  u32x4_t cw[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  u32x2_t sw = {0, 0};
  if (any_rows && wave < ntiles) {
    const uint8_t* row = rowp(pA);
#pragma unroll
    for (int c = 0; c < 4; ++c) cw[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
    sw = *(const u32x2_t*)(row + 256 + 8 * kg);
  }

  for (int tile = wave; tile < ntiles; tile += 4) {
    const int pC = idx_of(tile + 8);
    u32x4_t cwn[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    u32x2_t swn = {0, 0};
    if (any_rows && tile + 4 < ntiles) {
      const uint8_t* row = rowp(pB);
#pragma unroll
      for (int c = 0; c < 4; ++c) cwn[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
      swn = *(const u32x2_t*)(row + 256 + 8 * kg);
    }
    const bool valid = pA >= 0 && pA < nb;
    const uint64_t vmask = __ballot(valid);

    // dequantize 128 dims (128kg .. 128kg+127) to fp16, feed QK and copy the tile
    // to the wave's LDS area (row = entry r); logits^T: rows = entries, columns = heads
    f32x4_t lg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t sbyte = (sw[j >> 3] >> (8 * ((j >> 1) & 3))) & 0xFFu;
      const f16x8_t ca = dequant_latent8(cw[j >> 2][j & 3], scale_pair(sbyte));
      lg = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qb[j], lg, 0, 0, 0);
      *(f16x8_t*)(wlds + r * AT_PITCH + 256 * kg + 16 * j) = ca;
    }

    // online softmax for head r; this lane holds entries 4kg + i of the tile
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v = (vmask >> (4 * kg + i)) & 1ull;
      x[i] = v ? lg[i] * lscale : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
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
    // O^T[dims x heads] += C^T[dims x entries] P^T[entries x heads].
    // M-tile (u, v): lane row r <-> dim 32u + 2r + v; K = entries 4kg .. 4kg+3.
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      uint32_t d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = *(const uint32_t*)(wlds + (4 * kg + i) * AT_PITCH + 64 * u + 4 * r);
      const u32x2_t lo = {__builtin_amdgcn_perm(d[1], d[0], 0x05040100u), __builtin_amdgcn_perm(d[3], d[2], 0x05040100u)};
      const u32x2_t hi = {__builtin_amdgcn_perm(d[1], d[0], 0x07060302u), __builtin_amdgcn_perm(d[3], d[2], 0x07060302u)};
      f16x4_t a0, a1;
      __builtin_memcpy(&a0, &lo, 8);
      __builtin_memcpy(&a1, &hi, 8);
      O[2 * u] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, pb, O[2 * u], 0, 0, 0);
      O[2 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, pb, O[2 * u + 1], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c) cw[c] = cwn[c];
    sw = swn;
    pA = pB;
    pB = pC;
  }

  // --- merge the 4 waves: per head max, weights, then pairwise sums of O in LDS
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (lane < 16) { sm_m[wave][lane] = m_ref; sm_l[wave][lane] = l_run; }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][r]);
  float L = 0.0f, f_own = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = sm_m[w][r];
    const float f = (mw == -INFINITY) ? 0.0f : __expf(mw - M);
    L += f * sm_l[w][r];
    if (w == wave) f_own = f;
  }
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] *= f_own;

  f32x4_t* bufA = (f32x4_t*)smem;                  // [32][64] x 16 B = 32 KiB
  f32x4_t* bufB = (f32x4_t*)(smem + 32768);
  if (wave == 1 || wave == 3) {
    f32x4_t* buf = wave == 1 ? bufA : bufB;
#pragma unroll
    for (int t = 0; t < 32; ++t) buf[t * 64 + lane] = O[t];
  }
  __syncthreads();
  if (wave == 0 || wave == 2) {
    const f32x4_t* buf = wave == 0 ? bufA : bufB;
#pragma unroll
    for (int t = 0; t < 32; ++t) O[t] += buf[t * 64 + lane];
  }
  __syncthreads();
  if (wave == 2) {
#pragma unroll
    for (int t = 0; t < 32; ++t) bufA[t * 64 + lane] = O[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] += bufA[t * 64 + lane];
  if (!head_ok) return;

  // lane (r, kg) holds dims 32u + 8kg + 2i + v of head r in O[2u + v][i]
  if (S == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float* ob = out + ((int64_t)b * H + head) * 512;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const f32x4_t x0 = O[2 * u], x1 = O[2 * u + 1];
      float4 lo4 = {x0[0] * inv, x1[0] * inv, x0[1] * inv, x1[1] * inv};
      float4 hi4 = {x0[2] * inv, x1[2] * inv, x0[3] * inv, x1[3] * inv};
      *(float4*)(ob + 32 * u + 8 * kg) = lo4;
      *(float4*)(ob + 32 * u + 8 * kg + 4) = hi4;
    }
    if (lse && kg == 0) lse[(int64_t)b * H + head] = L > 0.0f ? M + logf(L) : -INFINITY;
  } else {
    // partial: [B][H][S][512 + 2] -> unnormalised O, then (M, L)
    float* pb = part + (((int64_t)b * H + head) * S + s) * 514;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const f32x4_t x0 = O[2 * u], x1 = O[2 * u + 1];
      float* o = pb + 32 * u + 8 * kg;
      o[0] = x0[0]; o[1] = x1[0]; o[2] = x0[1]; o[3] = x1[1];
      o[4] = x0[2]; o[5] = x1[2]; o[6] = x0[3]; o[7] = x1[3];
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
  // enough workgroups to cover the 256 compute units, at least 4 tiles per split
  while (base * S < 256 && (k + 2 * S - 1) / (2 * S) >= 64) S *= 2;
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
