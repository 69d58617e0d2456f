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
// group with fewer heads runs with zero queries in the missing columns). The
// workgroups of one sequence are numbered so that they land on one XCD and
// share its L2 for the gathered rows. Eight waves in two roles, which run at
// the same time on every SIMD (one of each per SIMD), so that the VALU-heavy
// dequantization overlaps the LDS- and MFMA-heavy PV product:
//   Producers (waves 0-3) take 16-entry tiles in turn. Per tile a lane holds a
//   quarter row (64 code bytes, 8 scale bytes) of one entry and dequantizes
//   it to fp16: the gfx950 scaled FP4->fp16 conversion (which applies a power
//   of two exactly) gives 256 * E2M1, and one packed fp16 multiply by the
//   E4M3 scale / 256 (the E4M3 bit pattern shifted into fp16 position) gives
//   the exact latent value (an E2M1 x E4M3 product has at most 6 significant
//   bits and lies in [2^-10, 2688], so fp16 holds it exactly). QK^T is
//   v_mfma_f32_16x16x32_f16 with the dequantized tile as the A operand
//   straight from registers and the queries as B. The tile goes to an LDS
//   slot and the softmax weights to a small LDS buffer. Rows are gathered two
//   tiles ahead.
//   Queries are bf16; each head is multiplied by a power of two that puts its
//   largest magnitude in [2^14, 2^15) before rounding to fp16, so only values
//   below 2^-16 of the head's maximum can lose bits; the power is divided out
//   of the logit. Softmax: online, in fp32, with each producer's reference
//   maximum raised only when a tile's maximum exceeds it by more than 11.5
//   in log2 units (logits carry the factor log2(e); P = 2^(x - m) <= 2^11.5
//   fits fp16 and rescaling is rare).
//   Consumers (waves 4-7) own 128 dimensions each: O^T += C^T P^T with
//   v_mfma_f32_16x16x32_f16 over the slots of the previous round (two slots =
//   one K step of 32 entries); C^T comes from gfx950's transposing LDS read
//   (ds_read_b64_tr_b16), which hands every lane 4 entries of one dimension;
//   rows are 1056 B apart so the 16 rows of a read fall on distinct banks.
//   P^T is rescaled from the producer's reference to the consumers' common
//   one.
// Two sets of four slots alternate: in round r the producers fill set r & 1
// while the consumers drain set (r - 1) & 1; one barrier ends each round. With
// several splits the workgroup writes an unnormalised partial that a small
// kernel combines.
#include "device.h"
#include "kernels.h"
#include "select_dev.h"
#include <math.h>
#include <atomic>

namespace csa2 {

constexpr int AT_PROD = 4;                     // producer waves, then as many consumers
constexpr int AT_WAVES = 2 * AT_PROD;          // one producer and one consumer per SIMD
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_PITCH = 1056;                 // bytes per entry row of the fp16 tile (rows 8 banks apart)
constexpr int AT_SLOT = 16 * AT_PITCH;         // 16896: one tile of 16 entries
constexpr int AT_LDS = 2 * AT_PROD * AT_SLOT;  // 135168: two sets of AT_PROD slots (the queries in set 1 first)
constexpr float AT_RESCALE = 11.5f;           // log2 units: weights stay below 2^11.5 (fp16)
constexpr int AT_QPITCH = 1040;                // bytes per head row of the fp16 queries
constexpr int AT_MAX_CHUNK = 2048;             // positions of one split (k <= CSA2_MAX_K)
constexpr int AT_DIMS_PER_CONS = 512 / AT_PROD;  // 128 output dimensions per consumer

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

// One entry's quarter row as a lane holds it: 64 code bytes and 8 scale bytes.
struct QuarterRow {
  u32x4_t cw[4];
  u32x2_t sw;
};

// FIN: the workgroup first runs the direct top-k finish of its sequence (the
// finish's LDS is carved from the tile slots, the weight buffer and the index
// list, all free until the rounds start) and takes its split of the result;
// idx is then not read.
template <bool FIN>
__global__ __launch_bounds__(AT_THREADS) void attention_kernel(
    const uint8_t* __restrict__ kv, const int64_t* __restrict__ entry_offset,
    const int32_t* __restrict__ n_entries, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ q, int B, int H, float tau, int S,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part, FusedFinish ff) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // tile slots; the queries in set 1 first
  __shared__ float4 pbuf[2][AT_PROD][64];      // softmax weights of each slot, lane layout of the producer
  __shared__ float mref[2][AT_PROD][16];       // producer reference maximum per head
  __shared__ float sm_lscale[16];
  __shared__ int32_t sidx[AT_MAX_CHUNK];       // the split's positions (-1 = skip)

  const int HG = (H + 15) / 16;
  const int G = B * HG * S;
  // dispatch deals workgroups to the 8 XCDs in turn; number them so that the
  // workgroups of one sequence share an XCD (and its L2)
  const int wg = blockIdx.x;
  const int lin = (G & 7) == 0 ? (wg & 7) * (G >> 3) + (wg >> 3) : wg;
  const int s = lin % S;
  const int hg = (lin / S) % HG;
  const int b = lin / (S * HG);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int head = 16 * hg + r;
  const bool head_ok = head < H;
  const bool producer = wave < AT_PROD;
  const int pw = producer ? wave : wave - AT_PROD;   // index within the role

  // --- entry range of this split, in tiles of 16; producer pw takes tiles
  // pw, pw + AT_PROD, ...
  const int chunk = ((k + S - 1) / S + 15) & ~15;
  const int e_lo = s * chunk;
  const int e_hi = min(k, e_lo + chunk);
  const int nent = max(e_hi - e_lo, 0);
  const int ntiles = (nent + 15) / 16;
  const int64_t nb = n_entries[b];
  const int64_t row_base = entry_offset[b];
  const int32_t* ib = idx + (int64_t)b * k + e_lo;
  const bool any_rows = nb > 0 && ntiles > 0;
  const int nrp = (ntiles + AT_PROD - 1) / AT_PROD;   // rounds with a tile to produce
  const int R = any_rows ? nrp + 1 : 0;              // plus one round to drain

  // --- early loads: this thread's query slice, its share of the index list,
  // and (producers) the rows of their first two tiles
  const int qh = tid >> 5, qc = tid & 31;
  const int hq = 16 * hg + qh;
  u32x4_t raw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (hq < H) {
    const uint16_t* src = q + ((int64_t)b * H + hq) * 512 + 16 * qc;
    raw[0] = *(const u32x4_t*)src;
    raw[1] = *(const u32x4_t*)(src + 8);
  }
  int32_t iv[AT_MAX_CHUNK / AT_THREADS];
  if (FIN) {
    // the finish, while the queries are in flight: positions of this split go
    // to sidx, the first workgroup of the sequence writes all k of them
    static_assert(AT_MAX_CHUNK >= FIN_MAX_WG && AT_LDS >= 8 * (FIN_LDS_CANDS + FIN_SUB_CAP) &&
                  sizeof(pbuf) >= 4608, "the finish's LDS fits the attention's");
    uint8_t* pb8 = (uint8_t*)&pbuf[0][0][0];
    const FinLds fl{(uint64_t*)smem, (uint64_t*)(smem + 8 * FIN_LDS_CANDS), (uint32_t*)sidx,
                    (uint32_t*)(pb8 + 512), (uint64_t*)pb8, (uint32_t*)(pb8 + 256), (uint32_t*)(pb8 + 384),
                    (uint64_t*)(pb8 + 2560), (uint32_t*)(pb8 + 416)};
    const bool writer = hg == 0 && s == 0;
    int32_t* tk = ff.topk + (int64_t)b * k;
    finish_direct_body<AT_THREADS>(b, n_entries, ff.max_n, ff.scores + (int64_t)lin * ff.scores_stride,
                                   ff.gscr + (int64_t)lin * ff.gscr_stride, ff.sb, k, ff.src, 1, fl,
                                   [&](int j, int32_t v) {
                                     if (writer) tk[j] = v;
                                     const int jj = j - e_lo;
                                     if (jj >= 0 && jj < nent) sidx[jj] = (v >= 0 && v < nb) ? v : -1;
                                   });
    for (int i = nent + tid; i < 16 * ntiles; i += AT_THREADS) sidx[i] = -1;
    __syncthreads();
  } else {
#pragma unroll
    for (int c = 0; c < AT_MAX_CHUNK / AT_THREADS; ++c) {
      const int i = tid + c * AT_THREADS;
      iv[c] = i < nent ? ib[i] : -1;
    }
  }
  // a producer lane's row of tile t (clamped to the last tile; skipped entries
  // read row 0 of the sequence)
  auto row_of = [&](int p) -> const uint8_t* {
    p = (p >= 0 && p < nb) ? p : 0;
    return kv + (row_base + p) * 288;
  };
  auto load_quarter = [&](QuarterRow& qr, const uint8_t* row) {
#pragma unroll
    for (int c = 0; c < 4; ++c) qr.cw[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
    qr.sw = *(const u32x2_t*)(row + 256 + 8 * kg);
  };
  QuarterRow bufA, bufB;
#pragma unroll
  for (int c = 0; c < 4; ++c) { bufA.cw[c] = u32x4_t{0, 0, 0, 0}; bufB.cw[c] = u32x4_t{0, 0, 0, 0}; }
  bufA.sw = u32x2_t{0, 0};
  bufB.sw = u32x2_t{0, 0};
  if (producer) {
    // unconditional, so that the wait counts in the round loop stay exact; a
    // split without rows reads the start of the query buffer (at least 1 KiB,
    // never used)
    const int t0 = max(min(pw, ntiles - 1), 0), t1 = max(min(pw + AT_PROD, ntiles - 1), 0);
    const int e0 = 16 * t0 + r, e1 = 16 * t1 + r;
    const int p0 = e0 < nent ? (FIN ? sidx[e0] : ib[e0]) : -1;
    const int p1 = e1 < nent ? (FIN ? sidx[e1] : ib[e1]) : -1;
    const uint8_t* const qrow = (const uint8_t*)q;
    load_quarter(bufA, any_rows ? row_of(p0) : qrow);
    load_quarter(bufB, any_rows ? row_of(p1) : qrow);
  }
  if (!FIN) {
#pragma unroll
    for (int c = 0; c < AT_MAX_CHUNK / AT_THREADS; ++c) {
      const int i = tid + c * AT_THREADS;
      if (i < 16 * ntiles) sidx[i] = (iv[c] >= 0 && iv[c] < nb) ? iv[c] : -1;
    }
  }

  // --- queries to fp16 in LDS (slot set 1, first written in round 1). Each
  // head is scaled by a power of two that puts its largest magnitude in
  // [2^14, 2^15) before rounding; the logit divides it out again.
  uint8_t* qlds = smem + AT_PROD * AT_SLOT;
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

  // Producer state: B operand of QK (column = head r, K-slice = dims
  // 128kg + 8j .. +7), reference maximum and partial sum for head r.
  // Consumer state: the common reference M_c and O^T[dims][heads] for dims
  // 128 pw .. 128 pw + 127 in eight 16-dim M-tiles.
  f16x8_t qb[16];
  float lscale = 0.0f;
  if (producer) {
#pragma unroll
    for (int j = 0; j < 16; ++j) qb[j] = *(const f16x8_t*)(qlds + r * AT_QPITCH + 256 * kg + 16 * j);
    lscale = sm_lscale[r] * 1.4426950408889634f;   // logits in log2 units
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) qb[j] = f16x8_t{};
  }
  float m_w = -INFINITY, l_w = 0.0f, M_c = -INFINITY;
  f32x4_t O[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- produce round j: tile pw + AT_PROD j from qr into slot set `set`;
  // qr is reloaded with the rows of the tile two rounds ahead
  auto produce = [&](int j, QuarterRow& qr, int set) {
    const int t = pw + AT_PROD * j;
    const bool t_ok = t < ntiles;
    const uint64_t vmask = t_ok ? __ballot(sidx[16 * t + r] >= 0) : 0ull;
    const int tn = min(t + 2 * AT_PROD, ntiles - 1);
    const uint8_t* rown = row_of(sidx[16 * tn + r]);
    uint8_t* wlds = smem + (set * AT_PROD + pw) * AT_SLOT;
    // two accumulators halve the dependent MFMA chain
    f32x4_t lg2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const uint32_t sbyte = (qr.sw[jj >> 3] >> (8 * ((jj >> 1) & 3))) & 0xFFu;
      const f16x8_t ca = dequant_latent8(qr.cw[jj >> 2][jj & 3], scale_pair(sbyte));
      lg2[jj & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qb[jj], lg2[jj & 1], 0, 0, 0);
      *(f16x8_t*)(wlds + r * AT_PITCH + 256 * kg + 16 * jj) = ca;
    }
    const f32x4_t lg = lg2[0] + lg2[1];
    // the reloads go after the buffer's last use, so that they land in the
    // same registers (no copies, hence no early waits, at the loop edge)
    __builtin_amdgcn_sched_barrier(0);
    load_quarter(qr, rown);

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
    // so the weights stay below 2^AT_RESCALE
    if (tmax > m_w + AT_RESCALE || (m_w == -INFINITY && tmax > -INFINITY)) {
      const float m_new = fmaxf(m_w, tmax);
      l_w *= (m_w == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_w - m_new);
      m_w = m_new;
    }
    float4 pv;
    pv.x = (m_w == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[0] - m_w);
    pv.y = (m_w == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[1] - m_w);
    pv.z = (m_w == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[2] - m_w);
    pv.w = (m_w == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[3] - m_w);
    l_w += (pv.x + pv.y) + (pv.z + pv.w);
    pbuf[set][pw][lane] = pv;
    if (kg == 0) mref[set][pw][r] = m_w;
  };

  // ---- consume the slot set `set`: O^T[128 dims] += C^T P^T over its 4 slots
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  // lane 4m + a of lane group kg points at entry 4kg + m, dims 16u + 4a .. +3;
  // after the transposing read, lane i of the group holds dim 16u + i of entries 4kg .. 4kg+3
  const int toff = (4 * kg + (r >> 2)) * AT_PITCH + 8 * (r & 3) + 2 * AT_DIMS_PER_CONS * pw;
  auto consume = [&](int set) {
    float mw[AT_PROD];
    float mr = M_c;
#pragma unroll
    for (int w = 0; w < AT_PROD; ++w) { mw[w] = mref[set][w][r]; mr = fmaxf(mr, mw[w]); }
    if (mr > M_c) {
      const float alpha = (M_c == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M_c - mr);
#pragma unroll
      for (int u = 0; u < 8; ++u) O[u] *= alpha;
      M_c = mr;
    }
    // all 32 transposing reads of the round are issued before the first MFMA
    i16x4_t av[AT_PROD][8];
#pragma unroll
    for (int w = 0; w < AT_PROD; ++w) {
      __attribute__((address_space(3))) uint8_t* tw =
          (__attribute__((address_space(3))) uint8_t*)smem + (set * AT_PROD + w) * AT_SLOT + toff;
#pragma unroll
      for (int u = 0; u < 8; ++u) av[w][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tw + 32 * u));
    }
#pragma unroll
    for (int pr = 0; pr < AT_PROD / 2; ++pr) {
      const int w0 = 2 * pr, w1 = 2 * pr + 1;
      const float f0 = (mw[w0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w0] - M_c);
      const float f1 = (mw[w1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w1] - M_c);
      const float4 p0 = pbuf[set][w0][lane], p1 = pbuf[set][w1][lane];
      // K-slots 8kg .. 8kg+3: slot w0 entries 4kg .. 4kg+3; 8kg+4 .. 8kg+7: slot w1
      const f16x8_t pb = {(_Float16)(p0.x * f0), (_Float16)(p0.y * f0), (_Float16)(p0.z * f0),
                          (_Float16)(p0.w * f0), (_Float16)(p1.x * f1), (_Float16)(p1.y * f1),
                          (_Float16)(p1.z * f1), (_Float16)(p1.w * f1)};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        f16x8_t a;
        __builtin_memcpy(&a, &av[w0][u], 8);
        __builtin_memcpy((uint8_t*)&a + 8, &av[w1][u], 8);
        O[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, O[u], 0, 0, 0);
      }
    }
  };

  // round rd: producers fill set rd & 1 (rounds >= nrp produce nothing
  // visible: no valid entry, weights 0), consumers drain set (rd - 1) & 1
  // (rounds >= 1). One barrier per round; each role runs its own loop, unrolled
  // by two so that the set and the row buffer of each half are fixed and every
  // load in the loop is unconditional.
  if (R > 0) {
    int rd = 0;
    if (producer) {
      for (; rd + 1 < R; rd += 2) {
        produce(rd, bufA, 0);
        __syncthreads();
        produce(rd + 1, bufB, 1);
        __syncthreads();
      }
      if (rd < R) {
        produce(rd, bufA, 0);
        __syncthreads();
      }
    } else {
      for (; rd + 1 < R; rd += 2) {
        if (rd > 0) consume(1);
        __syncthreads();
        consume(0);
        __syncthreads();
      }
      if (rd < R) {
        consume(1);                          // rd >= 2 here: R >= 2 whenever rows exist
        __syncthreads();
      }
    }
  }

  // --- the sum of the weights: per producer (its own reference), then over producers
  float* lsum = (float*)pbuf;                // [AT_PROD][16], after the last barrier
  float* mfin = lsum + AT_PROD * 16;
  if (producer) {
    l_w = sum_lane_groups_a(l_w);
    if (lane < 16) { lsum[pw * 16 + lane] = l_w; mfin[pw * 16 + lane] = m_w; }
  }
  __syncthreads();
  if (producer || !head_ok) return;
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < AT_PROD; ++w) {
    const float mw = mfin[w * 16 + r];
    if (mw != -INFINITY) L += lsum[w * 16 + r] * __builtin_amdgcn_exp2f(mw - M_c);
  }

  // lane (r, kg) holds dims 128 pw + 16u + 4kg + i of head r in O[u][i]
  const int d0 = AT_DIMS_PER_CONS * pw + 4 * kg;
  if (S == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float* ob = out + ((int64_t)b * H + head) * 512 + d0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4_t x = O[u];
      *(float4*)(ob + 16 * u) = float4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    }
    if (lse && pw == 0 && kg == 0)
      lse[(int64_t)b * H + head] = L > 0.0f ? (M_c + log2f(L)) * 0.6931471805599453f : -INFINITY;
  } else {
    // partial: [B][H][S][512 + 2] -> unnormalised O, then (M, L)
    float* pb = part + (((int64_t)b * H + head) * S + s) * 514;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4_t x = O[u];
      float* o = pb + d0 + 16 * u;
      o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
    }
    if (pw == 0 && kg == 0) { pb[512] = M_c * 0.6931471805599453f; pb[513] = L; }   // M in natural units
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

int attention_workgroups(int B, int H, int k) { return B * ((H + 15) / 16) * attention_splits(B, H, k); }

size_t attention_lds_bytes() { return AT_LDS; }

hipError_t launch_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                            const int32_t* idx, int k, const uint16_t* q, int B, int H, float tau,
                            int S, float* out, float* lse, float* part, const FusedFinish* fin,
                            hipStream_t stream) {
  // the dynamic LDS limit is raised once per device (per-device flags: the
  // attribute belongs to the current device)
  static std::atomic<uint32_t> attr_set[64];
  int dev = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return e0;
  if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)attention_kernel<false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, AT_LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)attention_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              AT_LDS);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev].store(1u, std::memory_order_release);
  }
  dim3 grid((unsigned)(B * ((H + 15) / 16) * S)), block(AT_THREADS);
  if (fin)
    hipLaunchKernelGGL(attention_kernel<true>, grid, block, AT_LDS, stream, kv, entry_offset, n_entries, idx,
                       k, q, B, H, tau, S, out, lse, part, *fin);
  else
    hipLaunchKernelGGL(attention_kernel<false>, grid, block, AT_LDS, stream, kv, entry_offset, n_entries, idx,
                       k, q, B, H, tau, S, out, lse, part, FusedFinish{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)(B * H)), dim3(128), 0, stream, part, S,
                     out, lse);
  return hipGetLastError();
}

}  // namespace csa2
