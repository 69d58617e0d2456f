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
// Workgroup = (sequence, group of 16 heads; a last group with fewer heads runs
// with zero queries in the missing columns), 8 waves. The workgroups of one
// sequence are numbered so that they land on one XCD and share its L2 for the
// gathered rows. Every wave gathers the rows of its tiles (16 entries each,
// tiles w, w + 8, ...) as soon as the positions are known: with k = 512 all 32
// tiles of the list are requested at once (four tiles of quarter rows per
// lane), so the gather costs one memory round trip instead of one per tile
// group. Then rounds of 8 tiles, one per wave:
//   produce: a lane holds a quarter row (64 code bytes, 8 scale bytes) of one
//   entry and dequantizes it to fp16: the gfx950 scaled FP4->fp16 conversion
//   (which applies a power of two exactly) gives 256 * E2M1, and one packed
//   fp16 multiply by the E4M3 scale / 256 (the E4M3 bit pattern shifted into
//   fp16 position) gives the exact latent value (an E2M1 x E4M3 product has
//   at most 6 significant bits and lies in [2^-10, 2688], so fp16 holds it
//   exactly). QK^T is v_mfma_f32_16x16x32_f16 with the dequantized tile as the
//   A operand straight from registers and the queries as B. The tile goes to
//   the wave's LDS slot, its softmax weights to a small LDS buffer.
//   Queries are bf16; each head is multiplied by a power of two that puts its
//   largest magnitude in [2^14, 2^15) before rounding to fp16, so only values
//   below 2^-16 of the head's maximum can lose bits; the power is divided out
//   of the logit. Softmax: online, in fp32, with each wave's reference
//   maximum raised only when a tile's maximum exceeds it by more than 11.5
//   in log2 units (logits carry the factor log2(e); P = 2^(x - m) <= 2^11.5
//   fits fp16 and rescaling is rare).
//   consume: wave w owns output dimensions 64w .. 64w+63 and adds the round's
//   8 tiles: O^T += C^T P^T with v_mfma_f32_16x16x32_f16 (two slots = one K
//   step of 32 entries); C^T comes from gfx950's transposing LDS read
//   (ds_read_b64_tr_b16), which hands every lane 4 entries of one dimension;
//   rows are 1056 B apart so the 16 rows of a read fall on distinct banks.
//   P^T is rescaled from each tile's reference to the common one.
// Two barriers per round. A list is padded to whole rounds with skipped
// entries (weight 0, reading row 0 of the sequence), so every slot a round
// reads holds finite values.
#include "device.h"
#include "kernels.h"
#include "select_dev.h"
#include <math.h>
#include <atomic>

namespace csa2 {

constexpr int AT_WAVES = 8;
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_PITCH = 1056;                 // bytes per entry row of the fp16 tile (rows 8 banks apart)
constexpr int AT_SLOT = 16 * AT_PITCH;         // 16896: one tile of 16 entries
constexpr int AT_LDS = AT_WAVES * AT_SLOT;     // 135168: one slot per wave (the queries and the finish first)
constexpr float AT_RESCALE = 11.5f;           // log2 units: weights stay below 2^11.5 (fp16)
constexpr int AT_QPITCH = 1040;                // bytes per head row of the fp16 queries
constexpr int AT_MAX_K = 2048;                 // positions of a list (k <= CSA2_MAX_K)
constexpr int AT_NPF = 4;                      // tiles of rows a wave has in flight
constexpr int AT_DIMS = 512 / AT_WAVES;        // 64 output dimensions per wave

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
// list, all free until the rounds start) and the first workgroup of the
// sequence writes the result to ff.topk; idx is then not read.
template <bool FIN>
__global__ __launch_bounds__(AT_THREADS) void attention_kernel(
    const uint8_t* __restrict__ kv, const int64_t* __restrict__ entry_offset,
    const int32_t* __restrict__ n_entries, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ q, int B, int H, float tau,
    float* __restrict__ out, float* __restrict__ lse, FusedFinish ff) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // tile slots; the queries first
  __shared__ float4 pbuf[AT_WAVES][64];        // softmax weights of each slot, lane layout of the producer
  __shared__ float mref[AT_WAVES][16];         // producer reference maximum per head
  __shared__ float sm_lscale[16];
  __shared__ int32_t sidx[AT_MAX_K];           // the list's positions (-1 = skip), padded to whole rounds

  const int HG = (H + 15) / 16;
  const int G = B * HG;
  const int wg = blockIdx.x;
  if (FIN && wg >= G) {
    // one of the launch's last B * P workgroups: part wg - G mod P of the pool
    // finish of sequence (wg - G) / P; part 0 has the sequence's scratch rows
    uint8_t* pb8 = (uint8_t*)&pbuf[0][0];
    const FinLds fl{(uint64_t*)smem, (uint64_t*)(smem + 8 * FIN_LDS_CANDS), (uint32_t*)sidx,
                    (uint32_t*)(pb8 + 512), (uint64_t*)pb8, (uint32_t*)(pb8 + 256), (uint32_t*)(pb8 + 384),
                    (uint64_t*)(pb8 + 2560), (uint32_t*)(pb8 + 416)};
    const int P = ff.px.parts;
    const int bp = (wg - G) / P, part = (wg - G) % P;
    float* sall = part == 0 ? ff.scores + (int64_t)(G + bp) * ff.scores_stride : nullptr;
    uint64_t* gs = part == 0 ? ff.gscr + (int64_t)(G + bp) * ff.gscr_stride : nullptr;
    int32_t* po = ff.pool + (int64_t)bp * ff.pool_k;
    auto emit = [&](int j, int32_t v) { po[j] = v; };
    if (pool_finish_body<AT_THREADS>(bp, n_entries, ff.max_n, ff.pool_k, ff.sb, sall, gs, ff.src, fl, emit, &ff.px,
                                     part)) {
      __syncthreads();
      // a wait ran out of time: the whole finish, unsplit
      pool_finish_body<AT_THREADS>(bp, n_entries, ff.max_n, ff.pool_k, ff.sb, sall, gs, ff.src, fl, emit);
    }
    return;
  }
  // dispatch deals workgroups to the 8 XCDs in turn; number them so that the
  // workgroups of one sequence share an XCD (and its L2)
  const int lin = (G & 7) == 0 ? (wg & 7) * (G >> 3) + (wg >> 3) : wg;
  const int hg = lin % HG;
  const int b = lin / HG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int head = 16 * hg + r;
  const bool head_ok = head < H;

  const int ntiles = (k + 15) / 16;
  const int64_t nb = n_entries[b];
  const int64_t row_base = entry_offset[b];
  const int32_t* ib = idx + (int64_t)b * k;
  const bool any_rows = nb > 0 && ntiles > 0;
  const int R = any_rows ? (ntiles + AT_WAVES - 1) / AT_WAVES : 0;   // rounds (uniform)
  const int npad = 16 * AT_WAVES * R;                                // padded list length

  // --- early loads: this thread's query slice, and the index list
  const int qh = tid >> 5, qc = tid & 31;
  const int hq = 16 * hg + qh;
  u32x4_t raw[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (hq < H) {
    const uint16_t* src = q + ((int64_t)b * H + hq) * 512 + 16 * qc;
    raw[0] = *(const u32x4_t*)src;
    raw[1] = *(const u32x4_t*)(src + 8);
  }
  constexpr int NIV = AT_MAX_K / AT_THREADS;
  int32_t iv[NIV];
  // the finish's first loads (headers, list entries) go out with the queries'
  FinPrefetch<AT_THREADS> pf;
  if (FIN) {
    finish_prefetch<AT_THREADS>(pf, b, ff.max_n, ff.sb, ff.src);
  } else {
#pragma unroll
    for (int c = 0; c < NIV; ++c) {
      const int i = tid + c * AT_THREADS;
      iv[c] = i < k ? ib[i] : -1;
    }
  }

  // --- queries to fp16 in LDS (the first 16 KiB of the slot area, which the
  // finish's register path leaves alone). Each head is scaled by a power of
  // two that puts its largest magnitude in [2^14, 2^15) before rounding; the
  // logit divides it out again.
  uint8_t* qlds = smem;
  auto stage_queries = [&]() {
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
  };

  if (FIN) {
    // the queries while the finish's loads are in flight, then the finish
    static_assert(AT_MAX_K >= FIN_MAX_WG && AT_LDS >= 8 * (FIN_LDS_CANDS + FIN_SUB_CAP) &&
                  sizeof(pbuf) >= 4608 && 16 * AT_QPITCH <= 8 * FIN_LDS_CANDS,
                  "the finish's LDS fits the attention's; the queries lie in its list area only");
    stage_queries();
    uint8_t* pb8 = (uint8_t*)&pbuf[0][0];
    const FinLds fl{(uint64_t*)smem, (uint64_t*)(smem + 8 * FIN_LDS_CANDS), (uint32_t*)sidx,
                    (uint32_t*)(pb8 + 512), (uint64_t*)pb8, (uint32_t*)(pb8 + 256), (uint32_t*)(pb8 + 384),
                    (uint64_t*)(pb8 + 2560), (uint32_t*)(pb8 + 416)};
    // (the positions go to sidx only; the first workgroup of the sequence
    // copies them to ff.topk at the end: every position is below n_entries)
    const bool lists_in_lds =
        finish_direct_body<AT_THREADS>(b, n_entries, ff.max_n, ff.scores + (int64_t)lin * ff.scores_stride,
                                       ff.gscr + (int64_t)lin * ff.gscr_stride, ff.sb, k, ff.src, 1, fl, pf,
                                       [&](int j, int32_t v) { sidx[j] = (v >= 0 && v < nb) ? v : -1; });
    if (lists_in_lds) {                      // the list copy overwrote the queries
      __syncthreads();
      stage_queries();
    }
    for (int i = k + tid; i < npad; i += AT_THREADS) sidx[i] = -1;
    __syncthreads();
  }
  // a lane's row for list entry e (skipped entries read row 0 of the sequence);
  // before the list is in LDS (no finish) it is read from idx
  // (a call without rows reads the start of the query buffer, at least 1 KiB and
  // never used, so that every load is unconditional and the wait counts stay exact)
  const uint8_t* const rows = any_rows ? kv + row_base * 288 : (const uint8_t*)q;
  auto row_at = [&](int p) -> const uint8_t* {
    p = (p >= 0 && p < nb) ? p : 0;
    return rows + (int64_t)p * 288;
  };
  auto row_of = [&](int e) -> const uint8_t* { return row_at(sidx[e]); };
  auto load_quarter = [&](QuarterRow& qr, const uint8_t* row) {
#pragma unroll
    for (int c = 0; c < 4; ++c) qr.cw[c] = *(const u32x4_t*)(row + 64 * kg + 16 * c);
    qr.sw = *(const u32x2_t*)(row + 256 + 8 * kg);
  };
  // the rows of this wave's first AT_NPF tiles (tiles wave + 8 j), requested at
  // once: every position first, then every row (one round trip for all)
  QuarterRow buf[AT_NPF];
  int pe[AT_NPF];
#pragma unroll
  for (int j = 0; j < AT_NPF; ++j) {
    const int e = 16 * max(min(wave + AT_WAVES * j, AT_WAVES * R - 1), 0) + r;
    pe[j] = FIN ? sidx[e] : (e < k ? ib[e] : -1);
  }
  if (!FIN) {
    // (stored before the rows are requested: the stores wait for these loads only)
#pragma unroll
    for (int c = 0; c < NIV; ++c) sidx[tid + c * AT_THREADS] = (iv[c] >= 0 && iv[c] < nb) ? iv[c] : -1;
  }
#pragma unroll
  for (int j = 0; j < AT_NPF; ++j) load_quarter(buf[j], row_at(pe[j]));
  if (!FIN) {
    stage_queries();
    __syncthreads();
  }

  // B operand of QK (column = head r, K-slice = dims 128kg + 8j .. +7); the
  // slots are overwritten once every wave has read it
  f16x8_t qb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) qb[j] = *(const f16x8_t*)(qlds + r * AT_QPITCH + 256 * kg + 16 * j);
  const float lscale = sm_lscale[r] * 1.4426950408889634f;   // logits in log2 units
  __syncthreads();

  // per head r: this wave's producer reference and sum; the common reference
  // M_c and O^T[dims 64 wave ..][heads] in four 16-dim M-tiles
  float m_w = -INFINITY, l_w = 0.0f, M_c = -INFINITY;
  f32x4_t O[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- produce tile t of the list from qr into this wave's slot
  uint8_t* wlds = smem + wave * AT_SLOT;
  auto produce = [&](int t, const QuarterRow& qr) {
    const uint64_t vmask = __ballot(sidx[16 * t + r] >= 0);
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
    pbuf[wave][lane] = pv;
    if (kg == 0) mref[wave][r] = m_w;
  };

  // ---- consume the round's 8 slots: O^T[64 dims] += C^T P^T
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  // lane 4m + a of lane group kg points at entry 4kg + m, dims 16u + 4a .. +3;
  // after the transposing read, lane i of the group holds dim 16u + i of entries 4kg .. 4kg+3
  const int toff = (4 * kg + (r >> 2)) * AT_PITCH + 8 * (r & 3) + 2 * AT_DIMS * wave;
  auto consume = [&]() {
    float mw[AT_WAVES];
    float mr = M_c;
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) { mw[w] = mref[w][r]; mr = fmaxf(mr, mw[w]); }
    if (mr > M_c) {
      const float alpha = (M_c == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M_c - mr);
#pragma unroll
      for (int u = 0; u < 4; ++u) O[u] *= alpha;
      M_c = mr;
    }
    i16x4_t av[AT_WAVES][4];
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) {
      __attribute__((address_space(3))) uint8_t* tw =
          (__attribute__((address_space(3))) uint8_t*)smem + w * AT_SLOT + toff;
#pragma unroll
      for (int u = 0; u < 4; ++u) av[w][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tw + 32 * u));
    }
#pragma unroll
    for (int pr = 0; pr < AT_WAVES / 2; ++pr) {
      const int w0 = 2 * pr, w1 = 2 * pr + 1;
      const float f0 = (mw[w0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w0] - M_c);
      const float f1 = (mw[w1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w1] - M_c);
      const float4 p0 = pbuf[w0][lane], p1 = pbuf[w1][lane];
      // K-slots 8kg .. 8kg+3: slot w0 entries 4kg .. 4kg+3; 8kg+4 .. 8kg+7: slot w1
      const f16x8_t pb = {(_Float16)(p0.x * f0), (_Float16)(p0.y * f0), (_Float16)(p0.z * f0),
                          (_Float16)(p0.w * f0), (_Float16)(p1.x * f1), (_Float16)(p1.y * f1),
                          (_Float16)(p1.z * f1), (_Float16)(p1.w * f1)};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f16x8_t a;
        __builtin_memcpy(&a, &av[w0][u], 8);
        __builtin_memcpy((uint8_t*)&a + 8, &av[w1][u], 8);
        O[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, O[u], 0, 0, 0);
      }
    }
  };

  // Rounds: wave w produces tile 8 rd + w, then every wave consumes the
  // round's 8 tiles. In groups of AT_NPF rounds (so that each row buffer is a
  // fixed register set); a tile's buffer is reloaded with the tile AT_NPF
  // rounds ahead while more rounds follow, and the last group (rounds
  // without reloads) is peeled so that every load is unconditional and the
  // wait counts stay exact.
  int rd = 0;
  for (; rd + AT_NPF < R; rd += AT_NPF) {
#pragma unroll
    for (int j = 0; j < AT_NPF; ++j) {
      const int t = AT_WAVES * (rd + j) + wave;
      produce(t, buf[j]);
      __builtin_amdgcn_sched_barrier(0);
      load_quarter(buf[j], row_of(16 * min(t + AT_WAVES * AT_NPF, AT_WAVES * R - 1) + r));
      __syncthreads();
      consume();
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < AT_NPF; ++j) {
    if (rd + j < R) {
      produce(AT_WAVES * (rd + j) + wave, buf[j]);
      __syncthreads();
      consume();
      __syncthreads();
    }
  }

  // --- the sum of the weights: per producer (its own reference), then over producers
  float* lsum = (float*)pbuf;                // [AT_WAVES][16], after the last barrier
  float* mfin = lsum + AT_WAVES * 16;
  l_w = sum_lane_groups_a(l_w);
  if (lane < 16) { lsum[wave * 16 + lane] = l_w; mfin[wave * 16 + lane] = m_w; }
  if (FIN && hg == 0) {
    int32_t* tk = ff.topk + (int64_t)b * k;
    for (int j = tid; j < k; j += AT_THREADS) tk[j] = sidx[j];
  }
  __syncthreads();
  if (!head_ok) return;
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) {
    const float mw = mfin[w * 16 + r];
    if (mw != -INFINITY) L += lsum[w * 16 + r] * __builtin_amdgcn_exp2f(mw - M_c);
  }
  // lane (r, kg) holds dims 64 wave + 16u + 4kg + i of head r in O[u][i]
  const int d0 = AT_DIMS * wave + 4 * kg;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float* ob = out + ((int64_t)b * H + head) * 512 + d0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4_t x = O[u];
    *(float4*)(ob + 16 * u) = float4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
  }
  if (lse && wave == 0 && kg == 0)
    lse[(int64_t)b * H + head] = L > 0.0f ? (M_c + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

int attention_splits(int, int, int) { return 1; }

int attention_workgroups(int B, int H, int) { return B * ((H + 15) / 16); }

size_t attention_lds_bytes() { return AT_LDS; }

hipError_t launch_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                            const int32_t* idx, int k, const uint16_t* q, int B, int H, float tau,
                            int S, float* out, float* lse, float* part, const FusedFinish* fin,
                            hipStream_t stream) {
  (void)part;
  if (S != 1 || k > AT_MAX_K) return hipErrorInvalidValue;
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
  const int G = B * ((H + 15) / 16);
  if (fin && fin->pool_k > 0 && (fin->px.parts < 1 || fin->px.parts > kPoolMaxParts)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(G + (fin && fin->pool_k > 0 ? B * fin->px.parts : 0))), block(AT_THREADS);
  if (fin)
    hipLaunchKernelGGL(attention_kernel<true>, grid, block, AT_LDS, stream, kv, entry_offset, n_entries, idx,
                       k, q, B, H, tau, out, lse, *fin);
  else
    hipLaunchKernelGGL(attention_kernel<false>, grid, block, AT_LDS, stream, kv, entry_offset, n_entries, idx,
                       k, q, B, H, tau, out, lse, FusedFinish{});
  return hipGetLastError();
}

}  // namespace csa2
