// Indexer scoring and exact top-k selection over the compressed cache, for gfx950.
//
// What is computed ("Le cache KV en FP4 — les 890 octets, vérifiés", section
// "Les ingrédients": the 128-channel indexer key scores positions; "DeepSeek
// V4.1 Flash : 890 octets de cache KV par token", section "L'architecture :
// trois leviers contre le cache": a Full layer picks new top-512 indices and a
// hierarchical indexer caps the candidates at 16384; "KV cache da 890 byte per
// token", section "Tre meccanismi al posto di un solo trucco": deeper layers
// rescore only that pool). Score S_i = sum_h w_h * max(0, q_h . k_i) (or the
// plain dot product for a single head); selection order is score descending,
// position ascending; selected positions are written in ascending order.
//
// Kernels
// -------
// score_kernel   streams the packed MXFP4 keys (one 16-byte load of codes and
//                one scale byte per lane, several tiles in flight), dequantizes
//                them in registers with the gfx950 scaled FP4->bf16 conversion
//                (exact: an E2M1 value times a power of two fits bf16), and
//                contracts 16 entries x 16 heads x 32 channels per
//                v_mfma_f32_16x16x32_bf16; the head sum is a 4-term in-lane sum
//                plus two VALU lane swaps. Scores are staged in LDS and written
//                with coalesced 16-byte stores. The quantized-query variant
//                (score-mode flag) first converts the queries to MXFP8 in LDS
//                and contracts each tile with one block-scaled FP8 x FP4 MFMA
//                that reads the keys as stored.
//                Selection without contended atomics: each workgroup finds a
//                local cutoff over its 1024 score keys that keeps a multiple of
//                its expected share of the top-k, and writes to its own slot the
//                (bin, count) pairs above that cutoff (pool) or, for k <= 512,
//                the candidates themselves with a header word.
// finish_*_kernel  one workgroup per sequence merges the slots: bins at or
//                above the highest cutoff are complete, so the bin holding the
//                k-th best key follows exactly whenever it lies there
//                (otherwise a full histogram of the sequence's scores is the
//                fallback). For k <= 512 the k best among the candidates are
//                written in ascending order (finish_direct_body, which a Full
//                decode layer runs inside its attention launch instead); larger
//                k (the hierarchical pool) go on to select_kernel.
// select_kernel  (large k) marks every position whose key lies above that bin
//                in a per-sequence bitmap and appends the ones inside it as
//                (key, position) candidates; the last workgroup of the sequence
//                radix-selects the missing ones among the candidates, then
//                compacts the bitmap into ascending positions.
// select_small_kernel  one workgroup per sequence for at most 16384 slots
//                (the pool, a Reindex candidate list or a short sequence):
//                keys in LDS, 8-bit radix select on (key, slot), bitmap
//                compaction in slot order.
// The per-sequence control block (counters, at a fixed place in the
// workspace) is left zero by the last workgroups; bitmap words are cleared by
// the score pass before use; every other workspace region is rewritten before
// it is read.
#include "device.h"
#include "kernels.h"
#include "select_dev.h"

namespace csa2 {

constexpr int SC_THREADS = 256;   // also the threads that stage a quantized query

constexpr int SC_SUB = 1;           // selection chunks per score workgroup
constexpr int SC_SPAN = SC_SUB * SC_CHUNK;   // slots a score workgroup streams
constexpr int SC_UNROLL = 4;        // tiles in flight per wave
constexpr int SUM_PAIRS = kSumWords;   // (bin, count) pairs a workgroup reports above its cutoff

constexpr int FIN_THREADS = 1024;  // finish workgroup of the direct top-k
constexpr int SEL_THREADS = 256;
constexpr int SEL_CHUNK = 4096;     // slots per select workgroup
constexpr int SEL_LDS_CAP = 4096;   // candidates staged in LDS by the last select workgroup
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_MAX = 16384;

// Ascending compaction of a bitmap of nbits bits into out[0..cnt), -1 padding up
// to K. The bitmap is read in chunks of `stage_words` words into the LDS buffer
// `stage` with independent coalesced loads; a global bitmap filled by other
// workgroups of the launch is read after the caller's acquire fence.
__device__ void compact_bitmap(const uint32_t* bm, int64_t nbits, const int32_t* slot_pos, int K,
                               int32_t* out, uint32_t* scan_tmp, uint32_t* stage, int stage_words) {
  const int64_t nwords = (nbits + 31) / 32;
  const int nt = blockDim.x;
  uint32_t base = 0;                     // positions written by the previous chunks
  for (int64_t c0 = 0; c0 < nwords; c0 += stage_words) {
    const int cw = (int)min((int64_t)stage_words, nwords - c0);
#pragma unroll 8
    for (int i = threadIdx.x; i < cw; i += nt) stage[i] = bm[c0 + i];
    __syncthreads();
    const int per = (cw + nt - 1) / nt;
    const int w0 = min((int)threadIdx.x * per, cw), w1 = min(w0 + per, cw);
    uint32_t cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(stage[i]);
    uint32_t total;
    uint32_t off = base + block_exclusive_scan(cnt, scan_tmp, &total);
    for (int i = w0; i < w1; ++i) {
      uint32_t word = stage[i];
      while (word) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        const int64_t slot = (c0 + i) * 32 + bit;
        if (off < (uint32_t)K) out[off] = slot_pos ? slot_pos[slot] : (int32_t)slot;
        ++off;
      }
    }
    base += total;
    __syncthreads();
  }
  for (int64_t j = (int64_t)base + threadIdx.x; j < K; j += nt) out[j] = -1;
}

// ---------------------------------------------------------------- score kernel


// CAND: score the listed positions (Reindex) instead of every entry. A listed
//      position is used when it lies in [0, n) and is greater than every
//      in-range position listed before it (so the used positions ascend with
//      the slot); the pass stores every slot's score, with the key 0 for a
//      slot it does not use, and selects on (score, position).
// SEL: SEL_NONE (scores only); SEL_THRESHOLD (also the (bin, count) summary of
//      the keys above a local cutoff, for k > 512); SEL_DIRECT (the local
//      cutoff and its candidates, for a finish that picks the top-K); SEL_POOL
//      (SEL_DIRECT's list plus a pool list: every key above a second, lower
//      local cutoff for the pool_k best, with its own header).
// MODE: 0 = dot product of head 0, 1 = sum_h w_h * ReLU(q_h . k).
// QMX: the query is quantized to MXFP8 in registers and each tile is one
//      block-scaled FP8 x FP4 MFMA (the quantized-query variant).
// MQ: queries per workgroup (the multi-query pass of a prefill; Full pass,
//      direct top-k, exact scores only). Sequence index y of the grid is then
//      (sequence bs, query group): queries t0 .. t0+MQ-1 of the Tq queries of
//      sequence bs, which are the virtual sequences bs*Tq + t of the
//      per-query arrays (entry_offset, n_entries = the query's visible
//      entries, q_idx, w, and the selection's headers and lists). Each key
//      tile is read and dequantized once and contracted with every query.
// A workgroup streams SC_SPAN slots (SC_SUB selection chunks of SC_CHUNK);
// eight workgroups of four waves share a compute unit, each wave with
// SC_UNROLL tiles in flight.
template <bool CAND, int SEL, int MODE, bool QMX, int MQ = 1>
__global__ __launch_bounds__(SC_THREADS) __attribute__((amdgpu_waves_per_eu(CAND ? 4 : (MQ > 1 ? 2 : 8)))) void score_kernel(
    const uint8_t* __restrict__ ik, const uint8_t* __restrict__ iks,
    const int64_t* __restrict__ entry_offset, const int32_t* __restrict__ n_entries, int64_t max_n,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int Hi,
    const int32_t* __restrict__ cand, int cand_stride,
    float* __restrict__ scores, int64_t sstride, SelBufs sb, int K, int store_scores, int pool_k, int Tq,
    PrefillViews pv) {
  static_assert(MQ == 1 || (!CAND && SEL == SEL_DIRECT && !QMX), "the multi-query pass is a direct Full pass");
  static_assert(MQ <= SC_THREADS / 64, "one wave per query in the multi-query tail");
  // a candidate-list direct pass takes chunks of kCandChunk slots: more
  // workgroups gather the listed rows, and the finish gets short lists
  constexpr bool SMALL = CAND && SEL == SEL_DIRECT;
  constexpr int SPAN = SMALL ? kCandChunk : SC_SPAN;      // slots of this workgroup
  constexpr int CHUNK = SMALL ? kCandChunk : SC_CHUNK;    // slots of one selection chunk
  static_assert(SPAN % (16 * (SC_THREADS / 64)) == 0 && SPAN <= 4 * SC_THREADS, "whole tiles per wave");
  // histogram with 16-bit counts (two bins per word) + staged scores: 12 KiB,
  // so that eight workgroups fit one compute unit
  __shared__ __attribute__((aligned(16))) uint32_t lbuf[NBINS / 2 + MQ * SC_SPAN];
  __shared__ uint32_t scan_tmp[SC_THREADS / 64 + 1];
  __shared__ uint32_t ctl[8];
  __shared__ __attribute__((aligned(16))) float lw[16 * MQ];   // head weights (per query)
  __shared__ SelBufs sbs;   // the workspace views, parked in LDS while the keys stream (frees SGPRs)
  __shared__ __attribute__((aligned(16))) uint8_t lq[QMX ? QMX_LDS_BYTES : 16];   // the quantized query
  __shared__ uint32_t used_bm[CAND ? SC_SPAN / 32 : 1];     // candidate list: slots used
  __shared__ int32_t lpos[CAND ? SC_SPAN : 1];               // candidate list: the row of each slot
  uint32_t* lhist = lbuf;
  float* lsc = (float*)(lbuf + NBINS / 2);
  auto hcount = [&](uint32_t bin) -> uint32_t { return (lhist[bin >> 1] >> ((bin & 1) * 16)) & 0xFFFFu; };
  constexpr bool LISTS = SEL == SEL_DIRECT || SEL == SEL_POOL;

  // the sequence (or, MQ > 1, query) index of each query's selection
  int vq[MQ];
  bool qok[MQ];
  if constexpr (MQ == 1) {
    vq[0] = blockIdx.y;
    qok[0] = true;
  } else {
    const int QG = (Tq + MQ - 1) / MQ;
    const int bs = blockIdx.y / QG, t0 = (blockIdx.y % QG) * MQ;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      qok[m] = t0 + m < Tq;
      vq[m] = bs * Tq + min(t0 + m, Tq - 1);
    }
  }
  const int b = vq[0];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // the counters of the split pool finish that follows this pass start at zero
  if (SEL == SEL_POOL && blockIdx.x == 0 && tid < 4 && sb.psync) sb.psync[(int64_t)b * 4 + tid] = 0u;
  // independent loads first (the sequence's length and first row, the queries,
  // the head weights), so the keys are requested one round trip after the start
  int32_t neq[MQ];
  int64_t row_base;
  // (MQ > 1: the sequence's arrays and the queries' token positions)
  int64_t nseq = 0, pq[MQ];
  if constexpr (MQ == 1) {
    neq[0] = n_entries[b];
    row_base = entry_offset[b];
    asm volatile("" ::"s"(neq[0]), "s"(row_base));   // both loads issued here, before any branch on them
  } else {
    const int bs = vq[0] / Tq;
    nseq = pv.n_entries[bs];
    row_base = pv.entry_offset[bs];
#pragma unroll
    for (int m = 0; m < MQ; ++m) pq[m] = pv.pos[vq[m]];
#pragma unroll
    for (int m = 0; m < MQ; ++m) asm volatile("" ::"s"(pq[m]));
    asm volatile("" ::"s"(nseq), "s"(row_base));       // every load issued here, the queries' next
  }
  // A operand: q[head = n][channels 32g + 8j .. +7] for MFMA j (the quantized
  // variant builds its operand once the first keys are requested)
  bf16x8_t qa[MQ][4];
  QueryMx qm;
  if constexpr (!QMX) {
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t v = {0, 0, 0, 0};
        if (n < Hi) v = *(const u32x4_t*)(q_idx + ((int64_t)vq[m] * Hi + n) * 128 + 32 * g + 8 * j);
        __builtin_memcpy(&qa[m][j], &v, 16);
      }
  }
  // head weights of the output rows (lane group g takes heads 4g .. 4g+3), in
  // LDS and read per tile, which keeps the wave within 64 registers
  const int wq = tid >> 4, wh = tid & 15;
  const float wv = (tid < 16 * MQ && wh < Hi) ? (w ? w[(int64_t)vq[wq < MQ ? wq : 0] * Hi + wh] : 1.0f) : 0.0f;
  if constexpr (MQ > 1) {
    // the queries' views: the sequence's rows, floor((pos + 1) / m) of them
    // visible (at most its n_entries); the first workgroup of each query
    // group writes them out for the finish and the attention
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      // (a 32-bit division whenever the position allows it)
      const int64_t p1 = pq[m] + 1;
      const int64_t vis = pq[m] < 0 ? 0
                          : (p1 >> 31) == 0 ? (int64_t)((uint32_t)p1 / (uint32_t)pv.m) : p1 / pv.m;
      neq[m] = (int32_t)(vis < nseq ? vis : (nseq < 0 ? 0 : nseq));
    }
    if (blockIdx.x == 0) {
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        if (tid == m && qok[m]) {
          pv.eo[vq[m]] = row_base;
          pv.ne[vq[m]] = neq[m];
        }
      }
    }
  }
  // positions each query's selection covers (MQ > 1: its visible entries)
  int64_t npq[MQ];
  int64_t n_pos = 0;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    npq[m] = qok[m] ? min((int64_t)neq[m], max_n) : 0;
    n_pos = max(n_pos, npq[m]);
  }
  const int64_t nslots = CAND ? (int64_t)cand_stride : n_pos;
  const int64_t start = (int64_t)blockIdx.x * SPAN;
  if (start >= nslots) return;
  if (CAND && n_pos <= 0 && !LISTS) return;        // no listed position can be valid (lists: still written)
  const int end = (int)min((int64_t)SPAN, nslots - start);   // slots of this workgroup
  // the sequence's rows: a uniform base plus a 32-bit byte offset per lane
  // (positions below 2^26, checked on the host), one address register per load
  const uint8_t* ikb = ik + row_base * 64;
  const uint8_t* iksb = iks + row_base * 4;
  const int32_t* crow = CAND ? cand + (int64_t)b * cand_stride : nullptr;
  // Full pass: the first SC_UNROLL tiles of this wave are requested right away
  u32x4_t codes[SC_UNROLL];
  uint32_t sbyte[SC_UNROLL];
  if (!CAND) {
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const uint32_t p = (uint32_t)(start + min(16 * wave + 64 * u + n, end - 1));
      codes[u] = __builtin_nontemporal_load((const u32x4_t*)(ikb + (p * 64u + 16u * g)));
      sbyte[u] = iksb[p * 4u + (uint32_t)g];
    }
  }

  if constexpr (QMX) query_mx_stage(q_idx + (int64_t)b * Hi * 128, Hi, lq, tid);

  if (SEL == SEL_THRESHOLD) {
    for (int i = tid; i < NBINS / 2; i += SC_THREADS) lhist[i] = 0;
  }
  if (SEL == SEL_THRESHOLD) {
    // select_kernel ORs into the bitmap words of this chunk: clear them here
    uint32_t* bm = sb.bitmap + (int64_t)b * sb.bm_stride;
    for (int64_t wd = start / 32 + tid; wd < (start + end + 31) / 32; wd += SC_THREADS) bm[wd] = 0;
  }
  if (tid < 16 * MQ) lw[tid] = wv;
  if (SEL != SEL_NONE && tid == 0) sbs = sb;
  // CAND: each wave's tiles of listed rows, requested before the rule that
  // decides which slots are used is known
  constexpr int CT = SPAN / (16 * (SC_THREADS / 64));      // tiles per wave
  u32x4_t ccw[CAND ? CT : 1];
  uint32_t csb[CAND ? CT : 1];
  if constexpr (CAND) {
    // this workgroup's listed positions (thread t: slots 4t .. 4t+3); a slot
    // reads the row of its position when that lies in [0, n), else row 0 of
    // the sequence, and every tile of the wave is requested at once (one
    // memory round trip for the gathers, overlapping the rule's scan)
    uint32_t pp[4], lmax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      const int32_t c = i < end ? crow[start + i] : -1;
      pp[q] = (c >= 0 && c < n_pos) ? (uint32_t)c + 1u : 0u;
      lmax = max(lmax, pp[q]);
    }
    // (with them, the rule's input: the largest in-range position listed
    // before the workgroup's first slot)
    uint32_t pm = 0;                                   // position + 1, 0 = none
    auto take = [&](int32_t c) { if (c >= 0 && c < n_pos) pm = max(pm, (uint32_t)c + 1u); };
    if ((cand_stride & 3) == 0) {                      // 16-byte rows: four entries per load
#pragma unroll 16
      for (int64_t i = 4 * tid; i < start; i += 4 * SC_THREADS) {
        const u32x4_t v = *(const u32x4_t*)(crow + i);
        take((int32_t)v[0]); take((int32_t)v[1]); take((int32_t)v[2]); take((int32_t)v[3]);
      }
    } else {
#pragma unroll 8
      for (int64_t i = tid; i < start; i += SC_THREADS) take(crow[i]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) lpos[4 * tid + q] = pp[q] > 0u ? (int32_t)pp[q] - 1 : 0;
    __syncthreads();
    if (n_pos > 0) {
#pragma unroll
      for (int u = 0; u < CT; ++u) {
        const uint32_t p = (uint32_t)lpos[16 * wave + 64 * u + n];
        ccw[u] = __builtin_nontemporal_load((const u32x4_t*)(ikb + (p * 64u + 16u * g)));
        csb[u] = iksb[p * 4u + (uint32_t)g];
      }
    }
    // which slots the rule uses: a scan of the workgroup's own slots
    pm = wave_max_u32(pm);
    uint32_t incl = lmax;                              // inclusive max over this wave's threads
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)incl, sh, 64);
      if (lane >= sh) incl = max(incl, o);
    }
    const uint32_t up = (uint32_t)__shfl_up((int)incl, 1, 64);
    if (lane == 63) scan_tmp[wave] = max(incl, pm);
    if (lane == 0) ctl[wave] = pm;
    __syncthreads();
    uint32_t run = lane > 0 ? max(up, pm) : pm;
    for (int v = 0; v < SC_THREADS / 64; ++v) {
      run = max(run, ctl[v]);                          // every wave's share of the earlier slots
      if (v < wave) run = max(run, scan_tmp[v]);
    }
    uint32_t m4 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m4 |= (pp[q] > run ? 1u : 0u) << q;
      run = max(run, pp[q]);
    }
    // 8 threads per word: gather their 4-bit masks
    uint32_t wd = m4 << (4 * (tid & 7));
    wd |= (uint32_t)__shfl_xor((int)wd, 1, 64);
    wd |= (uint32_t)__shfl_xor((int)wd, 2, 64);
    wd |= (uint32_t)__shfl_xor((int)wd, 4, 64);
    if ((tid & 7) == 0) used_bm[tid >> 3] = wd;
  }
  __syncthreads();
  if constexpr (QMX) qm = query_mx_operand(lq, lane);
  // four queries with head weights: each query's weights of this lane
  // group's heads, kept in registers
  constexpr bool QUAD = MQ == 4 && MODE == 1;
  float4 wr4[QUAD ? 4 : 1];
  if constexpr (QUAD) {
#pragma unroll
    for (int m = 0; m < 4; ++m) wr4[m] = *(const float4*)&lw[16 * m + 4 * g];
  }

  // one tile = 16 slots x 16 heads: 4 MFMAs over the 128 channels; the head sum
  // goes to the lanes of group 0, which stage the score in LDS
  auto score_tile = [&](const u32x4_t cw, uint32_t sbyte) -> float {
    if constexpr (QMX) return score_tile_mx<MODE>(qm, cw, sbyte, lw, g);
    else return score_tile_fn<MODE>(qa[0], cw, sbyte, lw, g);
  };
  // The local cutoff of a chunk: a 20-bit key prefix with at least `budget`
  // of the chunk's valid keys at or above it (0 when it has fewer). The keys
  // within two octaves of the chunk's largest prefix M are in a band
  // histogram of 256 bins of 16 prefix units counted down from M; spread over
  // 256 bins the LDS atomics rarely collide. The bin where the running count
  // reaches the budget gives the cutoff; a chunk with fewer than `budget` keys
  // in the band takes the exact path (the 12-bit histogram, then the 256
  // 20-bit sub-bins of the cutoff bin). Thread t owns slots 4t .. 4t+3.
  auto exact_cutoff = [&](const uint32_t (&keys)[4], uint32_t vmask, uint32_t budget) -> uint32_t {
    __syncthreads();                                 // the band histogram's readers are done
    for (int i = tid; i < NBINS / 2; i += SC_THREADS) lhist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((vmask >> q) & 1u) {
        const uint32_t bin = keys[q] >> BIN_SHIFT;
        atomicAdd(&lhist[bin >> 1], 1u << ((bin & 1) * 16));
      }
    }
    __syncthreads();
    uint32_t cnt_all;
    hist_kth_bin<SC_THREADS, true>(lhist, budget, scan_tmp, ctl, &cnt_all);
    const uint32_t cbin = ctl[0], cabove = ctl[1];
    uint32_t fine = 0;                               // fewer keys than the budget: keep all
    if (cbin != 0xFFFFFFFFu) {
      uint32_t* h2 = lhist;                          // every read of the 4096 bins is done (256 words)
      h2[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (((vmask >> q) & 1u) && (keys[q] >> BIN_SHIFT) == cbin) atomicAdd(&h2[(keys[q] >> 12) & 255u], 1u);
      __syncthreads();
      if (tid < 64) digit_kth(h2, budget - cabove, ctl + 4);
      __syncthreads();
      fine = (cbin << 8) | ctl[4];
    }
    return fine;
  };
  // ---- per selection chunk (sub = 0 .. SC_SUB-1): store its scores, then the
  // local cutoff (every slot of a Full pass is a valid position). Chunk cix
  // reports into its own slot of the workspace (a header word and a list), so
  // no global atomics are needed.
  auto chunk_tail = [&](int sub, int mq) {
  const int bq = vq[mq];                             // the selection's sequence (or query) index
  const int64_t npos_q = npq[mq];
  const int end_q = MQ == 1 ? end : (int)max((int64_t)0, min((int64_t)SC_SPAN, npos_q - start));
  const int soff = sub * CHUNK;
  const int send = min(CHUNK, end_q - soff);         // slots of this chunk
  if (send <= 0) return;
  __syncthreads();                                   // its scores are staged; the previous tail is done
  const float* lss = lsc + mq * SC_SPAN + soff;
  const int64_t cix = (int64_t)blockIdx.x * SC_SUB + sub;
  // coalesced store of the chunk's scores (slots of unused candidates hold the key 0)
  if (store_scores) {
    float* srow = scores + (int64_t)bq * sstride + start + soff;
    for (int i4 = 4 * tid; i4 < send; i4 += 4 * SC_THREADS) {
      if (i4 + 3 < send && (((uintptr_t)(srow + i4)) & 15) == 0) {
        *(float4*)(srow + i4) = *(const float4*)(lss + i4);
      } else {
        for (int i = i4; i < min(i4 + 4, send); ++i) srow[i] = lss[i];
      }
    }
  }
  if (SEL == SEL_NONE) return;
  const SelBufs sbl = sbs;
  const int64_t nref = CAND ? nslots : npos_q;       // slots the shares refer to
  const int64_t nwg = (nref + CHUNK - 1) / CHUNK;
  // local budget: a multiple of the chunk's expected share of the top-K plus a
  // margin, so that the highest cutoff over the workgroups still leaves at
  // least K keys of the sequence above it (the finish checks this)
  const int64_t share = ((int64_t)K * CHUNK + nref - 1) / nref;
  int64_t budget64 = LISTS ? 2 * share + 16 : 4 * share + 32;
  if (LISTS) budget64 = min(budget64, max((int64_t)8, (int64_t)FIN_LDS_CANDS / nwg));
  const uint32_t budget = (uint32_t)min(budget64, (int64_t)send);
  uint64_t* hdr = sbl.hdr + (int64_t)bq * sbl.hdr_stride + cix;
  if (SEL == SEL_THRESHOLD) {
    if (sub > 0) {
      for (int i = tid; i < NBINS / 2; i += SC_THREADS) lhist[i] = 0;
      __syncthreads();
    }
    for (int i = tid; i < send; i += SC_THREADS) {
      const uint32_t bin = score_key(lss[i]) >> BIN_SHIFT;
      atomicAdd(&lhist[bin >> 1], 1u << ((bin & 1) * 16));
    }
    __syncthreads();
    uint32_t cnt_all;
    hist_kth_bin<SC_THREADS, true>(lhist, budget, scan_tmp, ctl, &cnt_all);
    const uint32_t cbin = ctl[0];
    // (bin, count) pairs for the non-empty bins >= cut
    const uint32_t cut = (cbin == 0xFFFFFFFFu) ? 0u : cbin;   // fewer keys than the budget: keep all
    uint32_t np = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t bin = NBINS - 1 - (16 * tid + q);
      np += (bin >= cut && hcount(bin) != 0) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t off = block_exclusive_scan(np, scan_tmp, &tot);
    uint32_t* pl = sbl.summ + (int64_t)bq * sbl.summ_stride + cix * SUM_PAIRS;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t bin = NBINS - 1 - (16 * tid + q);
      const uint32_t c = hcount(bin);
      if (bin >= cut && c != 0) {
        if (off < SUM_PAIRS) pl[off] = (bin << 16) | c;
        ++off;
      }
    }
    if (tid == 0) *hdr = ((uint64_t)cut << 32) | (tot > SUM_PAIRS ? 0x80000000u : tot);
  }
  if (LISTS) {
    constexpr uint32_t sh = 4;
    uint32_t* hb = lhist;                            // 256 words
    uint32_t keys[4], pmax = 0, vmask = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      keys[q] = i < send ? score_key(lss[i]) : 0u;
      const bool v = i < send && (!CAND || keys[q] != 0u);
      vmask |= (v ? 1u : 0u) << q;
      if (v) pmax = max(pmax, keys[q] >> 12);
    }
    pmax = wave_max_u32(pmax);
    if (lane == 0) scan_tmp[wave] = pmax;
    hb[tid] = 0;
    __syncthreads();
    uint32_t M = 0;
#pragma unroll
    for (int v = 0; v < SC_THREADS / 64; ++v) M = max(M, scan_tmp[v]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t d = (M - (keys[q] >> 12)) >> sh;
      if (((vmask >> q) & 1u) && d < 256u) atomicAdd(&hb[d], 1u);
    }
    __syncthreads();
    // pool budget: the same rule for the pool_k best
    uint32_t budget_p = 0;
    if (SEL == SEL_POOL) {
      const int64_t share_p = ((int64_t)pool_k * CHUNK + nref - 1) / nref;
      budget_p = (uint32_t)min(2 * share_p + 16, (int64_t)send);
    }
    if (wave == 0) {
      uint32_t hv[4], sl = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { hv[j] = hb[4 * lane + j]; sl += hv[j]; }
      const uint32_t incl = wave_incl_sum(sl);
      // the band bin where the running count reaches each budget (-1: too few in the band)
#pragma unroll
      for (int which = 0; which < (SEL == SEL_POOL ? 2 : 1); ++which) {
        const uint32_t bud = which == 0 ? budget : budget_p;
        uint32_t cum = incl - sl;
        if (cum < bud && incl >= bud) {
          uint32_t ds = 0xFFFFFFFFu;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool hit = ds == 0xFFFFFFFFu && cum + hv[j] >= bud;
            ds = hit ? 4 * lane + j : ds;
            cum += hv[j];
          }
          ctl[4 + which] = ds;
        }
        if (lane == 63 && incl < bud) ctl[4 + which] = 0xFFFFFFFFu;
      }
    }
    __syncthreads();
    const uint32_t ds_k = ctl[4], ds_p = ctl[5];
    // bin ds holds prefixes M - (ds << sh) - (2^sh - 1) .. M - (ds << sh)
    auto band_fine = [&](uint32_t ds) { const uint32_t lo = ((ds + 1u) << sh) - 1u; return M >= lo ? M - lo : 0u; };
    const uint32_t fine = ds_k != 0xFFFFFFFFu ? band_fine(ds_k) : exact_cutoff(keys, vmask, budget);
    uint32_t fine_p = 0;
    if (SEL == SEL_POOL) fine_p = ds_p != 0xFFFFFFFFu ? band_fine(ds_p) : exact_cutoff(keys, vmask, budget_p);
    // candidates: every valid slot whose top 20 key bits are >= fine, in slot order
    auto position = [&](int i) -> uint32_t {
      return CAND ? (uint32_t)crow[start + soff + i] : (uint32_t)(start + soff + i);
    };
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) m |= ((((vmask >> q) & 1u) && (keys[q] >> 12) >= fine) ? 1u : 0u) << q;
    uint32_t tot;
    uint32_t off = block_exclusive_scan((uint32_t)__popc(m), scan_tmp, &tot);
    uint64_t* wc = sbl.wgc + (int64_t)bq * sbl.wgc_stride + cix * CAND_CAP;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((m >> q) & 1u) {
        if (off < CAND_CAP) wc[off] = composite(keys[q], position(4 * tid + q));
        ++off;
      }
    }
    if (tid == 0) *hdr = ((uint64_t)fine << 32) | (tot > CAND_CAP ? 0x80000000u : tot);
    if (SEL == SEL_POOL) {
      // the pool list (never overflows: its capacity is the chunk) and its
      // header: count | cutoff << 11 | M << 32
      uint32_t mp = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) mp |= ((((vmask >> q) & 1u) && (keys[q] >> 12) >= fine_p) ? 1u : 0u) << q;
      uint32_t totp;
      uint32_t offp = block_exclusive_scan((uint32_t)__popc(mp), scan_tmp, &totp);
      uint64_t* wcp = sbl.wgcp + (int64_t)bq * sbl.wgcp_stride + cix * kPoolCap;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((mp >> q) & 1u) {
          wcp[offp] = composite(keys[q], position(4 * tid + q));
          ++offp;
        }
      }
      if (tid == 0)
        sbl.hdrp[(int64_t)bq * sbl.hdr_stride + cix] = ((uint64_t)M << 32) | ((uint64_t)fine_p << 11) | totp;
    }
  }
  };
  if (!CAND) {
    // each wave takes tiles of 16 slots, SC_UNROLL of them in flight: a tile's
    // registers are reloaded with the same tile of the next group as soon as it
    // has been scored, so loads stay in flight all along the chunk
    // (the reloads past the chunk's end re-read its last row, which is in
    // cache; unconditional loads in a fully unrolled loop keep the wait counts
    // exact, and a short last chunk scores its clamped rows without storing them)
    constexpr int NIT = SC_SPAN / (SC_THREADS * SC_UNROLL / 4);
    static_assert(SC_SUB == 1, "one selection chunk per workgroup");
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t0 = 16 * wave + it * 64 * SC_UNROLL;
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        const int ls = t0 + 64 * u + n;
        if constexpr (MQ == 1) {
          const float sc = score_tile(codes[u], sbyte[u]);
          if (g == 0 && ls < end) lsc[ls] = sc;
        } else if constexpr (QUAD) {
          const float sc = score_tile_quad(qa, codes[u], sbyte[u], wr4);   // lane group g: query g
          if (ls < end) lsc[g * SC_SPAN + ls] = sc;
        } else {
          float sc[MQ];
          score_tile_multi<MODE, MQ>(qa, codes[u], sbyte[u], lw, g, sc);
#pragma unroll
          for (int m = 0; m < MQ; ++m)
            if (g == 0 && ls < end) lsc[m * SC_SPAN + ls] = sc[m];
        }
        const uint32_t p = (uint32_t)(start + min(ls + 64 * SC_UNROLL, end - 1));
        codes[u] = __builtin_nontemporal_load((const u32x4_t*)(ikb + (p * 64u + 16u * g)));
        sbyte[u] = iksb[p * 4u + (uint32_t)g];
      }
    }
  } else if (n_pos <= 0) {
    // an empty sequence: no listed position is used
    const float unused = LISTS ? __uint_as_float(0xFFFFFFFFu) : 0.0f;
    for (int i = tid; i < end; i += SC_THREADS) lsc[i] = unused;
  } else {
    // listed positions: the tiles requested above; unused slots hold the key 0
    const float unused = __uint_as_float(0xFFFFFFFFu);     // key 0
#pragma unroll
    for (int u = 0; u < CT; ++u) {
      const float sc = score_tile(ccw[u], csb[u]);
      const int ls = 16 * wave + 64 * u + n;
      const bool ok = ls < end && ((used_bm[ls >> 5] >> (ls & 31)) & 1u);
      if (g == 0 && ls < end) lsc[ls] = ok ? sc : (LISTS ? unused : 0.0f);
    }
  }
  // (the multi-query pass: one wave per query computes that query's local
  // cutoff and list, so the queries' tails run side by side; a single query's
  // tail is faster on the whole workgroup)
  if constexpr (MQ == 1) {
    chunk_tail(0, 0);
  } else {
    __syncthreads();                                 // every query's scores are staged
    if (wave < MQ) {
      const int64_t nref = npq[wave];
      const int send = (int)max((int64_t)0, min((int64_t)SC_SPAN, nref - start));
      if (send > 0) {
        const SelBufs sbl = sbs;
        const int64_t nwg = (nref + SC_CHUNK - 1) / SC_CHUNK;
        const int64_t share = ((int64_t)K * SC_CHUNK + nref - 1) / nref;
        const int64_t budget64 = min(2 * share + 16, max((int64_t)8, (int64_t)FIN_LDS_CANDS / nwg));
        const int64_t cix = blockIdx.x;
        wave_direct_tail(lsc + wave * SC_SPAN, send, (uint32_t)min(budget64, (int64_t)send), lhist + 256 * wave,
                         sbl.hdr + (int64_t)vq[wave] * sbl.hdr_stride + cix,
                         sbl.wgc + (int64_t)vq[wave] * sbl.wgc_stride + cix * CAND_CAP, CAND_CAP,
                         [&](int i) { return (uint32_t)(start + i); });
      }
    }
  }
}

// ---------------------------------------------------------------- finish (one workgroup per sequence)
// Runs after the score pass. Every score workgroup w of the sequence left a
// header word (count | overflow bit 31, cutoff << 32) and a list in its own
// slot. The cutoffs differ per workgroup; at or above the highest of them
// every workgroup's list is complete.

// Threshold bin of the K-th best key from the (bin, count) pair lists, exact
// when the merged bins at or above the highest cutoff hold at least K keys;
// otherwise from a histogram of every score of the sequence. The bin and the
// count above it go to the control block for select_kernel.
__global__ __launch_bounds__(SC_THREADS) void finish_threshold_kernel(
    const int32_t* __restrict__ n_entries, int64_t max_n, const float* __restrict__ scores, int64_t sstride,
    SelBufs sb, int K) {
  __shared__ uint32_t lhist[NBINS];
  __shared__ uint32_t lcnt[FIN_MAX_WG];
  __shared__ uint32_t scan_tmp[32];
  __shared__ uint32_t ctl[8];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t n_pos = min((int64_t)n_entries[b], max_n);
  SelState* st = ctrl_state(sb.ctrl, b);
  if (tid == 0) st->ncand = 0;            // select_kernel counts its candidates from here
  if (n_pos <= K) {                       // every position is selected (or none exists)
    if (tid == 0) { st->thr_bin = -1; st->above = 0; }
    return;
  }
  const float* sall = scores + (int64_t)b * sstride;
  const int64_t nw = (n_pos + SC_CHUNK - 1) / SC_CHUNK;
  for (int i = tid; i < NBINS; i += SC_THREADS) lhist[i] = 0;
  bool exact = false;
  uint32_t T = 0, above = 0, tot = 0;
  if (nw <= FIN_MAX_WG) {
    const uint64_t* hd = sb.hdr + (int64_t)b * sb.hdr_stride;
    uint32_t cmax = 0, ovf = 0;
    for (int w = tid; w < nw; w += SC_THREADS) {
      const uint64_t h = hd[w];
      lcnt[w] = min((uint32_t)h & 0x7FFFFFFFu, (uint32_t)SUM_PAIRS);
      ovf |= (uint32_t)h >> 31;
      cmax = max(cmax, (uint32_t)(h >> 32));
    }
    block_max_or_u32(&cmax, &ovf, scan_tmp);
    if (ovf == 0) {
      const uint32_t* pl = sb.summ + (int64_t)b * sb.summ_stride;
      for (int64_t i = tid; i < nw * SUM_PAIRS; i += SC_THREADS) {
        if ((uint32_t)(i % SUM_PAIRS) < lcnt[i / SUM_PAIRS]) {
          const uint32_t v = pl[i];
          if ((v >> 16) >= cmax) atomicAdd(&lhist[v >> 16], v & 0xFFFFu);
        }
      }
      __syncthreads();
      hist_kth_bin<SC_THREADS>(lhist, (uint32_t)K, scan_tmp, ctl, &tot);
      exact = ctl[0] != 0xFFFFFFFFu;
      T = ctl[0];
      above = ctl[1];
    }
  }
  if (!exact) {
    __syncthreads();
    for (int i = tid; i < NBINS; i += SC_THREADS) lhist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n_pos; i += SC_THREADS) atomicAdd(&lhist[score_key(sall[i]) >> BIN_SHIFT], 1u);
    __syncthreads();
    hist_kth_bin<SC_THREADS>(lhist, (uint32_t)K, scan_tmp, ctl, &tot);
    T = ctl[0];
    above = ctl[1];
  }
  if (tid == 0) { st->thr_bin = (int32_t)T; st->above = above; }
}

// Direct top-K (K <= kDirectMaxK), one workgroup per sequence: the steps of
// finish_direct_body, written to out[b][0 .. K).
__global__ __launch_bounds__(FIN_THREADS) void finish_direct_kernel(
    const int32_t* __restrict__ n_entries, int64_t max_n, float* __restrict__ scores, int64_t sstride,
    SelBufs sb, int K, int32_t* __restrict__ out, int out_stride, ScoreSrc src, int rescore) {
  __shared__ uint64_t lc[FIN_LDS_CANDS];
  __shared__ uint64_t sub[FIN_SUB_CAP];
  __shared__ uint32_t loff[FIN_MAX_WG];
  __shared__ uint32_t h[512];
  __shared__ uint64_t red[32];
  __shared__ uint32_t scan_tmp[32];
  __shared__ uint32_t ctl[8];
  __shared__ uint64_t binl[FIN_RANK_MAX];
  __shared__ uint32_t bin_count;
  const int b = blockIdx.x;
  int32_t* ob = out + (int64_t)b * out_stride;
  const FinLds L{lc, sub, loff, h, red, scan_tmp, ctl, binl, &bin_count};
  FinPrefetch<FIN_THREADS> pf;
  finish_prefetch<FIN_THREADS>(pf, b, max_n, sb, src);
  finish_direct_body<FIN_THREADS>(b, n_entries, max_n, scores + (int64_t)b * sstride,
                                  sb.gscr + (int64_t)b * sb.gscr_stride, sb, K, src, rescore, L, pf,
                                  [&](int j, int32_t v) { ob[j] = v; });
}

// Pool finish, one workgroup per sequence: pool_finish_body written to
// pool[b][0 .. pool_k). sc_rows / g_rows: the sequence's scratch rows for the
// fallback (scores recomputed, composites of a large threshold bin).
__global__ __launch_bounds__(FIN_THREADS) void pool_finish_kernel(
    const int32_t* __restrict__ n_entries, int64_t max_n, SelBufs sb, int pool_k, int32_t* __restrict__ pool,
    float* __restrict__ sc_rows, int64_t sc_stride, uint64_t* __restrict__ g_rows, int64_t g_stride, ScoreSrc src) {
  __shared__ uint64_t lc[FIN_LDS_CANDS];
  __shared__ uint64_t sub[FIN_SUB_CAP];
  __shared__ uint32_t loff[FIN_MAX_WG];
  __shared__ uint32_t h[512];
  __shared__ uint64_t red[32];
  __shared__ uint32_t scan_tmp[32];
  __shared__ uint32_t ctl[8];
  __shared__ uint64_t binl[FIN_RANK_MAX];
  __shared__ uint32_t bin_count;
  const int b = blockIdx.x;
  int32_t* ob = pool + (int64_t)b * pool_k;
  const FinLds L{lc, sub, loff, h, red, scan_tmp, ctl, binl, &bin_count};
  pool_finish_body<FIN_THREADS>(b, n_entries, max_n, pool_k, sb, sc_rows + (int64_t)b * sc_stride,
                                g_rows + (int64_t)b * g_stride, src, L, [&](int j, int32_t v) { ob[j] = v; });
}

// ---------------------------------------------------------------- select (long)
// Marking pass: every key above the threshold bin sets its bit in the
// sequence's bitmap; keys inside the bin are appended as (key, position)
// candidates. select_finish_kernel completes the selection.
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t sstride, const int32_t* __restrict__ n_entries,
    int64_t max_n, uint8_t* __restrict__ ctrl, uint32_t* __restrict__ bitmap, int64_t bm_stride,
    uint64_t* __restrict__ cbuf, int64_t cb_stride) {
  const int b = blockIdx.y;
  const int64_t nb = min((int64_t)n_entries[b], max_n);
  const int64_t start = (int64_t)blockIdx.x * SEL_CHUNK;
  if (start >= nb) return;
  const int64_t end = min(start + (int64_t)SEL_CHUNK, nb);
  SelState* st = ctrl_state(ctrl, b);
  const int thr = st->thr_bin;
  uint32_t* bm = bitmap + (int64_t)b * bm_stride;
  uint64_t* cb = cbuf + (int64_t)b * cb_stride;
  const float* sb = scores + (int64_t)b * sstride;
  const int lane = threadIdx.x & 63;

  for (int64_t base = start + (threadIdx.x & ~63); base < end; base += SEL_THREADS) {
    const int64_t i = base + lane;
    bool sel = false, cnd = false;
    uint32_t key = 0;
    if (i < end) {
      key = score_key(sb[i]);
      const int bin = (int)(key >> BIN_SHIFT);
      sel = bin > thr;
      cnd = bin == thr;
    }
    const uint64_t bs = __ballot(sel);
    if (bs) {   // a wave covers 64 consecutive slots: base is a multiple of 64
      if (lane == 0 && (uint32_t)bs) atomicOr(&bm[base >> 5], (uint32_t)bs);
      if (lane == 32 && (uint32_t)(bs >> 32)) atomicOr(&bm[(base >> 5) + 1], (uint32_t)(bs >> 32));
    }
    const uint64_t bc = __ballot(cnd);
    if (bc) {
      uint32_t basei = 0;
      if (lane == 0) basei = atomicAdd(&st->ncand, (uint32_t)__popcll(bc));
      basei = readlane_u32(basei, 0);
      if (cnd) {
        // (ncand was set to zero by finish_threshold_kernel; the bound keeps
        // the writes inside the row)
        const uint64_t at = (uint64_t)basei + (uint32_t)__popcll(bc & ((1ull << lane) - 1ull));
        if (at < (uint64_t)cb_stride) cb[at] = composite(key, (uint32_t)i);
      }
    }
  }
}

// One workgroup per sequence: picks the missing keys among the threshold-bin
// candidates, then compacts the bitmap into ascending positions.
__global__ __launch_bounds__(SEL_THREADS) void select_finish_kernel(
    const int32_t* __restrict__ n_entries, int64_t max_n, uint8_t* __restrict__ ctrl,
    uint32_t* __restrict__ bitmap, int64_t bm_stride, const uint64_t* __restrict__ cbuf, int64_t cb_stride,
    int K, int32_t* __restrict__ out, int out_stride) {
  __shared__ uint32_t h[512];
  __shared__ uint32_t ctl[8];
  __shared__ uint32_t scan_tmp[SEL_THREADS / 64 + 1];
  __shared__ uint64_t lcand[SEL_LDS_CAP];
  __shared__ uint64_t red[32];
  const int b = blockIdx.x;
  const int64_t nb = min((int64_t)n_entries[b], max_n);
  int32_t* ob = out + (int64_t)b * out_stride;
  SelState* st = ctrl_state(ctrl, b);
  const int thr = st->thr_bin;
  const uint32_t above = st->above;
  // the candidates are a subset of the sequence's nb slots: clamp defensively
  const uint32_t ncand = min(st->ncand, (uint32_t)max(nb, (int64_t)0));
  __syncthreads();
  if (threadIdx.x == 0) { st->ncand = 0; st->thr_bin = 0; st->above = 0; }
  if (nb <= 0) {
    for (int j = threadIdx.x; j < K; j += SEL_THREADS) ob[j] = -1;
    return;
  }
  uint32_t* bm = bitmap + (int64_t)b * bm_stride;
  const uint64_t* cb = cbuf + (int64_t)b * cb_stride;
  const uint32_t need = (thr >= 0 && (uint32_t)K > above) ? (uint32_t)K - above : 0u;
  if (need > 0) {
    if (need >= ncand) {
      for (uint32_t i = threadIdx.x; i < ncand; i += SEL_THREADS) {
        const uint32_t pos = 0xFFFFFFFFu - (uint32_t)cb[i];
        atomicOr(&bm[pos >> 5], 1u << (pos & 31));
      }
    } else {
      const bool in_lds = ncand <= SEL_LDS_CAP;
      if (in_lds) {
        for (uint32_t i = threadIdx.x; i < ncand; i += SEL_THREADS) lcand[i] = cb[i];
        __syncthreads();
      }
      const uint64_t* src = in_lds ? (const uint64_t*)lcand : cb;
      uint64_t prefix, mask;
      const int top = radix_top_shift(src, ncand, red);
      radix_select_u64(src, ncand, need, top, h, ctl, &prefix, &mask);
      for (uint32_t i = threadIdx.x; i < ncand; i += SEL_THREADS) {
        const uint64_t c = src[i];
        if ((c & mask) >= prefix) {
          const uint32_t pos = 0xFFFFFFFFu - (uint32_t)c;
          atomicOr(&bm[pos >> 5], 1u << (pos & 31));
        }
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  compact_bitmap(bm, nb, nullptr, K, ob, scan_tmp, (uint32_t*)lcand, 2 * SEL_LDS_CAP);
}

// ---------------------------------------------------------------- select (small)
// slot_pos: [B][pstride] slot -> position (NULL: slot == position, nslots =
// min(n_entries[b], max_n)). score_by_pos: the score of a slot is
// scores[position] (pool of a Full layer) rather than scores[slot].
// A listed position is used when it lies in [0, n) and is greater than every
// in-range position listed before it, so the used slots are in ascending
// position order and distinct (a pool is written that way; out-of-order and
// repeated entries of a caller's list are skipped) and slot order is position
// order for the tie rule and the output.
__global__ __launch_bounds__(SMALL_THREADS) void select_small_kernel(
    const float* __restrict__ scores, int64_t sstride, const int32_t* __restrict__ slot_pos,
    int pstride, int score_by_pos, const int32_t* __restrict__ n_entries, int64_t max_n, int K,
    int32_t* __restrict__ out, int out_stride) {
  constexpr int PER = SMALL_MAX / SMALL_THREADS;   // 16 consecutive slots per thread
  __shared__ uint32_t keys[SMALL_MAX];
  __shared__ uint32_t valid[SMALL_MAX / 32];
  __shared__ uint32_t selbm[SMALL_MAX / 32];
  __shared__ uint32_t h[256];
  __shared__ uint32_t ctl[4];
  __shared__ uint32_t scan_tmp[SMALL_THREADS / 64 + 1];

  const int b = blockIdx.x;
  const int64_t n_pos = min((int64_t)n_entries[b], max_n);
  const int nslots = slot_pos ? pstride : (int)min(n_pos, (int64_t)SMALL_MAX);
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)b * pstride : nullptr;
  const float* sb = scores + (int64_t)b * sstride;
  int32_t* ob = out + (int64_t)b * out_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < SMALL_MAX / 32; i += SMALL_THREADS) selbm[i] = 0;
  // this thread's slots PER*tid .. +PER-1: positions (+1; 0 = not in range)
  uint32_t pp[PER], lmax = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = PER * tid + q;
    int64_t pos = -1;
    if (i < nslots) pos = sp ? (int64_t)sp[i] : (int64_t)i;
    pp[q] = (pos >= 0 && pos < n_pos) ? (uint32_t)pos + 1u : 0u;
    lmax = max(lmax, pp[q]);
  }
  // exclusive max over the threads before this one (slot order)
  uint32_t incl = lmax;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)incl, sh, 64);
    if (lane >= sh) incl = max(incl, o);
  }
  if (lane == 63) scan_tmp[wave] = incl;
  const uint32_t up = (uint32_t)__shfl_up((int)incl, 1, 64);
  __syncthreads();
  uint32_t run = lane > 0 ? up : 0u;
  for (int v = 0; v < wave; ++v) run = max(run, scan_tmp[v]);
  uint32_t m16 = 0, nvalid = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const bool ok = pp[q] > run;
    run = max(run, pp[q]);
    if (ok) {
      const int i = PER * tid + q;
      keys[i] = score_key(sb[score_by_pos ? (int64_t)pp[q] - 1 : (int64_t)i]);
      m16 |= 1u << q;
      ++nvalid;
    }
  }
  {
    const uint32_t other = (uint32_t)__shfl_xor((int)m16, 1, 64);
    if ((tid & 1) == 0) valid[tid >> 1] = m16 | (other << 16);
  }
  __syncthreads();
  uint32_t total;
  block_exclusive_scan(nvalid, scan_tmp, &total);
  if (total <= (uint32_t)K) {
    for (int i = threadIdx.x; i < SMALL_MAX / 32; i += SMALL_THREADS) selbm[i] = valid[i];
  } else {
    // composite (key << 14) | (16383 - slot): larger is better, distinct per slot.
    // Radix select over 48 bits with the composites formed on the fly.
    uint64_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)K;
    int shift = 40;
    for (;;) {
      for (int i = threadIdx.x; i < 256; i += SMALL_THREADS) h[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < nslots; i += SMALL_THREADS) {
        if (!((valid[i >> 5] >> (i & 31)) & 1u)) continue;
        const uint64_t c = ((uint64_t)keys[i] << 14) | (uint64_t)(SMALL_MAX - 1 - i);
        if ((c & pmask) == prefix) atomicAdd(&h[(uint32_t)(c >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) digit_kth(h, need, ctl);
      __syncthreads();
      const uint32_t d = ctl[0], above = ctl[1], cnt = ctl[2];
      __syncthreads();
      prefix |= (uint64_t)d << shift;
      pmask |= (uint64_t)255 << shift;
      need -= above;
      if (cnt == need || shift == 0) break;
      shift = shift >= 8 ? shift - 8 : 0;
    }
    for (int i = threadIdx.x; i < nslots; i += SMALL_THREADS) {
      if (!((valid[i >> 5] >> (i & 31)) & 1u)) continue;
      const uint64_t c = ((uint64_t)keys[i] << 14) | (uint64_t)(SMALL_MAX - 1 - i);
      if ((c >> shift) >= (prefix >> shift)) atomicOr(&selbm[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  compact_bitmap(selbm, nslots, sp, K, ob, scan_tmp, keys, SMALL_MAX);
}

// ---------------------------------------------------------------- prefill views
// Query t of sequence b becomes sequence b * Tq + t of a decode batch: the same
// cache rows, with the entries its token has completed visible, floor((pos + 1) / m)
// of them (at most the sequence's n_entries).
__global__ void prefill_views_kernel(const int64_t* __restrict__ entry_offset, const int32_t* __restrict__ n_entries,
                                     const int64_t* __restrict__ pos, int m, int B, int Tq,
                                     int64_t* __restrict__ eo, int32_t* __restrict__ ne) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * Tq) return;
  const int b = i / Tq;
  const int64_t p = pos[i];
  const int64_t vis = p < 0 ? 0 : (p + 1) / m;
  const int64_t n = n_entries[b];
  eo[i] = entry_offset[b];
  ne[i] = (int32_t)(vis < n ? vis : (n < 0 ? 0 : n));
}

hipError_t launch_prefill_views(const int64_t* entry_offset, const int32_t* n_entries, const int64_t* pos, int m,
                                int B, int Tq, int64_t* eo, int32_t* ne, hipStream_t stream) {
  const int n = B * Tq;
  hipLaunchKernelGGL(prefill_views_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, entry_offset,
                     n_entries, pos, m, B, Tq, eo, ne);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
hipError_t launch_score(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                        const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                        const float* w, int Hi, int mode, const int32_t* cand, int cand_stride,
                        float* scores, int64_t sstride, const SelBufs& sb, int sel, int K,
                        bool store_scores, int pool_k, hipStream_t stream) {
  const bool store = store_scores || cand || (sel != SEL_DIRECT && sel != SEL_POOL);
  const int64_t nslots = cand ? cand_stride : max_n;
  if (nslots <= 0) return hipSuccess;
  const int span = (cand && sel == SEL_DIRECT) ? kCandChunk : SC_SPAN;   // the kernel's SPAN
  const int64_t nx = (nslots + span - 1) / span;
  dim3 grid((unsigned)nx, (unsigned)B), block(SC_THREADS);
  const bool qmx = (mode & kScoreQmx8) != 0;
  const int base = mode & ~kScoreQmx8;
#define CSA2_SCORE_LAUNCH1(C, S, Mo, Q)                                                          \
  hipLaunchKernelGGL((score_kernel<C, S, Mo, Q>), grid, block, 0, stream, ik, iks, entry_offset, \
                     n_entries, max_n, q_idx, w, Hi, cand, cand_stride, scores, sstride, sb, K,  \
                     (int)store, pool_k, 0, PrefillViews{})
#define CSA2_SCORE_LAUNCH(C, S)                                                                  \
  if (base == 0) {                                                                               \
    if (qmx) CSA2_SCORE_LAUNCH1(C, S, 0, true); else CSA2_SCORE_LAUNCH1(C, S, 0, false);         \
  } else {                                                                                       \
    if (qmx) CSA2_SCORE_LAUNCH1(C, S, 1, true); else CSA2_SCORE_LAUNCH1(C, S, 1, false);         \
  }
  if (cand) {
    if (sel == SEL_DIRECT) {
      CSA2_SCORE_LAUNCH(true, SEL_DIRECT)
    } else {
      CSA2_SCORE_LAUNCH(true, SEL_NONE)
    }
  } else if (sel == SEL_THRESHOLD) {
    CSA2_SCORE_LAUNCH(false, SEL_THRESHOLD)
  } else if (sel == SEL_DIRECT) {
    CSA2_SCORE_LAUNCH(false, SEL_DIRECT)
  } else if (sel == SEL_POOL) {
    CSA2_SCORE_LAUNCH(false, SEL_POOL)
  } else {
    CSA2_SCORE_LAUNCH(false, SEL_NONE)
  }
#undef CSA2_SCORE_LAUNCH
#undef CSA2_SCORE_LAUNCH1
  return hipGetLastError();
}

// The multi-query pass of a prefill: B sequences of Tq queries each, scored
// PREFILL_MQ queries per workgroup, selections per query (the virtual
// sequences b * Tq + t of q_idx, w, sb and the views it writes to pv.eo and
// pv.ne); direct mode, exact scores.
constexpr int PREFILL_MQ = 4;

hipError_t launch_score_prefill(const uint8_t* ik, const uint8_t* iks, int B, int Tq, int64_t max_n,
                                const uint16_t* q_idx, const float* w, int Hi, int mode, const SelBufs& sb, int K,
                                const PrefillViews& pv, hipStream_t stream) {
  if (max_n <= 0)   // nothing to score: the views alone
    return launch_prefill_views(pv.entry_offset, pv.n_entries, pv.pos, pv.m, B, Tq, pv.eo, pv.ne, stream);
  if ((mode & kScoreQmx8) != 0) return hipErrorInvalidValue;
  const int QG = (Tq + PREFILL_MQ - 1) / PREFILL_MQ;
  dim3 grid((unsigned)((max_n + SC_SPAN - 1) / SC_SPAN), (unsigned)(B * QG)), block(SC_THREADS);
  if (mode == 0)
    hipLaunchKernelGGL((score_kernel<false, SEL_DIRECT, 0, false, PREFILL_MQ>), grid, block, 0, stream, ik, iks, nullptr,
                       nullptr, max_n, q_idx, w, Hi, nullptr, 0, nullptr, 0, sb, K, 0, 0, Tq, pv);
  else
    hipLaunchKernelGGL((score_kernel<false, SEL_DIRECT, 1, false, PREFILL_MQ>), grid, block, 0, stream, ik, iks, nullptr,
                       nullptr, max_n, q_idx, w, Hi, nullptr, 0, nullptr, 0, sb, K, 0, 0, Tq, pv);
  return hipGetLastError();
}

hipError_t launch_pool_finish(const int32_t* n_entries, int B, int64_t max_n, const SelBufs& sb, int pool_k,
                              int32_t* pool, float* sc_rows, int64_t sc_stride, uint64_t* g_rows, int64_t g_stride,
                              const ScoreSrc& src, hipStream_t stream) {
  hipLaunchKernelGGL(pool_finish_kernel, dim3((unsigned)B), dim3(FIN_THREADS), 0, stream, n_entries, max_n, sb,
                     pool_k, pool, sc_rows, sc_stride, g_rows, g_stride, src);
  return hipGetLastError();
}

hipError_t launch_finish(int sel, const int32_t* n_entries, int B, int64_t max_n, float* scores,
                         int64_t sstride, const SelBufs& sb, int K, int32_t* out, int out_stride,
                         const ScoreSrc* src, hipStream_t stream) {
  if (sel == SEL_DIRECT)
    hipLaunchKernelGGL(finish_direct_kernel, dim3((unsigned)B), dim3(FIN_THREADS), 0, stream, n_entries, max_n,
                       scores, sstride, sb, K, out, out_stride, src ? *src : ScoreSrc{},
                       (src && !src->cand) ? 1 : 0);
  else
    hipLaunchKernelGGL(finish_threshold_kernel, dim3((unsigned)B), dim3(SC_THREADS), 0, stream, n_entries,
                       max_n, scores, sstride, sb, K);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t sstride, const int32_t* n_entries, int B,
                         int64_t max_n, uint8_t* ctrl, uint32_t* bitmap, int64_t bm_stride,
                         uint64_t* cbuf, int64_t cb_stride, int K, int32_t* out, int out_stride,
                         hipStream_t stream) {
  if (max_n > 0) {
    dim3 grid((unsigned)((max_n + SEL_CHUNK - 1) / SEL_CHUNK), (unsigned)B), block(SEL_THREADS);
    hipLaunchKernelGGL(select_kernel, grid, block, 0, stream, scores, sstride, n_entries, max_n, ctrl, bitmap,
                       bm_stride, cbuf, cb_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)B), dim3(SEL_THREADS), 0, stream, n_entries, max_n,
                     ctrl, bitmap, bm_stride, cbuf, cb_stride, K, out, out_stride);
  return hipGetLastError();
}

hipError_t launch_select_small(const float* scores, int64_t sstride, const int32_t* slot_pos,
                               int pstride, int score_by_pos, const int32_t* n_entries, int B,
                               int64_t max_n, int K, int32_t* out, int out_stride, hipStream_t stream) {
  dim3 grid((unsigned)B), block(SMALL_THREADS);
  hipLaunchKernelGGL(select_small_kernel, grid, block, 0, stream, scores, sstride, slot_pos, pstride,
                     score_by_pos, n_entries, max_n, K, out, out_stride);
  return hipGetLastError();
}

}  // namespace csa2
