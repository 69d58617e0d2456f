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
//                with coalesced 16-byte stores.
//                Selection without contended atomics: each workgroup builds an
//                LDS histogram of its 1024 score keys, picks a local cutoff bin
//                that keeps about four times its expected share of the top-k,
//                and writes to its own slot the (bin, count) pairs above that
//                cutoff (and, for k <= 512, the candidates themselves). The last
//                workgroup of a sequence merges the slots: bins at or above the
//                highest cutoff are complete, so the bin holding the k-th best
//                key follows exactly whenever it lies there (otherwise it falls
//                back to a full histogram of the sequence's scores). For
//                k <= 512 it then radix-selects the k best among the gathered
//                candidates and writes them in ascending order; larger k (the
//                hierarchical pool) go on to select_kernel.
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

namespace csa2 {

constexpr int SC_THREADS = 256;
constexpr int SC_CHUNK = kScoreChunk;   // slots per score workgroup

constexpr int SC_SUB = 1;           // selection chunks per score workgroup
constexpr int SC_SPAN = SC_SUB * SC_CHUNK;   // slots a score workgroup streams
constexpr int SC_UNROLL = 4;        // tiles in flight per wave
constexpr int NBINS = 4096;         // histogram over the top 12 bits of the key
constexpr int BIN_SHIFT = 20;
constexpr int SUM_PAIRS = kSumWords;   // (bin, count) pairs a workgroup reports above its cutoff
constexpr int CAND_CAP = kCandCap;     // candidates a workgroup reports in direct top-k mode

constexpr int FIN_THREADS = 1024;  // finish workgroup of the direct top-k
constexpr int FIN_MAX_WG = kFinMaxWg;        // score workgroups per sequence the finish reads
constexpr int FIN_LDS_CANDS = kFinLdsCands;  // candidates the direct finish keeps in LDS
constexpr int FIN_SUB_CAP = 4096;   // keys of the threshold bin the direct finish keeps in LDS
constexpr int FIN_RANK_MAX = 256;   // threshold bins up to this size are resolved by ranking
constexpr int FIN_RUN = (kFinLdsCands + FIN_THREADS - 1) / FIN_THREADS;   // candidates per thread (direct finish)
constexpr int SEL_THREADS = 256;
constexpr int SEL_CHUNK = 4096;     // slots per select workgroup
constexpr int SEL_LDS_CAP = 4096;   // candidates staged in LDS by the last select workgroup
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_MAX = 16384;

// ---------------------------------------------------------------- block scan
// Exclusive prefix sum over the workgroup (blockDim.x multiple of 64); returns
// the total in *total. `tmp` holds at least blockDim.x/64 + 1 words of LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  // the wave totals, scanned across lanes 0 .. nw-1 of every wave
  const uint32_t t = lane < nw ? tmp[lane] : 0u;
  const uint32_t ti = wave_incl_sum(t);
  const uint32_t pre = readlane_u32(ti - t, wave);
  *total = readlane_u32(ti, nw - 1);
  __syncthreads();
  return pre + x - v;
}

// ---------------------------------------------------------------- scoring helpers
__device__ __forceinline__ bf16x8_t dequant_mx_block8(uint32_t dw, float scale) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 0);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 1);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 2);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 3);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Sum of v over the four lanes l, l^16, l^32, l^48 (VALU lane swaps, no LDS).
__device__ __forceinline__ float sum_lane_groups(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float t = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// ---------------------------------------------------------------- radix select
// Run by the 64 lanes of wave 0: among the 256 digit counts h (digit 255 is the
// best), finds the digit that holds the need-th best element (1 <= need <= the
// sum of h): ctl[0] = digit, ctl[1] = count strictly above it, ctl[2] = count
// with it. Lane l scans digits 255-4l .. 252-4l.
__device__ __forceinline__ void digit_kth(const uint32_t* h, uint32_t need, uint32_t* ctl) {
  const int l = threadIdx.x & 63;
  uint32_t c4[4], loc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) { c4[q] = h[255 - 4 * l - q]; loc += c4[q]; }
  const uint32_t pre = wave_incl_sum(loc) - loc;
  if (pre < need && pre + loc >= need) {
    uint32_t cum = pre;
    for (int q = 0; q < 4; ++q) {
      if (cum + c4[q] >= need) {
        ctl[0] = 255 - 4 * l - q;
        ctl[1] = cum;
        ctl[2] = c4[q];
        break;
      }
      cum += c4[q];
    }
  }
}

// Among n distinct 64-bit composites at `v` (LDS, or global memory read after
// an acquire fence), find the `need` largest (0 < need < n); all composites
// agree on the bits above top_shift + 7. On return the composites c with
// (c & *mask_out) >= *prefix_out are exactly the `need` largest. h holds 512
// words and ctl 8 words of LDS. All threads of the workgroup must call it.
__device__ void radix_select_u64(const uint64_t* v, uint32_t n, uint32_t need, int top_shift,
                                 uint32_t* h, uint32_t* ctl, uint64_t* prefix_out, uint64_t* mask_out) {
  // h: two 256-bin histograms and ctl: two 4-word results, alternating by pass,
  // so each pass needs two barriers
  uint64_t prefix = 0, pmask = 0;
  int shift = top_shift;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) h[i] = 0;
  __syncthreads();
  for (int p = 0;; p ^= 1) {
    uint32_t* hp = h + 256 * p;
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t c = v[i];
      if ((c & pmask) == prefix) atomicAdd(&hp[(uint32_t)(c >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) digit_kth(hp, need, ctl + 4 * p);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h[256 * (p ^ 1) + i] = 0;
    __syncthreads();
    const uint32_t d = ctl[4 * p], above = ctl[4 * p + 1], cnt = ctl[4 * p + 2];
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)255 << shift;
    need -= above;
    if (cnt == need || shift == 0) break;
    shift = shift >= 8 ? shift - 8 : 0;     // the last digit may overlap resolved bits
  }
  *prefix_out = prefix;
  *mask_out = pmask;
}

// Index in an LDS list for the lanes whose `take` is set: one LDS atomic per wave.
__device__ __forceinline__ uint32_t wave_append(bool take, uint32_t* counter) {
  const uint64_t m = __ballot(take);
  const int lane = threadIdx.x & 63;
  uint32_t base = 0;
  if (m) {
    const int leader = __ffsll((long long)m) - 1;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = readlane_u32(base, leader);
  }
  return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// Top shift for radix_select_u64 over n composites at v: the 8-bit digit that
// holds the highest bit in which any two composites differ (bits above it are
// common to all of them). All threads of the workgroup must call it.
__device__ int radix_top_shift(const uint64_t* v, uint32_t n, uint64_t* red) {
  uint64_t o = 0, a = ~0ull;
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) { o |= v[i]; a &= v[i]; }
  o = ((uint64_t)wave_or_u32((uint32_t)(o >> 32)) << 32) | wave_or_u32((uint32_t)o);
  a = ((uint64_t)wave_and_u32((uint32_t)(a >> 32)) << 32) | wave_and_u32((uint32_t)a);
  const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;   // at most 16 waves; red holds 32 words
  if (lane == 0) { red[threadIdx.x >> 6] = o; red[16 + (threadIdx.x >> 6)] = a; }
  __syncthreads();
  o = lane < nw ? red[lane] : 0ull;
  a = lane < nw ? red[16 + lane] : ~0ull;
  __syncthreads();
  o = ((uint64_t)wave_or_u32((uint32_t)(o >> 32)) << 32) | wave_or_u32((uint32_t)o);
  a = ((uint64_t)wave_and_u32((uint32_t)(a >> 32)) << 32) | wave_and_u32((uint32_t)a);
  const uint64_t diff = o ^ a;
  if (diff == 0) return 0;
  const int hb = 63 - __clzll(diff);
  return hb >= 7 ? hb - 7 : 0;
}

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


__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}

// Block-wide max / or of one value per thread; tmp holds blockDim.x/64 words of LDS.
__device__ uint32_t block_max_u32(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63;
  v = wave_max_u32(v);
  if (lane == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t r = wave_max_u32(lane < (int)(blockDim.x >> 6) ? tmp[lane] : 0u);
  __syncthreads();
  return r;
}
// Both at once (one barrier pair); tmp holds 32 words.
__device__ void block_max_or_u32(uint32_t* mx, uint32_t* ov, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const uint32_t m = wave_max_u32(*mx), o = wave_or_u32(*ov);
  if (lane == 0) { tmp[threadIdx.x >> 6] = m; tmp[16 + (threadIdx.x >> 6)] = o; }
  __syncthreads();
  *mx = wave_max_u32(lane < nw ? tmp[lane] : 0u);
  *ov = wave_or_u32(lane < nw ? tmp[16 + lane] : 0u);
  __syncthreads();
}
__device__ uint32_t block_or_u32(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63;
  v = wave_or_u32(v);
  if (lane == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t r = wave_or_u32(lane < (int)(blockDim.x >> 6) ? tmp[lane] : 0u);
  __syncthreads();
  return r;
}

// Bin holding the `need`-th best key of an LDS histogram (with BPT = NBINS /
// THREADS, thread t owns bins NBINS-1-BPT*t .. NBINS-BPT-BPT*t). Returns the number of keys counted in *total,
// the bin in ctl[0] and the count strictly above it in ctl[1] (ctl[0] = -1
// when total < need). All threads must call it.
// PACKED: two 16-bit counts per word (bin b in the half b & 1 of word b / 2).
template <int THREADS, bool PACKED = false>
__device__ void hist_kth_bin(const uint32_t* lhist, uint32_t need, uint32_t* scan_tmp, uint32_t* ctl,
                             uint32_t* total_out) {
  constexpr int BPT = NBINS / THREADS;
  uint32_t hv[BPT], local = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int bin = NBINS - 1 - (BPT * threadIdx.x + q);
    hv[q] = PACKED ? (lhist[bin >> 1] >> ((bin & 1) * 16)) & 0xFFFFu : lhist[bin];
    local += hv[q];
  }
  if (threadIdx.x == 0) { ctl[0] = 0xFFFFFFFFu; ctl[1] = 0; }
  uint32_t total;
  const uint32_t prefix = block_exclusive_scan(local, scan_tmp, &total);
  if (prefix < need && prefix + local >= need) {
    // the first of this thread's bins where the running count reaches `need`
    // (selects, not a loop with a break: no nest of saved execution masks)
    uint32_t cum = prefix, qf = BPT, cum_at = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const bool hit = qf == BPT && cum + hv[q] >= need;
      qf = hit ? (uint32_t)q : qf;
      cum_at = hit ? cum : cum_at;
      cum += hv[q];
    }
    ctl[0] = NBINS - 1 - (BPT * threadIdx.x + qf);
    ctl[1] = cum_at;
  }
  __syncthreads();
  *total_out = total;
}

// One tile of 16 slots x 16 heads: 4 MFMAs over the 128 channels (lane (n, g):
// slot n, channels 32g .. 32g+31); MODE 1 applies w_h * ReLU and sums the heads
// into the lanes of group 0. The score pass and the finish's recompute share
// it, so both give the same float32 scores.
template <int MODE>
__device__ __forceinline__ float score_tile_fn(const bf16x8_t (&qa)[4], const u32x4_t cw, uint32_t sbyte,
                                               const float* lw, int g) {
  const float scl = __uint_as_float(sbyte << 23);
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x8_t kb = dequant_mx_block8(cw[j], scl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], kb, acc, 0, 0, 0);
  }
  if (MODE == 0) return acc[0];          // head 0 is row 0, held by lanes 0..15
  const float4 wr = *(const float4*)&lw[4 * g];
  const float sc = wr.x * fmaxf(acc[0], 0.0f) + wr.y * fmaxf(acc[1], 0.0f) +
                   wr.z * fmaxf(acc[2], 0.0f) + wr.w * fmaxf(acc[3], 0.0f);
  return sum_lane_groups(sc);
}

// CAND: score the listed positions (Reindex) instead of every entry.
// SEL: SEL_NONE (scores only); SEL_THRESHOLD / SEL_DIRECT (also report the
//      local cutoff summary, and for SEL_DIRECT the candidates, that
//      finish_kernel turns into the threshold bin or the final top-K).
// MODE: 0 = dot product of head 0, 1 = sum_h w_h * ReLU(q_h . k).
// A workgroup streams SC_SPAN slots (SC_SUB selection chunks of SC_CHUNK);
// eight workgroups of four waves share a compute unit, each wave with
// SC_UNROLL tiles in flight.
template <bool CAND, int SEL, int MODE>
__global__ __launch_bounds__(SC_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void score_kernel(
    const uint8_t* __restrict__ ik, const uint8_t* __restrict__ iks,
    const int64_t* __restrict__ entry_offset, const int32_t* __restrict__ n_entries, int64_t max_n,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int Hi,
    const int32_t* __restrict__ cand, int cand_stride,
    float* __restrict__ scores, int64_t sstride, SelBufs sb, int K, int store_scores) {
  // histogram with 16-bit counts (two bins per word) + staged scores: 12 KiB,
  // so that eight workgroups fit one compute unit
  __shared__ uint32_t lbuf[NBINS / 2 + SC_SPAN];
  __shared__ uint32_t scan_tmp[SC_THREADS / 64 + 1];
  __shared__ uint32_t ctl[8];
  __shared__ __attribute__((aligned(16))) float lw[16];   // head weights
  __shared__ SelBufs sbs;   // the workspace views, parked in LDS while the keys stream (frees SGPRs)
  uint32_t* lhist = lbuf;
  float* lsc = (float*)(lbuf + NBINS / 2);
  auto hcount = [&](uint32_t bin) -> uint32_t { return (lhist[bin >> 1] >> ((bin & 1) * 16)) & 0xFFFFu; };

  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // independent loads first (the sequence's length and first row, the queries,
  // the head weights), so the keys are requested one round trip after the start
  const int32_t ne = n_entries[b];
  const int64_t row_base = entry_offset[b];
  asm volatile("" ::"s"(ne), "s"(row_base));   // both loads issued here, before any branch on them
  // A operand: q[head = n][channels 32g + 8j .. +7] for MFMA j
  bf16x8_t qa[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t v = {0, 0, 0, 0};
    if (n < Hi) v = *(const u32x4_t*)(q_idx + ((int64_t)b * Hi + n) * 128 + 32 * g + 8 * j);
    __builtin_memcpy(&qa[j], &v, 16);
  }
  // head weights of the output rows (lane group g takes heads 4g .. 4g+3), in
  // LDS and read per tile, which keeps the wave within 64 registers
  const float wv = tid < Hi ? (w ? w[(int64_t)b * Hi + tid] : 1.0f) : 0.0f;
  const int64_t n_pos = min((int64_t)ne, max_n);
  const int64_t nslots = CAND ? (int64_t)cand_stride : n_pos;
  const int64_t start = (int64_t)blockIdx.x * SC_SPAN;
  if (start >= nslots) return;
  if (CAND && n_pos <= 0) return;                  // no listed position can be valid
  const int end = (int)min((int64_t)SC_SPAN, nslots - start);   // slots of this workgroup
  // the sequence's rows: a uniform base plus a 32-bit byte offset per lane
  // (positions below 2^26, checked on the host), one address register per load
  const uint8_t* ikb = ik + row_base * 64;
  const uint8_t* iksb = iks + row_base * 4;
  const int32_t* crow = CAND ? cand + (int64_t)b * cand_stride + start : nullptr;
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

  if (SEL == SEL_THRESHOLD) {
    for (int i = tid; i < NBINS / 2; i += SC_THREADS) lhist[i] = 0;
  }
  if (SEL == SEL_THRESHOLD) {
    // select_kernel ORs into the bitmap words of this chunk: clear them here
    uint32_t* bm = sb.bitmap + (int64_t)b * sb.bm_stride;
    for (int64_t wd = start / 32 + tid; wd < (start + end + 31) / 32; wd += SC_THREADS) bm[wd] = 0;
  }
  if (tid < 16) lw[tid] = wv;
  if (SEL != SEL_NONE && tid == 0) sbs = sb;
  __syncthreads();

  // one tile = 16 slots x 16 heads: 4 MFMAs over the 128 channels; the head sum
  // goes to the lanes of group 0, which stage the score in LDS
  auto score_tile = [&](const u32x4_t cw, uint32_t sbyte) -> float {
    return score_tile_fn<MODE>(qa, cw, sbyte, lw, g);
  };
  // ---- per selection chunk (sub = 0 .. SC_SUB-1): store its scores, then the
  // local cutoff (every slot of a Full pass is a valid position). Chunk cix
  // reports into its own slot of the workspace (a header word and a list), so
  // no global atomics are needed. With two chunks per workgroup in direct
  // mode, the first chunk's tail runs in the middle of the stream, while the
  // second chunk's tiles are in flight.
  auto chunk_tail = [&](int sub) {
  const int soff = sub * SC_CHUNK;
  const int send = min(SC_CHUNK, end - soff);        // slots of this chunk
  if (send <= 0) return;
  __syncthreads();                                   // its scores are staged; the previous tail is done
  const float* lss = lsc + soff;
  const int64_t cix = (int64_t)blockIdx.x * SC_SUB + sub;
  // coalesced store of the chunk's scores (slots of invalid candidates hold 0)
  if (store_scores) {
    float* srow = scores + (int64_t)b * sstride + start + soff;
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
  const int64_t nwg = (n_pos + SC_CHUNK - 1) / SC_CHUNK;
  // local budget: a multiple of the chunk's expected share of the top-K plus a
  // margin, so that the highest cutoff over the workgroups still leaves at
  // least K keys of the sequence above it (the finish checks this)
  const int64_t share = ((int64_t)K * SC_CHUNK + n_pos - 1) / n_pos;
  int64_t budget64 = SEL == SEL_DIRECT ? 2 * share + 16 : 4 * share + 32;
  if (SEL == SEL_DIRECT) budget64 = min(budget64, max((int64_t)8, (int64_t)FIN_LDS_CANDS / nwg));
  const uint32_t budget = (uint32_t)min(budget64, (int64_t)send);
  uint64_t* hdr = sbl.hdr + (int64_t)b * sbl.hdr_stride + cix;
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
    uint32_t* pl = sbl.summ + (int64_t)b * sbl.summ_stride + cix * SUM_PAIRS;
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
  if (SEL == SEL_DIRECT) {
    // The cutoff: a 20-bit key prefix `fine` with at least `budget` keys of
    // the chunk at or above it. The keys within two octaves of the chunk's
    // largest prefix M go to a band histogram of 256 bins, 16 prefix units
    // each, counted down from M; spread over 256 bins the LDS atomics rarely
    // collide, unlike the 12-bit key bins, of which a chunk fills only a
    // handful. The bin where the running count reaches the budget gives the
    // cutoff. A chunk with fewer than `budget` keys in the band takes the
    // exact path instead (12-bit histogram, then the 256 20-bit sub-bins of
    // the cutoff bin). Thread t owns slots 4t .. 4t+3.
    constexpr uint32_t sh = 4;
    uint32_t* hb = lhist;                            // 256 words
    uint32_t keys[4], pmax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      keys[q] = i < send ? score_key(lss[i]) : 0u;
      if (i < send) pmax = max(pmax, keys[q] >> 12);
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
      if (4 * tid + q < send && d < 256u) atomicAdd(&hb[d], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t hv[4], sl = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { hv[j] = hb[4 * lane + j]; sl += hv[j]; }
      const uint32_t incl = wave_incl_sum(sl);
      uint32_t cum = incl - sl;
      if (cum < budget && incl >= budget) {
        uint32_t ds = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool hit = ds == 0xFFFFFFFFu && cum + hv[j] >= budget;
          ds = hit ? 4 * lane + j : ds;
          cum += hv[j];
        }
        ctl[4] = ds;
      }
      if (lane == 63 && incl < budget) ctl[4] = 0xFFFFFFFFu;   // too few keys within the octave
    }
    __syncthreads();
    const uint32_t ds = ctl[4];
    uint32_t fine;
    if (ds != 0xFFFFFFFFu) {
      // bin ds holds prefixes M - (ds << sh) - (2^sh - 1) .. M - (ds << sh)
      const uint32_t lo = ((ds + 1u) << sh) - 1u;
      fine = M >= lo ? M - lo : 0u;
    } else {
      // exact path: the 12-bit bin of the budget-th key, refined to 20 bits
      for (int i = tid; i < NBINS / 2; i += SC_THREADS) lhist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (4 * tid + q < send) {
          const uint32_t bin = keys[q] >> BIN_SHIFT;
          atomicAdd(&lhist[bin >> 1], 1u << ((bin & 1) * 16));
        }
      }
      __syncthreads();
      uint32_t cnt_all;
      hist_kth_bin<SC_THREADS, true>(lhist, budget, scan_tmp, ctl, &cnt_all);
      const uint32_t cbin = ctl[0], cabove = ctl[1];
      fine = 0;                                      // fewer keys than the budget: keep all
      if (cbin != 0xFFFFFFFFu) {
        uint32_t* h2 = lhist;                        // every read of the 4096 bins is done (256 words)
        h2[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * tid + q < send && (keys[q] >> BIN_SHIFT) == cbin) atomicAdd(&h2[(keys[q] >> 12) & 255u], 1u);
        __syncthreads();
        if (tid < 64) digit_kth(h2, budget - cabove, ctl + 4);
        __syncthreads();
        fine = (cbin << 8) | ctl[4];
      }
    }
    // candidates: every slot whose top 20 key bits are >= fine, in slot order
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) m |= ((4 * tid + q < send && (keys[q] >> 12) >= fine) ? 1u : 0u) << q;
    uint32_t tot;
    uint32_t off = block_exclusive_scan((uint32_t)__popc(m), scan_tmp, &tot);
    uint64_t* wc = sbl.wgc + (int64_t)b * sbl.wgc_stride + cix * CAND_CAP;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((m >> q) & 1u) {
        if (off < CAND_CAP) wc[off] = composite(keys[q], (uint32_t)(start + soff + 4 * tid + q));
        ++off;
      }
    }
    if (tid == 0) *hdr = ((uint64_t)fine << 32) | (tot > CAND_CAP ? 0x80000000u : tot);
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
    static_assert(SC_SUB <= 2 && NIT % SC_SUB == 0, "chunks end at stream iteration boundaries");
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (SC_SUB == 2 && SEL == SEL_DIRECT && it == NIT / 2) chunk_tail(0);   // the next tiles are in flight
      const int t0 = 16 * wave + it * 64 * SC_UNROLL;
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        const float sc = score_tile(codes[u], sbyte[u]);
        const int ls = t0 + 64 * u + n;
        if (g == 0 && ls < end) lsc[ls] = sc;
        const uint32_t p = (uint32_t)(start + min(ls + 64 * SC_UNROLL, end - 1));
        codes[u] = __builtin_nontemporal_load((const u32x4_t*)(ikb + (p * 64u + 16u * g)));
        sbyte[u] = iksb[p * 4u + (uint32_t)g];
      }
    }
  } else {
    // listed positions: SC_UNROLL tiles are loaded before any is used (invalid
    // slots read row 0 of the sequence and score 0)
    for (int t0 = 16 * wave; t0 < end; t0 += 64 * SC_UNROLL) {
      int pos[SC_UNROLL];
      bool ok[SC_UNROLL];
      int cv[SC_UNROLL];
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) cv[u] = crow[min(t0 + 64 * u + n, end - 1)];
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        ok[u] = (t0 + 64 * u + n < end) && cv[u] >= 0 && cv[u] < n_pos;
        pos[u] = ok[u] ? cv[u] : 0;
      }
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        codes[u] = __builtin_nontemporal_load((const u32x4_t*)(ikb + ((uint32_t)pos[u] * 64u + 16u * g)));
        sbyte[u] = iksb[(uint32_t)pos[u] * 4u + (uint32_t)g];
      }
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        const float sc = score_tile(codes[u], sbyte[u]);
        const int ls = t0 + 64 * u + n;
        if (g == 0 && ls < end) lsc[ls] = ok[u] ? sc : 0.0f;
      }
    }
  }
  if (SC_SUB == 1 || CAND || SEL != SEL_DIRECT) chunk_tail(0);   // (threshold mode: its tail needs the registers)
  if (SC_SUB == 2) chunk_tail(1);
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

// Ordered compaction over elements [0, n): pred(i) selects, emit(i, slot)
// receives the element's place among the selected ones. Every wave owns a
// contiguous range (a multiple of 64 elements) and ranks inside it with
// ballots, so only one exchange of wave totals is needed. Returns the number
// selected. All threads of the workgroup must call it.
template <typename Pred, typename Emit>
__device__ uint32_t ordered_compact(uint32_t n, Pred pred, Emit emit, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t span = (n + 64 * nw - 1) / (64 * nw) * 64;
  const uint32_t lo = min((uint32_t)wave * span, n), hi = min(lo + span, n);
  uint32_t cnt = 0;
  for (uint32_t i0 = lo; i0 < hi; i0 += 64) {
    const uint32_t i = i0 + lane;
    cnt += (uint32_t)__popcll(__ballot(i < hi && pred(i)));
  }
  if (lane == 0) tmp[wave] = cnt;
  __syncthreads();
  const uint32_t t = lane < nw ? tmp[lane] : 0u;
  const uint32_t ti = wave_incl_sum(t);
  uint32_t base = readlane_u32(ti - t, wave);
  const uint32_t total = readlane_u32(ti, nw - 1);
  __syncthreads();
  for (uint32_t i0 = lo; i0 < hi; i0 += 64) {
    const uint32_t i = i0 + lane;
    const bool p = i < hi && pred(i);
    const uint64_t m = __ballot(p);
    if (p) emit(i, base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull)));
    base += (uint32_t)__popcll(m);
  }
  return total;
}

// Direct top-K (K <= kDirectMaxK). The candidate lists hold, per workgroup,
// every key whose top 20 bits reach its refined cutoff, in position order, so
// their concatenation in workgroup order is in position order too; the ones
// at or above the highest cutoff are every key of the sequence there. While
// the lists are copied to LDS, their 20-bit prefixes (relative to that cutoff,
// the last bin holding everything 4095 or more above it) are histogrammed; the
// bin of the K-th best prefix follows, all keys above it are selected, and the
// few inside it are chosen on the full (key, position) composite: by ranking
// when the bin is small, else by radix select. Every thread owns a run of
// consecutive candidates, so one scan of the per-thread counts places the K
// positions in ascending order. When a list
// overflowed, the lists exceed LDS or fewer than K keys reach the highest
// cutoff, the same steps run on a histogram of every score of the sequence.
__global__ __launch_bounds__(FIN_THREADS) void finish_direct_kernel(
    const int32_t* __restrict__ n_entries, int64_t max_n, float* __restrict__ scores, int64_t sstride,
    SelBufs sb, int K, int32_t* __restrict__ out, int out_stride, ScoreSrc src, int rescore) {
  __shared__ uint64_t lc[FIN_LDS_CANDS];          // the candidate lists, concatenated
  __shared__ uint64_t sub[FIN_SUB_CAP];           // histogram, then the keys inside the threshold bin
  __shared__ uint32_t loff[FIN_MAX_WG + 1];       // list offsets of the workgroups
  __shared__ uint32_t h[512];
  __shared__ uint64_t red[32];
  __shared__ uint32_t scan_tmp[32];
  __shared__ uint32_t ctl[8];
  __shared__ uint64_t binl[FIN_RANK_MAX];          // keys of a small threshold bin
  __shared__ uint32_t bin_count;
  uint32_t* hist = (uint32_t*)sub;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int NWAVE = FIN_THREADS / 64;
  if (tid == 0) bin_count = 0;                     // first read after several barriers
  // the first header words, and the first 128 candidates of the four lists
  // this wave copies first (workgroups wave, wave + NWAVE, ...), are requested
  // before the sequence length and the list lengths are known
  const int64_t nw_max = (max_n + SC_CHUNK - 1) / SC_CHUNK;
  const uint64_t* hd = sb.hdr + (int64_t)b * sb.hdr_stride;
  const uint64_t h0 = tid < nw_max ? hd[tid] : 0ull;
  const uint64_t* wc = sb.wgc + (int64_t)b * sb.wgc_stride;
  const int nbk = (int)(sb.wgc_stride / CAND_CAP);   // list slots per sequence (>= 1)
  uint64_t v0[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int w = min(wave + s * NWAVE, nbk - 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) v0[s][u] = wc[(int64_t)w * CAND_CAP + lane + 64 * u];
  }
  // keeps the compiler from sinking these loads below the early return (their
  // latency then overlaps the sequence-length load)
  asm volatile("" ::: "memory");
  const int64_t n_pos = min((int64_t)n_entries[b], max_n);
  int32_t* ob = out + (int64_t)b * out_stride;
  if (n_pos <= K) {                       // every position is selected (or none exists)
    for (int j = tid; j < K; j += FIN_THREADS) ob[j] = j < n_pos ? j : -1;
    return;
  }
  for (int i = tid; i < NBINS; i += FIN_THREADS) hist[i] = 0;
  const int64_t nw = (n_pos + SC_CHUNK - 1) / SC_CHUNK;
  bool fast = false;
  uint32_t total = 0, cmax = 0;
  if (nw <= FIN_MAX_WG) {
    // list lengths -> offsets; thread t owns workgroups [w0, w1)
    const int per = (int)((nw + FIN_THREADS - 1) / FIN_THREADS);
    const int w0 = (int)min((int64_t)tid * per, nw), w1 = (int)min((int64_t)w0 + per, nw);
    uint32_t cnt = 0, ovf = 0;
    for (int w = w0; w < w1; ++w) {
      const uint64_t hv = (per == 1) ? h0 : hd[w];
      const uint32_t c = (uint32_t)hv & 0x7FFFFFFFu;
      ovf |= (uint32_t)hv >> 31;
      cmax = max(cmax, (uint32_t)(hv >> 32));
      loff[w] = c;
      cnt += c;
    }
    uint32_t run = block_exclusive_scan(cnt, scan_tmp, &total);
    for (int w = w0; w < w1; ++w) {
      const uint32_t c = loff[w];
      loff[w] = run;
      run += c;
    }
    if (tid == 0) loff[nw] = total;
    block_max_or_u32(&cmax, &ovf, scan_tmp);
    if (ovf == 0 && total <= (uint32_t)FIN_LDS_CANDS) {
      // copy the lists in workgroup order (wave v takes workgroups v, v + 16, ...,
      // eight independent loads per lane in flight) and histogram the prefixes
      auto take = [&](uint64_t c, uint32_t at) {
        lc[at] = c;
        const uint32_t p20 = (uint32_t)(c >> 44);
        if (p20 >= cmax) atomicAdd(&hist[min(p20 - cmax, (uint32_t)NBINS - 1)], 1u);
      };
      for (int w0 = wave; w0 < nw; w0 += 4 * NWAVE) {
        uint64_t v[4][2];
        uint32_t cn[4], of[4];
        int ws[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ws[s] = min(w0 + s * NWAVE, (int)nw - 1);
          cn[s] = (w0 + s * NWAVE < nw) ? loff[ws[s] + 1] - loff[ws[s]] : 0u;
          of[s] = loff[ws[s]];
          if (w0 == wave) {                 // the first round: already requested
#pragma unroll
            for (int u = 0; u < 2; ++u) v[s][u] = v0[s][u];
          } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) v[s][u] = wc[(int64_t)ws[s] * CAND_CAP + lane + 64 * u];
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if ((uint32_t)(lane + 64 * u) < cn[s]) take(v[s][u], of[s] + lane + 64 * u);
          for (uint32_t j = 128 + lane; j < cn[s]; j += 64) take(wc[(int64_t)ws[s] * CAND_CAP + j], of[s] + j);
        }
      }
      __syncthreads();
      uint32_t tot;
      hist_kth_bin<FIN_THREADS>(hist, (uint32_t)K, scan_tmp, ctl, &tot);
      fast = ctl[0] != 0xFFFFFFFFu;       // at least K keys reach the highest cutoff
    }
  }
  if (fast) {
    // Keys above the threshold bin are selected; inside it (20-bit prefixes
    // lo20 .. hi20) the `need` largest. Thread t owns the run of candidates
    // [t R, t R + R), so one scan of the per-thread counts orders the output.
    const uint32_t T = ctl[0], above = ctl[1], in_bin = hist[T];
    const uint32_t need = (uint32_t)K - above;      // 1 .. in_bin
    const uint32_t lo20 = cmax + T;
    const uint32_t hi20 = T == NBINS - 1 ? 0xFFFFFu : cmax + T;
    const uint32_t R = (total + FIN_THREADS - 1) / FIN_THREADS;   // <= FIN_RUN
    const uint32_t i0 = min((uint32_t)tid * R, total), i1 = min(i0 + R, total);
    uint64_t cv[FIN_RUN];                            // this thread's run, read once
#pragma unroll
    for (int q = 0; q < FIN_RUN; ++q) cv[q] = i0 + q < i1 ? lc[i0 + q] : 0ull;
    auto in_run = [&](int q) { return i0 + (uint32_t)q < i1; };
    auto is_above = [&](uint64_t c) { return (uint32_t)(c >> 44) > hi20; };
    auto is_in_bin = [&](uint64_t c) {
      const uint32_t p20 = (uint32_t)(c >> 44);
      return p20 >= lo20 && p20 <= hi20;
    };
    const bool split = need < in_bin;                // else every in-bin key is selected
    const bool small = in_bin <= (uint32_t)FIN_RANK_MAX;
    uint64_t prefix = 0, mask = 0;                   // large bins: in-bin keys with (c & mask) >= prefix
    uint64_t* dst = binl;
    if (split) {
      if (!small) {
        __syncthreads();                             // hist reads done before sub is reused
        dst = in_bin <= (uint32_t)FIN_SUB_CAP ? sub : sb.gscr + (int64_t)b * sb.gscr_stride;
      }
#pragma unroll
      for (int q = 0; q < FIN_RUN; ++q)
        if (in_run(q) && is_in_bin(cv[q])) {
          const uint32_t at = atomicAdd(&bin_count, 1u);
          if (at < in_bin) dst[at] = cv[q];
        }
      if (dst != sub && dst != binl) __threadfence_block();   // this workgroup reads its global copy back
      __syncthreads();
      if (!small) {
        const int top = radix_top_shift(dst, in_bin, red);
        radix_select_u64(dst, in_bin, need, top, h, ctl, &prefix, &mask);
      }
    }
    // small bins: keys are distinct (they carry the position), so a key is
    // selected when fewer than `need` keys of the bin are larger
    auto selected = [&](uint64_t c) {
      if (is_above(c)) return true;
      if (!is_in_bin(c)) return false;
      if (!split) return true;
      if (!small) return (c & mask) >= prefix;
      uint32_t larger = 0;
      for (uint32_t j = 0; j < in_bin; ++j) larger += binl[j] > c ? 1u : 0u;
      return larger < need;
    };
    uint32_t cnt = 0, selm = 0;
#pragma unroll
    for (int q = 0; q < FIN_RUN; ++q)
      if (in_run(q) && selected(cv[q])) { ++cnt; selm |= 1u << q; }
    uint32_t nsel;
    uint32_t at = block_exclusive_scan(cnt, scan_tmp, &nsel);
#pragma unroll
    for (int q = 0; q < FIN_RUN; ++q)
      if ((selm >> q) & 1u) {
        if (at < (uint32_t)K) ob[at] = (int32_t)(0xFFFFFFFFu - (uint32_t)cv[q]);
        ++at;
      }
    for (uint32_t j = nsel + tid; j < (uint32_t)K; j += FIN_THREADS) ob[j] = -1;
    return;
  }
  // Fallback: the same steps on a histogram of every score of the sequence
  // (12-bit key bins); the threshold bin is the range of the 256 20-bit
  // prefixes under bin T. When the score pass did not store the scores, this
  // workgroup recomputes the sequence's first.
  float* sall = scores + (int64_t)b * sstride;
  if (rescore) {
    __shared__ __attribute__((aligned(16))) float lwf[16];
    const int n = lane & 15, g = lane >> 4;
    const int64_t row_base = src.entry_offset[b];
    const uint8_t* ikb = src.ik + row_base * 64;
    const uint8_t* iksb = src.iks + row_base * 4;
    bf16x8_t qa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t v = {0, 0, 0, 0};
      if (n < src.Hi) v = *(const u32x4_t*)(src.q_idx + ((int64_t)b * src.Hi + n) * 128 + 32 * g + 8 * j);
      __builtin_memcpy(&qa[j], &v, 16);
    }
    if (tid < 16) lwf[tid] = tid < src.Hi ? (src.w ? src.w[(int64_t)b * src.Hi + tid] : 1.0f) : 0.0f;
    __syncthreads();
    for (int64_t t0 = 16 * wave; t0 < n_pos; t0 += 16 * (FIN_THREADS / 64)) {
      const uint32_t p = (uint32_t)min(t0 + n, n_pos - 1);
      const u32x4_t cw = *(const u32x4_t*)(ikb + ((uint64_t)p * 64u + 16u * g));
      const uint32_t sbyte = iksb[(uint64_t)p * 4u + (uint32_t)g];
      const float sc = src.mode == 0 ? score_tile_fn<0>(qa, cw, sbyte, lwf, g) : score_tile_fn<1>(qa, cw, sbyte, lwf, g);
      if (g == 0 && t0 + n < n_pos) sall[t0 + n] = sc;
    }
    __threadfence_block();                         // this workgroup reads them back
  }
  __syncthreads();
  for (int i = tid; i < NBINS; i += FIN_THREADS) hist[i] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n_pos; i += FIN_THREADS) atomicAdd(&hist[score_key(sall[i]) >> BIN_SHIFT], 1u);
  __syncthreads();
  {
    uint32_t tot;
    hist_kth_bin<FIN_THREADS>(hist, (uint32_t)K, scan_tmp, ctl, &tot);   // defined: n_pos > K
  }
  const uint32_t T = ctl[0], above = ctl[1], in_bin = hist[T];
  const uint32_t need = (uint32_t)K - above;      // 1 .. in_bin
  const uint32_t lo20 = T << 8;
  const uint32_t hi20 = (T << 8) | 255u;
  auto elem = [&](uint32_t i) -> uint64_t { return composite(score_key(sall[i]), i); };
  const uint32_t n_src = (uint32_t)n_pos;
  uint64_t prefix = 0, mask = 0;
  if (need < in_bin) {
    // the threshold bin is split: its keys (unordered) -> radix select
    __syncthreads();                               // hist reads done before sub is reused
    uint64_t* dst = in_bin <= (uint32_t)FIN_SUB_CAP ? sub : sb.gscr + (int64_t)b * sb.gscr_stride;
    if (tid == 0) ctl[6] = 0;
    __syncthreads();
    for (uint32_t i0 = 0; i0 < n_src; i0 += FIN_THREADS) {
      const uint32_t i = i0 + tid;
      const uint64_t c = i < n_src ? elem(i) : 0ull;
      const uint32_t p20 = (uint32_t)(c >> 44);
      const bool t = i < n_src && p20 >= lo20 && p20 <= hi20;
      const uint32_t at = wave_append(t, &ctl[6]);
      if (t && at < in_bin) dst[at] = c;
    }
    if (dst != sub) __threadfence_block();         // this workgroup reads its global copy back
    __syncthreads();
    const int top = radix_top_shift(dst, in_bin, red);
    radix_select_u64(dst, in_bin, need, top, h, ctl, &prefix, &mask);
  }
  // the K best in position order: above the threshold bin, or inside it and
  // radix-selected
  const uint32_t nsel = ordered_compact(
      n_src,
      [&](uint32_t i) {
        const uint64_t c = elem(i);
        const uint32_t p20 = (uint32_t)(c >> 44);
        return p20 > hi20 || (p20 >= lo20 && p20 <= hi20 && (c & mask) >= prefix);
      },
      [&](uint32_t i, uint32_t at) {
        if (at < (uint32_t)K) ob[at] = (int32_t)i;
      },
      scan_tmp);
  for (uint32_t j = nsel + tid; j < (uint32_t)K; j += FIN_THREADS) ob[j] = -1;
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
        const uint32_t rank = (uint32_t)__popcll(bc & ((1ull << lane) - 1ull));
        cb[basei + rank] = composite(key, (uint32_t)i);
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
__global__ __launch_bounds__(SMALL_THREADS) void select_small_kernel(
    const float* __restrict__ scores, int64_t sstride, const int32_t* __restrict__ slot_pos,
    int pstride, int score_by_pos, const int32_t* __restrict__ n_entries, int64_t max_n, int K,
    int32_t* __restrict__ out, int out_stride) {
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
  const int lane = threadIdx.x & 63;

  for (int i = threadIdx.x; i < SMALL_MAX / 32; i += SMALL_THREADS) { valid[i] = 0; selbm[i] = 0; }
  __syncthreads();
  uint32_t nvalid = 0;
  for (int base = (threadIdx.x & ~63); base < nslots; base += SMALL_THREADS) {
    const int i = base + lane;
    bool ok = false;
    uint32_t key = 0;
    if (i < nslots) {
      int64_t pos = sp ? (int64_t)sp[i] : (int64_t)i;
      ok = pos >= 0 && pos < n_pos;
      if (ok) key = score_key(sb[score_by_pos ? pos : (int64_t)i]);
      keys[i] = key;
    }
    const uint64_t bal = __ballot(ok);
    if (lane == 0) valid[base >> 5] = (uint32_t)bal;
    if (lane == 32) valid[(base >> 5) + 1] = (uint32_t)(bal >> 32);
    nvalid += ok ? 1u : 0u;
  }
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

// ---------------------------------------------------------------- launchers
hipError_t launch_score(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                        const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                        const float* w, int Hi, int mode, const int32_t* cand, int cand_stride,
                        float* scores, int64_t sstride, const SelBufs& sb, int sel, int K,
                        bool store_scores, hipStream_t stream) {
  const bool store = store_scores || cand || sel != SEL_DIRECT;
  const int64_t nslots = cand ? cand_stride : max_n;
  if (nslots <= 0) return hipSuccess;
  const int64_t nx = (nslots + SC_SPAN - 1) / SC_SPAN;
  dim3 grid((unsigned)nx, (unsigned)B), block(SC_THREADS);
#define CSA2_SCORE_LAUNCH(C, S, Mo)                                                              \
  hipLaunchKernelGGL((score_kernel<C, S, Mo>), grid, block, 0, stream, ik, iks, entry_offset,   \
                     n_entries, max_n, q_idx, w, Hi, cand, cand_stride, scores, sstride, sb, K,  \
                     (int)store)
  if (cand) {
    if (mode == 0) CSA2_SCORE_LAUNCH(true, SEL_NONE, 0); else CSA2_SCORE_LAUNCH(true, SEL_NONE, 1);
  } else if (sel == SEL_THRESHOLD) {
    if (mode == 0) CSA2_SCORE_LAUNCH(false, SEL_THRESHOLD, 0); else CSA2_SCORE_LAUNCH(false, SEL_THRESHOLD, 1);
  } else if (sel == SEL_DIRECT) {
    if (mode == 0) CSA2_SCORE_LAUNCH(false, SEL_DIRECT, 0); else CSA2_SCORE_LAUNCH(false, SEL_DIRECT, 1);
  } else {
    if (mode == 0) CSA2_SCORE_LAUNCH(false, SEL_NONE, 0); else CSA2_SCORE_LAUNCH(false, SEL_NONE, 1);
  }
#undef CSA2_SCORE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_finish(int sel, const int32_t* n_entries, int B, int64_t max_n, float* scores,
                         int64_t sstride, const SelBufs& sb, int K, int32_t* out, int out_stride,
                         const ScoreSrc* src, hipStream_t stream) {
  if (sel == SEL_DIRECT)
    hipLaunchKernelGGL(finish_direct_kernel, dim3((unsigned)B), dim3(FIN_THREADS), 0, stream, n_entries, max_n,
                       scores, sstride, sb, K, out, out_stride, src ? *src : ScoreSrc{}, src ? 1 : 0);
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
