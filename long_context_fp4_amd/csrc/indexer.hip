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
//                one scale byte per lane), dequantizes them in registers with
//                the gfx950 scaled FP4->bf16 conversion (exact: an E2M1 value
//                times a power of two fits bf16), and contracts 16 entries x 16
//                heads x 32 channels per v_mfma_f32_16x16x32_bf16. The head sum
//                is a 4-term in-lane sum plus two cross-lane steps. Each
//                workgroup also builds a 4096-bin LDS histogram of its score
//                keys and adds it into a per-sequence histogram; the last
//                workgroup of a sequence to finish finds the bin that holds the
//                K-th best key.
// select_kernel  (long sequences) marks every position whose key lies above
//                that bin in a per-sequence bitmap and appends the ones inside
//                it as (key, position) candidates; the last workgroup of the
//                sequence radix-selects the missing ones among the candidates,
//                then compacts the bitmap into ascending positions.
// select_small_kernel  one workgroup per sequence for at most 16384 slots
//                (the pool, a Reindex candidate list or a short sequence):
//                keys in LDS, 8-bit radix select on (key, slot), bitmap
//                compaction in slot order.
// The per-sequence control block (state + histogram, at a fixed place in the
// workspace) is left zero by the last workgroups; bitmap words are cleared by
// the score pass before use.
#include "device.h"
#include "kernels.h"

namespace csa2 {

constexpr int SC_THREADS = 256;
constexpr int SC_CHUNK = 1024;      // slots per score workgroup
constexpr int SC_UNROLL = 4;        // tiles in flight per wave
constexpr int NBINS = 4096;         // histogram over the top 12 bits of the key
constexpr int BIN_SHIFT = 20;
constexpr int SEL_THREADS = 256;
constexpr int SEL_CHUNK = 4096;     // slots per select workgroup
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_MAX = 16384;

// ---------------------------------------------------------------- block scan
// Exclusive prefix sum over the workgroup (blockDim.x multiple of 64); returns
// the total in *total. `tmp` holds at least blockDim.x/64 + 1 words of LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < nw ? tmp[lane] : 0u, s = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      uint32_t y = __shfl_up(s, d, 64);
      if (lane >= d) s += y;
    }
    if (lane < nw) tmp[lane] = s - t;
    if (lane == nw - 1) tmp[nw] = s;
  }
  __syncthreads();
  uint32_t r = tmp[wave] + x - v;
  *total = tmp[nw];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- score kernel
__device__ __forceinline__ bf16x8_t dequant_mx_block8(uint32_t dw, float scale) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 0);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 1);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 2);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 3);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__global__ __launch_bounds__(SC_THREADS) void score_kernel(
    const uint8_t* __restrict__ ik, const uint8_t* __restrict__ iks,
    const int64_t* __restrict__ entry_offset, const int32_t* __restrict__ n_entries, int64_t max_n,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int Hi, int mode,
    const int32_t* __restrict__ cand, int cand_stride,
    float* __restrict__ scores, int64_t sstride,
    uint8_t* __restrict__ ctrl, uint32_t* __restrict__ bitmap, int64_t bm_stride, int K) {
  __shared__ uint32_t lhist[NBINS];
  __shared__ uint32_t scan_tmp[SC_THREADS / 64 + 1];
  __shared__ int s_last;

  const int b = blockIdx.y;
  const int64_t n_pos = min((int64_t)n_entries[b], max_n);
  const int64_t nslots = cand ? (int64_t)cand_stride : n_pos;
  const int64_t start = (int64_t)blockIdx.x * SC_CHUNK;
  if (start >= nslots) return;
  const int64_t end = min(start + (int64_t)SC_CHUNK, nslots);
  const bool do_hist = ctrl != nullptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  if (do_hist) {
    for (int i = tid; i < NBINS; i += SC_THREADS) lhist[i] = 0;
    // the select pass ORs into the bitmap words of this chunk: clear them here
    uint32_t* bm = bitmap + (int64_t)b * bm_stride;
    for (int64_t wd = start / 32 + tid; wd < (end + 31) / 32; wd += SC_THREADS) bm[wd] = 0;
  }

  // A operand: q[head = n][channels 32g + 8j .. +7] for MFMA j
  bf16x8_t qa[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t v = {0, 0, 0, 0};
    if (n < Hi) v = *(const u32x4_t*)(q_idx + ((int64_t)b * Hi + n) * 128 + 32 * g + 8 * j);
    __builtin_memcpy(&qa[j], &v, 16);
  }
  // head weights of this lane's output rows (heads 4g + i)
  float wr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    wr[i] = hh < Hi ? (w ? w[(int64_t)b * Hi + hh] : 1.0f) : 0.0f;
  }
  const int64_t row_base = entry_offset[b];
  float* srow = scores + (int64_t)b * sstride;
  if (do_hist) __syncthreads();

  for (int64_t t0 = start + 16 * wave; t0 < end; t0 += 16 * 4 * SC_UNROLL) {
    u32x4_t codes[SC_UNROLL];
    float scl[SC_UNROLL];
    bool ok[SC_UNROLL];
    int64_t slot[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      slot[u] = t0 + 64 * u + n;
      const bool in = slot[u] < end;
      int64_t pos = slot[u];
      if (cand) pos = in ? (int64_t)cand[(int64_t)b * cand_stride + slot[u]] : -1;
      ok[u] = in && pos >= 0 && pos < n_pos;
      codes[u] = u32x4_t{0, 0, 0, 0};
      scl[u] = 0.0f;
      if (ok[u]) {
        const int64_t row = row_base + pos;
        codes[u] = __builtin_nontemporal_load((const u32x4_t*)(ik + row * 64 + 16 * g));
        scl[u] = __uint_as_float((uint32_t)iks[row * 4 + g] << 23);
      }
    }
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t kb = dequant_mx_block8(codes[u][j], scl[u]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], kb, acc, 0, 0, 0);
      }
      float s;
      if (mode == 0) {
        s = acc[0];                       // head 0 is row 0, held by lanes 0..15
      } else {
        s = wr[0] * fmaxf(acc[0], 0.0f) + wr[1] * fmaxf(acc[1], 0.0f) +
            wr[2] * fmaxf(acc[2], 0.0f) + wr[3] * fmaxf(acc[3], 0.0f);
        s += shfl_xor_f(s, 16);
        s += shfl_xor_f(s, 32);
      }
      if (g == 0 && ok[u]) {
        srow[slot[u]] = s;
        if (do_hist) atomicAdd(&lhist[score_key(s) >> BIN_SHIFT], 1u);
      }
    }
  }
  if (!do_hist) return;

  __syncthreads();
  SelState* st = ctrl_state(ctrl, b);
  uint32_t* gh = ctrl_hist(ctrl, b);
  for (int i = tid; i < NBINS; i += SC_THREADS) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&gh[i], v);
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t nblk = (uint32_t)((nslots + SC_CHUNK - 1) / SC_CHUNK);
    s_last = atomicAdd(&st->done_score, 1u) == nblk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // last workgroup of sequence b: find the bin holding the K-th best key.
  // Thread t owns bins NBINS-1-16t down to NBINS-16-16t (best bins first).
  uint32_t hv[16], local = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int bin = NBINS - 1 - (16 * tid + q);
    hv[q] = __hip_atomic_load(&gh[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    local += hv[q];
    gh[bin] = 0;
  }
  uint32_t total;
  const uint32_t prefix = block_exclusive_scan(local, scan_tmp, &total);
  if (total <= (uint32_t)K) {
    if (tid == 0) { st->thr_bin = -1; st->above = 0; }
  } else if (prefix < (uint32_t)K && prefix + local >= (uint32_t)K) {
    uint32_t cum = prefix;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (cum + hv[q] >= (uint32_t)K) {
        st->thr_bin = NBINS - 1 - (16 * tid + q);
        st->above = cum;
        break;
      }
      cum += hv[q];
    }
  }
  if (tid == 0) st->done_score = 0;
}

// ---------------------------------------------------------------- radix select
// Among n distinct 64-bit composites at `v` (global memory written by other
// workgroups of the same launch, read through agent-scope atomic loads),
// find the `need` largest (0 < need < n). On return every composite c with
// (c >> *shift_out) >= (*prefix_out >> *shift_out) is selected, and exactly
// `need` composites qualify. All threads of the workgroup must call it.
__device__ void radix_select_u64(const uint64_t* v, uint32_t n, uint32_t need, int top_shift,
                                 uint32_t* h, uint32_t* ctl, uint64_t* prefix_out, int* shift_out) {
  uint64_t prefix = 0, pmask = 0;
  int shift = top_shift;
  for (;;) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t c = __hip_atomic_load(v + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((c & pmask) == prefix) atomicAdd(&h[(uint32_t)(c >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits 255-4l .. 252-4l (best digits first)
      const int l = threadIdx.x;
      uint32_t c4[4], loc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c4[q] = h[255 - 4 * l - q]; loc += c4[q]; }
      uint32_t inc = loc;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(inc, d, 64);
        if (l >= d) inc += y;
      }
      const uint32_t pre = inc - loc;
      if (pre < need && pre + loc >= need) {
        uint32_t cum = pre;
        for (int q = 0; q < 4; ++q) {
          if (cum + c4[q] >= need) {
            ctl[0] = 255 - 4 * l - q;   // digit
            ctl[1] = cum;               // count strictly above this digit
            ctl[2] = c4[q];             // count with this digit
            break;
          }
          cum += c4[q];
        }
      }
    }
    __syncthreads();
    const uint32_t d = ctl[0], above = ctl[1], cnt = ctl[2];
    __syncthreads();
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)255 << shift;
    need -= above;
    if (cnt == need || shift == 0) break;
    shift -= 8;
  }
  *prefix_out = prefix;
  *shift_out = shift;
}

// Ascending compaction of a bitmap of nbits bits into out[0..cnt), -1 padding up to K.
// kGlobal: the bitmap lives in global memory and was filled by other workgroups
// of the same launch; it is read through agent-scope atomic loads.
template <bool kGlobal>
__device__ void compact_bitmap(uint32_t* bm, int64_t nbits, const int32_t* slot_pos, int K,
                               int32_t* out, uint32_t* scan_tmp) {
  const int64_t nwords = (nbits + 31) / 32;
  const int nt = blockDim.x;
  const int64_t per = (nwords + nt - 1) / nt;
  const int64_t w0 = min((int64_t)threadIdx.x * per, nwords), w1 = min(w0 + per, nwords);
  uint32_t cnt = 0;
  auto rd = [&](int64_t i) -> uint32_t {
    if (kGlobal) return __hip_atomic_load(bm + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return bm[i];
  };
  for (int64_t i = w0; i < w1; ++i) cnt += __popc(rd(i));
  uint32_t total;
  uint32_t off = block_exclusive_scan(cnt, scan_tmp, &total);
  for (int64_t i = w0; i < w1; ++i) {
    uint32_t word = rd(i);
    while (word) {
      const int bit = __ffs(word) - 1;
      word &= word - 1;
      const int64_t slot = i * 32 + bit;
      if (off < (uint32_t)K) out[off] = slot_pos ? slot_pos[slot] : (int32_t)slot;
      ++off;
    }
  }
  for (int64_t j = (int64_t)total + threadIdx.x; j < K; j += nt) out[j] = -1;
}

// ---------------------------------------------------------------- select (long)
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t sstride, const int32_t* __restrict__ n_entries,
    int64_t max_n, uint8_t* __restrict__ ctrl, uint32_t* __restrict__ bitmap, int64_t bm_stride,
    uint64_t* __restrict__ cbuf, int64_t cb_stride, int K, int32_t* __restrict__ out, int out_stride) {
  __shared__ uint32_t h[256];
  __shared__ uint32_t ctl[4];
  __shared__ uint32_t scan_tmp[SEL_THREADS / 64 + 1];
  __shared__ int s_last;

  const int b = blockIdx.y;
  const int64_t nb = min((int64_t)n_entries[b], max_n);
  int32_t* ob = out + (int64_t)b * out_stride;
  if (nb <= 0) {
    if (blockIdx.x == 0)
      for (int j = threadIdx.x; j < K; j += SEL_THREADS) ob[j] = -1;
    return;
  }
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
      basei = __shfl(basei, 0, 64);
      if (cnd) {
        const uint32_t rank = (uint32_t)__popcll(bc & ((1ull << lane) - 1ull));
        cb[basei + rank] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t nblk = (uint32_t)((nb + SEL_CHUNK - 1) / SEL_CHUNK);
    s_last = atomicAdd(&st->done_select, 1u) == nblk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // the candidates are a subset of the sequence's nb slots: clamp defensively
  const uint32_t ncand = min(__hip_atomic_load(&st->ncand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                             (uint32_t)nb);
  const uint32_t above = st->above;
  const uint32_t need = (thr >= 0 && (uint32_t)K > above) ? (uint32_t)K - above : 0u;
  if (need > 0) {
    if (need >= ncand) {
      for (uint32_t i = threadIdx.x; i < ncand; i += SEL_THREADS) {
        const uint64_t c = __hip_atomic_load(cb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t pos = 0xFFFFFFFFu - (uint32_t)c;
        atomicOr(&bm[pos >> 5], 1u << (pos & 31));
      }
    } else {
      uint64_t prefix;
      int shift;
      radix_select_u64(cb, ncand, need, 56, h, ctl, &prefix, &shift);
      for (uint32_t i = threadIdx.x; i < ncand; i += SEL_THREADS) {
        const uint64_t c = __hip_atomic_load(cb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((c >> shift) >= (prefix >> shift)) {
          const uint32_t pos = 0xFFFFFFFFu - (uint32_t)c;
          atomicOr(&bm[pos >> 5], 1u << (pos & 31));
        }
      }
    }
  }
  __threadfence();
  __syncthreads();
  compact_bitmap<true>(bm, nb, nullptr, K, ob, scan_tmp);
  if (threadIdx.x == 0) {
    st->done_select = 0;
    st->ncand = 0;
    st->thr_bin = 0;
    st->above = 0;
  }
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
      if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        uint32_t c4[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c4[q] = h[255 - 4 * l - q]; loc += c4[q]; }
        uint32_t inc = loc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          uint32_t y = __shfl_up(inc, d, 64);
          if (l >= d) inc += y;
        }
        const uint32_t pre = inc - loc;
        if (pre < need && pre + loc >= need) {
          uint32_t cum = pre;
          for (int q = 0; q < 4; ++q) {
            if (cum + c4[q] >= need) { ctl[0] = 255 - 4 * l - q; ctl[1] = cum; ctl[2] = c4[q]; break; }
            cum += c4[q];
          }
        }
      }
      __syncthreads();
      const uint32_t d = ctl[0], above = ctl[1], cnt = ctl[2];
      __syncthreads();
      prefix |= (uint64_t)d << shift;
      pmask |= (uint64_t)255 << shift;
      need -= above;
      if (cnt == need || shift == 0) break;
      shift -= 8;
    }
    for (int i = threadIdx.x; i < nslots; i += SMALL_THREADS) {
      if (!((valid[i >> 5] >> (i & 31)) & 1u)) continue;
      const uint64_t c = ((uint64_t)keys[i] << 14) | (uint64_t)(SMALL_MAX - 1 - i);
      if ((c >> shift) >= (prefix >> shift)) atomicOr(&selbm[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  compact_bitmap<false>(selbm, nslots, sp, K, ob, scan_tmp);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_score(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                        const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                        const float* w, int Hi, int mode, const int32_t* cand, int cand_stride,
                        float* scores, int64_t sstride, uint8_t* ctrl, uint32_t* bitmap,
                        int64_t bm_stride, int K, hipStream_t stream) {
  const int64_t nslots = cand ? cand_stride : max_n;
  if (nslots <= 0) return hipSuccess;
  dim3 grid((unsigned)((nslots + SC_CHUNK - 1) / SC_CHUNK), (unsigned)B), block(SC_THREADS);
  hipLaunchKernelGGL(score_kernel, grid, block, 0, stream, ik, iks, entry_offset, n_entries, max_n,
                     q_idx, w, Hi, mode, cand, cand_stride, scores, sstride, ctrl, bitmap, bm_stride, K);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t sstride, const int32_t* n_entries, int B,
                         int64_t max_n, uint8_t* ctrl, uint32_t* bitmap, int64_t bm_stride,
                         uint64_t* cbuf, int64_t cb_stride, int K, int32_t* out, int out_stride,
                         hipStream_t stream) {
  const int64_t nx = max_n > 0 ? (max_n + SEL_CHUNK - 1) / SEL_CHUNK : 1;
  dim3 grid((unsigned)nx, (unsigned)B), block(SEL_THREADS);
  hipLaunchKernelGGL(select_kernel, grid, block, 0, stream, scores, sstride, n_entries, max_n, ctrl,
                     bitmap, bm_stride, cbuf, cb_stride, K, out, out_stride);
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
