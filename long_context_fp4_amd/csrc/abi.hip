// Host side of the C ABI declared in include/csa2fp4.h: argument validation
// (before any HIP call), workspace layout and kernel launches.
#include "csa2fp4.h"
#include "kernels.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <algorithm>
#include <atomic>
#include <mutex>

static_assert(CSA2_SCORE_QMX8 == csa2::kScoreQmx8, "score-mode flag differs between the header and the kernels");

namespace {

thread_local char g_err[512] = "";
// one-shot events recorded around the next scoring launch of this thread
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return CSA2_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Indexer workspace layout, all regions 256-byte aligned. No region holds
// state between calls (every kernel writes what it reads), so a workspace needs
// no initialisation and can be reused by calls of any kind and size.
struct IndexerWs {
  size_t ctrl, bitmap, cand, scores, hdr, summ, wgc, gscr, hdrp, wgcp, psync, pxh, pxk, pxn, pxc, total;
  int64_t slots, bm_words, nblk, gscr_stride;
  int pool_parts_max;   // workgroups per sequence the pool exchange is sized for
};

// Most workgroups per sequence a split pool finish may use for B sequences.
int pool_parts_max(int B) {
  const int p = csa2::kPoolPartBudget / (B > 0 ? B : 1);
  return p < 1 ? 1 : (p > csa2::kPoolMaxParts ? csa2::kPoolMaxParts : p);
}

IndexerWs indexer_layout(int B, int64_t max_n, int k, int pool_k, int cand_stride) {
  IndexerWs L;
  L.slots = max_n > (int64_t)cand_stride ? max_n : (int64_t)cand_stride;
  if (L.slots < 1) L.slots = 1;
  L.bm_words = (L.slots + 31) / 32;
  L.nblk = (L.slots + csa2::kScoreChunk - 1) / csa2::kScoreChunk;
  // (a candidate list's direct pass reports per chunk of kCandChunk slots)
  const int64_t cblk = ((int64_t)cand_stride + csa2::kCandChunk - 1) / csa2::kCandChunk;
  if (cblk > L.nblk) L.nblk = cblk;
  const bool thr = k > csa2::kDirectMaxK;          // the threshold path's regions
  const bool pl = pool_k > 0;                      // the pool lists
  size_t off = 0;
  L.ctrl = off;   off = round_up(off + (size_t)B * csa2::kCtrlStride, 256);
  L.bitmap = off; off = round_up(off + (thr ? (size_t)B * L.bm_words * 4 : 0), 256);
  L.cand = off;   off = round_up(off + (thr ? (size_t)B * L.slots * 8 : 0), 256);
  L.scores = off; off = round_up(off + (size_t)B * L.slots * 4, 256);
  L.hdr = off;    off = round_up(off + (size_t)B * L.nblk * 8, 256);
  L.summ = off;   off = round_up(off + (thr ? (size_t)B * L.nblk * csa2::kSumWords * 4 : 0), 256);
  L.wgc = off;    off = round_up(off + (size_t)B * L.nblk * csa2::kCandCap * 8, 256);
  L.gscr_stride = L.slots > L.nblk * csa2::kCandCap ? L.slots : L.nblk * csa2::kCandCap;
  L.gscr = off;   off = round_up(off + (size_t)B * L.gscr_stride * 8, 256);
  L.hdrp = off;   off = round_up(off + (pl ? (size_t)B * L.nblk * 8 : 0), 256);
  L.wgcp = off;   off = round_up(off + (pl ? (size_t)B * L.nblk * csa2::kPoolCap * 8 : 0), 256);
  // a pool finish split over several workgroups per sequence: arrival
  // counters, per-part histograms and threshold-bin keys, per-chunk counts
  L.pool_parts_max = pl ? pool_parts_max(B) : 1;
  const size_t xp = L.pool_parts_max > 1 ? (size_t)B * L.pool_parts_max : 0;
  L.psync = off;  off = round_up(off + (pl ? (size_t)B * 16 : 0), 256);
  L.pxh = off;    off = round_up(off + xp * csa2::kPoolXBins * 4, 256);
  L.pxk = off;    off = round_up(off + xp * csa2::kPoolXKeys * 8, 256);
  L.pxn = off;    off = round_up(off + xp * 4, 256);
  L.pxc = off;    off = round_up(off + (xp ? (size_t)B * L.nblk * 4 : 0), 256);
  L.total = off;
  return L;
}

// Compute units of the current device in *out (queried once per device); a
// status code.
int device_cus(int* out) {
  static std::atomic<int> cus[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  int v = (dev >= 0 && dev < 64) ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (v <= 0) {
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute(multiprocessors)");
    if (dev >= 0 && dev < 64) cus[dev].store(v, std::memory_order_relaxed);
  }
  *out = v;
  return CSA2_OK;
}

// Scratch of the attention (its workgroups need none of their own).
size_t attention_scratch(int, int, int) { return 256; }

int check_indexer_args(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                       const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                       const float* w, int Hi, int score_mode, const int32_t* cand, int cand_stride,
                       int k, const int32_t* topk, int pool_k, const int32_t* pool) {
  if (!ik || !iks || !entry_offset || !n_entries || !q_idx || !topk)
    return fail(CSA2_ERR_NULL, "indexer: a required pointer is NULL");
  if (B < 1 || B > CSA2_MAX_BATCH)
    return fail(CSA2_ERR_SHAPE, "indexer: B must be in [1, %d] (got %d)", CSA2_MAX_BATCH, B);
  if (max_n < 0 || max_n > ((int64_t)1 << 26))
    return fail(CSA2_ERR_SHAPE, "indexer: max_n must be in [0, 2^26] (got %lld)", (long long)max_n);
  if (Hi < 1 || Hi > CSA2_MAX_INDEXER_HEADS)
    return fail(CSA2_ERR_SHAPE, "indexer: Hi must be in [1, %d] (got %d)", CSA2_MAX_INDEXER_HEADS, Hi);
  const int base_mode = score_mode & ~CSA2_SCORE_QMX8;
  if (base_mode != CSA2_SCORE_DOT && base_mode != CSA2_SCORE_RELU_W)
    return fail(CSA2_ERR_UNSUPPORTED, "indexer: unknown score_mode %d", score_mode);
  if (base_mode == CSA2_SCORE_DOT && Hi != 1)
    return fail(CSA2_ERR_SHAPE, "indexer: the DOT score takes exactly one head (got Hi=%d)", Hi);
  if (k < 1 || k > CSA2_MAX_K) return fail(CSA2_ERR_SHAPE, "indexer: k must be in [1, %d] (got %d)", CSA2_MAX_K, k);
  if (cand && (cand_stride < 1 || cand_stride > CSA2_MAX_POOL))
    return fail(CSA2_ERR_SHAPE, "indexer: cand_stride must be in [1, %d] (got %d)", CSA2_MAX_POOL, cand_stride);
  if (pool_k < 0 || pool_k > CSA2_MAX_POOL)
    return fail(CSA2_ERR_SHAPE, "indexer: pool_k must be in [0, %d] (got %d)", CSA2_MAX_POOL, pool_k);
  if (pool_k > 0 && !pool) return fail(CSA2_ERR_NULL, "indexer: pool_k > 0 needs a pool buffer");
  if (pool_k > 0 && cand) return fail(CSA2_ERR_UNSUPPORTED, "indexer: a pool is built by a Full pass only (cand must be NULL)");
  if (pool_k > 0 && pool_k < k) return fail(CSA2_ERR_SHAPE, "indexer: pool_k (%d) must be >= k (%d)", pool_k, k);
  if (!aligned16(ik) || !aligned4(iks) || !aligned16(q_idx) || !aligned16(entry_offset) ||
      !aligned16(n_entries) || !aligned16(topk) || (w && !aligned16(w)) || (cand && !aligned16(cand)) ||
      (pool && !aligned16(pool)))
    return fail(CSA2_ERR_ALIGN, "indexer: data pointers must be 16-byte aligned");
  return CSA2_OK;
}

int check_attention_args(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                         const int32_t* idx, int k, const uint16_t* q, int B, int H, const float* out) {
  if (!kv || !entry_offset || !n_entries || !idx || !q || !out)
    return fail(CSA2_ERR_NULL, "attention: a required pointer is NULL");
  if (B < 1) return fail(CSA2_ERR_SHAPE, "attention: B must be >= 1 (got %d)", B);
  if (k < 1 || k > CSA2_MAX_K) return fail(CSA2_ERR_SHAPE, "attention: k must be in [1, %d] (got %d)", CSA2_MAX_K, k);
  if (H < 1 || H > CSA2_MAX_HEADS)
    return fail(CSA2_ERR_SHAPE, "attention: H must be in [1, %d] (got %d)", CSA2_MAX_HEADS, H);
  if (!aligned16(kv) || !aligned16(entry_offset) || !aligned16(n_entries) || !aligned16(idx) ||
      !aligned16(q) || !aligned16(out))
    return fail(CSA2_ERR_ALIGN, "attention: data pointers must be 16-byte aligned");
  return CSA2_OK;
}

csa2::SelBufs make_selbufs(const IndexerWs& L, uint8_t* ws) {
  csa2::SelBufs sb;
  sb.ctrl = ws + L.ctrl;
  sb.bitmap = (uint32_t*)(ws + L.bitmap);
  sb.bm_stride = L.bm_words;
  sb.hdr = (uint64_t*)(ws + L.hdr);
  sb.hdr_stride = L.nblk;
  sb.summ = (uint32_t*)(ws + L.summ);
  sb.summ_stride = L.nblk * csa2::kSumWords;
  sb.wgc = (uint64_t*)(ws + L.wgc);
  sb.wgc_stride = L.nblk * csa2::kCandCap;
  sb.gscr = (uint64_t*)(ws + L.gscr);
  sb.gscr_stride = L.gscr_stride;
  sb.hdrp = (uint64_t*)(ws + L.hdrp);
  sb.wgcp = (uint64_t*)(ws + L.wgcp);
  sb.wgcp_stride = L.nblk * csa2::kPoolCap;
  sb.psync = L.psync != L.pxh ? (uint32_t*)(ws + L.psync) : nullptr;
  return sb;
}

// A Full pass's scoring launch, bracketed by the one-shot profiling events
// when they are set.
hipError_t score_full(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset, const int32_t* n_entries,
                      int B, int64_t max_n, const uint16_t* q_idx, const float* w, int Hi, int score_mode,
                      float* scores, int64_t sstride, const csa2::SelBufs& sb, int sel, int K, bool store,
                      int pool_k, hipStream_t stream) {
  hipEvent_t ev0 = g_ev_before, ev1 = g_ev_after;
  g_ev_before = g_ev_after = nullptr;
  hipError_t r;
  if (ev0 && (r = hipEventRecord(ev0, stream)) != hipSuccess) return r;
  r = csa2::launch_score(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, nullptr, 0,
                         scores, sstride, sb, sel, K, store, pool_k, stream);
  if (r != hipSuccess) return r;
  if (ev1 && (r = hipEventRecord(ev1, stream)) != hipSuccess) return r;
  return hipSuccess;
}

// Which selection a call takes.
bool direct_ok(int k) { return k <= csa2::kDirectMaxK; }
bool small_full(int64_t max_n) { return max_n <= csa2::kSmallMax; }

// A decode layer whose top-k is finished inside the attention launch (a Full
// layer with k <= 512 and more entries than the small path takes, or a
// Reindex layer with k <= 512): every attention workgroup, and the pool
// workgroups of a Full layer with a pool, get scratch rows of their own for
// the finish's fallback; the plan is off when they would exceed 4 GiB.
struct FusedPlan {
  bool on;
  int64_t sstride, gstride;   // floats / composites per workgroup row
  size_t bytes;
};

FusedPlan fused_plan(int mode, int B, int64_t max_n, int H, int k, int pool_k) {
  FusedPlan f{false, 0, 0, 0};
  if (!direct_ok(k)) return f;
  if (mode == CSA2_FULL && small_full(max_n)) return f;
  if (mode == CSA2_REUSE) return f;
  const size_t G = (size_t)csa2::attention_workgroups(B, H, k) + (mode == CSA2_FULL && pool_k > 0 ? (size_t)B : 0);
  const int64_t n = max_n > pool_k ? max_n : pool_k;
  f.sstride = (int64_t)round_up((size_t)n, 64);
  f.gstride = (int64_t)round_up((size_t)(n > csa2::kFinLdsCands ? n : csa2::kFinLdsCands), 32);
  f.bytes = round_up(G * (size_t)f.sstride * 4, 256) + round_up(G * (size_t)f.gstride * 8, 256);
  f.on = f.bytes <= ((size_t)1 << 32);
  if (!f.on) f.bytes = 0;
  return f;
}

// Runs the indexer with validated arguments on a validated workspace.
int run_indexer(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx, const float* w,
                int Hi, int score_mode, const int32_t* cand, int cand_stride, int k, int32_t* topk,
                int pool_k, int32_t* pool, float* scores_out, uint8_t* ws, hipStream_t stream) {
  const IndexerWs L = indexer_layout(B, max_n, k, pool_k, cand ? cand_stride : 0);
  const csa2::SelBufs sb = make_selbufs(L, ws);
  uint64_t* cbuf = (uint64_t*)(ws + L.cand);
  float* scores = scores_out ? scores_out : (float*)(ws + L.scores);
  const int64_t sstride = scores_out ? (cand ? cand_stride : max_n) : L.slots;
  const csa2::ScoreSrc src{ik, iks, entry_offset, q_idx, w, Hi, score_mode, nullptr, 0, nullptr, 0};
  hipError_t e;
  if (cand) {
    if (direct_ok(k)) {
      // Reindex: score the listed positions, local cutoffs, the finish
      e = csa2::launch_score(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, cand, cand_stride,
                             scores, sstride, sb, csa2::SEL_DIRECT, k, true, 0, stream);
      if (e != hipSuccess) return hip_status(e, "indexer score");
      csa2::ScoreSrc cs = src;
      cs.cand = cand;
      cs.cand_stride = cand_stride;
      cs.cand_scores = scores;
      cs.cand_scores_stride = sstride;
      e = csa2::launch_finish(csa2::SEL_DIRECT, n_entries, B, max_n, scores, sstride, sb, k, topk, k, &cs, stream);
      return hip_status(e, "indexer select");
    }
    e = csa2::launch_score(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, cand, cand_stride,
                           scores, sstride, sb, csa2::SEL_NONE, 0, true, 0, stream);
    if (e != hipSuccess) return hip_status(e, "indexer score");
    e = csa2::launch_select_small(scores, sstride, cand, cand_stride, 0, n_entries, B, max_n, k, topk, k, stream);
    return hip_status(e, "indexer select");
  }
  if (small_full(max_n)) {
    // every position fits one workgroup: scores, then the small select (the
    // pool first when asked, the top-k from it)
    e = score_full(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, scores, sstride, sb,
                   csa2::SEL_NONE, 0, true, 0, stream);
    if (e != hipSuccess) return hip_status(e, "indexer score");
    if (pool_k > 0) {
      e = csa2::launch_select_small(scores, sstride, nullptr, 0, 0, n_entries, B, max_n, pool_k, pool, pool_k, stream);
      if (e != hipSuccess) return hip_status(e, "indexer pool select");
      e = csa2::launch_select_small(scores, sstride, pool, pool_k, 1, n_entries, B, max_n, k, topk, k, stream);
      return hip_status(e, "indexer select");
    }
    e = csa2::launch_select_small(scores, sstride, nullptr, 0, 0, n_entries, B, max_n, k, topk, k, stream);
    return hip_status(e, "indexer select");
  }
  if (direct_ok(k)) {
    // local cutoffs in the score pass, then the finish (and the pool finish);
    // the top-k of the pool is the top-k of the sequence. Without scores_out
    // the pass keeps no scores; a finish recomputes a sequence's in its fallback
    e = score_full(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, scores, sstride, sb,
                   pool_k > 0 ? csa2::SEL_POOL : csa2::SEL_DIRECT, k, scores_out != nullptr, pool_k, stream);
    if (e != hipSuccess) return hip_status(e, "indexer score");
    e = csa2::launch_finish(csa2::SEL_DIRECT, n_entries, B, max_n, scores, sstride, sb, k, topk, k,
                            scores_out ? nullptr : &src, stream);
    if (e != hipSuccess) return hip_status(e, "indexer select");
    if (pool_k > 0) {
      // (its fallback rows: the scores region, which this path leaves unused,
      // and the gscr rows, free once the finish above has run)
      e = csa2::launch_pool_finish(n_entries, B, max_n, sb, pool_k, pool, (float*)(ws + L.scores), L.slots, sb.gscr,
                                   sb.gscr_stride, src, stream);
      if (e != hipSuccess) return hip_status(e, "indexer pool finish");
    }
    return ok();
  }
  // k > 512: threshold bin, marking pass, exact finish
  const int K1 = pool_k > 0 ? pool_k : k;
  int32_t* first_out = pool_k > 0 ? pool : topk;
  e = score_full(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, scores, sstride, sb,
                 csa2::SEL_THRESHOLD, K1, true, 0, stream);
  if (e != hipSuccess) return hip_status(e, "indexer score");
  e = csa2::launch_finish(csa2::SEL_THRESHOLD, n_entries, B, max_n, scores, sstride, sb, K1, nullptr, 0, nullptr,
                          stream);
  if (e != hipSuccess) return hip_status(e, "indexer threshold");
  e = csa2::launch_select(scores, sstride, n_entries, B, max_n, sb.ctrl, sb.bitmap, L.bm_words, cbuf, L.slots,
                          K1, first_out, K1, stream);
  if (e != hipSuccess) return hip_status(e, "indexer select");
  if (pool_k > 0) {
    e = csa2::launch_select_small(scores, sstride, pool, pool_k, 1, n_entries, B, max_n, k, topk, k, stream);
    if (e != hipSuccess) return hip_status(e, "indexer pool select");
  }
  return ok();
}

int check_decode_args(int mode, const uint8_t* kv, const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                      const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx, const float* w, int Hi,
                      int score_mode, const uint16_t* q, int H, int k, int pool_k, const int32_t* pool,
                      const int32_t* topk, const float* out, const float* lse) {
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_REUSE)
    return fail(CSA2_ERR_UNSUPPORTED, "decode_layer: unknown mode %d", mode);
  int rc = check_attention_args(kv, entry_offset, n_entries, topk, k, q, B, H, out);
  if (rc) return rc;
  if (lse && !aligned16(lse)) return fail(CSA2_ERR_ALIGN, "decode_layer: lse must be 16-byte aligned");
  if (mode == CSA2_FULL) {
    rc = check_indexer_args(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, nullptr, 0, k,
                            topk, pool_k, pool);
  } else if (mode == CSA2_REINDEX) {
    if (!pool || pool_k < 1) return fail(CSA2_ERR_NULL, "decode_layer: Reindex needs the pool (pool, pool_k >= 1)");
    rc = check_indexer_args(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, pool, pool_k, k,
                            topk, 0, nullptr);
  } else if (B > CSA2_MAX_BATCH) {
    return fail(CSA2_ERR_SHAPE, "decode_layer: B must be in [1, %d] (got %d)", CSA2_MAX_BATCH, B);
  }
  return rc;
}

}  // namespace

extern "C" {

int csa2_cache_write(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat, const float* w_idx,
                     int B, int64_t T, int m, const int64_t* n_tokens, const int64_t* out_entry_offset,
                     uint8_t* kv, uint8_t* ik, uint8_t* iks, void* stream) {
  if (!x_lat || !x_idx || !w_lat || !w_idx || !kv || !ik || !iks)
    return fail(CSA2_ERR_NULL, "cache_write: a required pointer is NULL");
  if (B < 1 || B > 65535) return fail(CSA2_ERR_SHAPE, "cache_write: B must be in [1, 65535] (got %d)", B);
  if (T < 0) return fail(CSA2_ERR_SHAPE, "cache_write: T must be >= 0 (got %lld)", (long long)T);
  if (m < 1 || m > CSA2_MAX_RATIO)
    return fail(CSA2_ERR_SHAPE, "cache_write: m must be in [1, %d] (got %d)", CSA2_MAX_RATIO, m);
  if ((int64_t)B * (T / m) > ((int64_t)1 << 35) || T / m > ((int64_t)1 << 35))
    return fail(CSA2_ERR_SHAPE, "cache_write: too many entries");
  if (!aligned16(x_lat) || !aligned16(x_idx) || !aligned16(w_lat) || !aligned16(w_idx) || !aligned16(kv) ||
      !aligned16(ik) || !aligned4(iks) || (n_tokens && !aligned16(n_tokens)) ||
      (out_entry_offset && !aligned16(out_entry_offset)))
    return fail(CSA2_ERR_ALIGN, "cache_write: data pointers must be 16-byte aligned (iks 4)");
  hipError_t e = csa2::launch_cache_write(x_lat, x_idx, w_lat, w_idx, B, T, m, n_tokens, out_entry_offset, kv, ik,
                                          iks, (hipStream_t)stream);
  return hip_status(e, "cache_write");
}

int csa2_cache_append(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat, const float* w_idx,
                      int B, int m, uint16_t* stage_lat, uint16_t* stage_idx, int32_t* stage_count,
                      const int64_t* entry_offset, int32_t* n_entries, const int64_t* capacity, uint8_t* kv,
                      uint8_t* ik, uint8_t* iks, int32_t* dropped, void* stream) {
  if (!x_lat || !x_idx || !w_lat || !w_idx || !stage_count || !entry_offset || !n_entries || !capacity || !kv ||
      !ik || !iks)
    return fail(CSA2_ERR_NULL, "cache_append: a required pointer is NULL");
  if (m > 1 && (!stage_lat || !stage_idx)) return fail(CSA2_ERR_NULL, "cache_append: m > 1 needs the stage buffers");
  if (B < 1 || B > CSA2_MAX_BATCH)
    return fail(CSA2_ERR_SHAPE, "cache_append: B must be in [1, %d] (got %d)", CSA2_MAX_BATCH, B);
  if (m < 1 || m > CSA2_MAX_RATIO)
    return fail(CSA2_ERR_SHAPE, "cache_append: m must be in [1, %d] (got %d)", CSA2_MAX_RATIO, m);
  if (!aligned16(x_lat) || !aligned16(x_idx) || !aligned16(w_lat) || !aligned16(w_idx) || !aligned16(kv) ||
      !aligned16(ik) || !aligned4(iks) || !aligned16(entry_offset) || !aligned16(capacity) ||
      !aligned4(stage_count) || !aligned4(n_entries) || (dropped && !aligned4(dropped)) ||
      (m > 1 && (!aligned16(stage_lat) || !aligned16(stage_idx))))
    return fail(CSA2_ERR_ALIGN, "cache_append: data pointers must be aligned (16 bytes; iks and counters 4)");
  hipError_t e = csa2::launch_cache_append(x_lat, x_idx, w_lat, w_idx, B, m, stage_lat, stage_idx, stage_count,
                                           entry_offset, n_entries, capacity, kv, ik, iks, dropped,
                                           (hipStream_t)stream);
  return hip_status(e, "cache_append");
}

int csa2_swa_write(const uint16_t* x_lat, int B, int64_t T, const int64_t* pos0, uint8_t* win, void* stream) {
  if (!x_lat || !pos0 || !win) return fail(CSA2_ERR_NULL, "swa_write: a required pointer is NULL");
  if (B < 1) return fail(CSA2_ERR_SHAPE, "swa_write: B must be >= 1 (got %d)", B);
  if (T < 0) return fail(CSA2_ERR_SHAPE, "swa_write: T must be >= 0");
  if (!aligned16(x_lat) || !aligned16(pos0) || !aligned16(win))
    return fail(CSA2_ERR_ALIGN, "swa_write: data pointers must be 16-byte aligned");
  return hip_status(csa2::launch_swa_write(x_lat, B, T, pos0, win, (hipStream_t)stream), "swa_write");
}

int csa2_swa_attention(const uint8_t* win, const int32_t* n_win, const uint16_t* q, int B, int H,
                       float softmax_scale, float* out, float* lse, void* stream) {
  if (!win || !n_win || !q || !out || !lse) return fail(CSA2_ERR_NULL, "swa_attention: a required pointer is NULL");
  if (B < 1 || B > CSA2_MAX_BATCH)
    return fail(CSA2_ERR_SHAPE, "swa_attention: B must be in [1, %d] (got %d)", CSA2_MAX_BATCH, B);
  if (H < 1 || H > CSA2_MAX_HEADS)
    return fail(CSA2_ERR_SHAPE, "swa_attention: H must be in [1, %d] (got %d)", CSA2_MAX_HEADS, H);
  if (!aligned16(win) || !aligned16(n_win) || !aligned16(q) || !aligned16(out) || !aligned16(lse))
    return fail(CSA2_ERR_ALIGN, "swa_attention: data pointers must be 16-byte aligned");
  return hip_status(csa2::launch_swa_attention(win, n_win, q, B, H, softmax_scale, out, lse, (hipStream_t)stream),
                    "swa_attention");
}

size_t csa2_indexer_workspace_bytes(int B, int64_t max_n, int k, int pool_k, int cand_stride) {
  if (B < 1 || B > CSA2_MAX_BATCH || max_n < 0 || k < 1 || pool_k < 0 || cand_stride < 0) return 0;
  return indexer_layout(B, max_n, k, pool_k, cand_stride).total;
}

int csa2_indexer_topk(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                      const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx, const float* w,
                      int Hi, int score_mode, const int32_t* cand, int cand_stride, int k, int32_t* topk,
                      int pool_k, int32_t* pool, float* scores_out, void* workspace, size_t ws_bytes,
                      void* stream) {
  int rc = check_indexer_args(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, cand,
                              cand_stride, k, topk, pool_k, pool);
  if (rc) return rc;
  if (scores_out && !aligned16(scores_out)) return fail(CSA2_ERR_ALIGN, "indexer: scores_out must be 16-byte aligned");
  const size_t need = indexer_layout(B, max_n, k, pool_k, cand ? cand_stride : 0).total;
  if (!workspace || ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE, "indexer: workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(CSA2_ERR_ALIGN, "indexer: workspace must be 16-byte aligned");
  return run_indexer(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, cand, cand_stride, k,
                     topk, pool_k, pool, scores_out, (uint8_t*)workspace, (hipStream_t)stream);
}

size_t csa2_attention_workspace_bytes(int B, int H, int k) {
  if (B < 1 || H < 1 || H > CSA2_MAX_HEADS || k < 1) return 0;
  return attention_scratch(B, H, k);
}

int csa2_sparse_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                          const int32_t* idx, int k, const uint16_t* q, int B, int H, float softmax_scale,
                          float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_attention_args(kv, entry_offset, n_entries, idx, k, q, B, H, out);
  if (rc) return rc;
  if (lse && !aligned16(lse)) return fail(CSA2_ERR_ALIGN, "attention: lse must be 16-byte aligned");
  const size_t need = attention_scratch(B, H, k);
  if (!workspace || ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE, "attention: workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(CSA2_ERR_ALIGN, "attention: workspace must be 16-byte aligned");
  hipError_t e = csa2::launch_attention(kv, entry_offset, n_entries, idx, k, q, B, H, softmax_scale, 1, out, lse,
                                        nullptr, nullptr, (hipStream_t)stream);
  return hip_status(e, "attention");
}

size_t csa2_decode_workspace_bytes(int B, int64_t max_n, int H, int k, int pool_k) {
  if (B < 1 || B > CSA2_MAX_BATCH || max_n < 0 || H < 1 || H > CSA2_MAX_HEADS || k < 1 || pool_k < 0) return 0;
  // the largest of the three modes' needs (a Reindex layer scores a list of pool_k)
  size_t need = 0;
  for (int mode = CSA2_FULL; mode <= CSA2_REUSE; ++mode) {
    const size_t idx = mode == CSA2_REUSE ? 0
                       : indexer_layout(B, max_n, k, mode == CSA2_FULL ? pool_k : 0,
                                        mode == CSA2_REINDEX ? pool_k : 0).total;
    const size_t t = idx + attention_scratch(B, H, k) + fused_plan(mode, B, max_n, H, k, pool_k).bytes;
    need = t > need ? t : need;
  }
  return need;
}

namespace {
// One decode layer with validated arguments on a validated workspace.
int run_decode_layer(int mode, const uint8_t* kv, const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                     const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx, const float* w, int Hi,
                     int score_mode, const uint16_t* q, int H, float softmax_scale, int k, int pool_k, int32_t* pool,
                     int32_t* topk, float* out, float* lse, uint8_t* ws, hipStream_t s, bool allow_fused = true,
                     int pre_B = 0, int pre_Tq = 0, const csa2::PrefillViews* pv = nullptr) {
  const FusedPlan fp = fused_plan(mode, B, max_n, H, k, pool_k);
  const int cand_stride = mode == CSA2_REINDEX ? pool_k : 0;
  int rc0 = CSA2_OK;
  // a prefill's virtual batch (pre_Tq > 0; pv: the sequences, positions and
  // the views' arrays entry_offset and n_entries): the multi-query pass
  // computes and writes the views itself; every other plan takes them from a
  // launch of their own first
  const bool multi_query = pre_Tq > 0 && fp.on && allow_fused && mode == CSA2_FULL && pool_k == 0 &&
                           (score_mode & CSA2_SCORE_QMX8) == 0;
  if (pre_Tq > 0 && !multi_query) {
    const hipError_t e = csa2::launch_prefill_views(pv->entry_offset, pv->n_entries, pv->pos, pv->m, pre_B, pre_Tq,
                                                    pv->eo, pv->ne, s);
    if (e != hipSuccess) return hip_status(e, "prefill_layer views");
  }
  if (fp.on && allow_fused) {
    // scoring launch, then the attention that runs the top-k finish itself
    // (and, for a Full layer with a pool, the pool finish in workgroups of its own)
    const IndexerWs L = indexer_layout(B, max_n, k, mode == CSA2_FULL ? pool_k : 0, cand_stride);
    const csa2::SelBufs sb = make_selbufs(L, ws);
    float* scores = (float*)(ws + L.scores);
    csa2::FusedFinish ff;
    ff.sb = sb;
    ff.src = csa2::ScoreSrc{ik, iks, entry_offset, q_idx, w, Hi, score_mode, nullptr, 0, nullptr, 0};
    ff.pool_k = 0;
    ff.pool = nullptr;
    ff.px = csa2::PoolExchange{nullptr, nullptr, nullptr, nullptr, L.nblk, 1};
    hipError_t e;
    if (multi_query) {
      // the multi-query pass reads each key tile once for several of a
      // sequence's queries
      e = csa2::launch_score_prefill(ik, iks, pre_B, pre_Tq, max_n, q_idx, w, Hi, score_mode, sb, k, *pv, s);
    } else if (mode == CSA2_FULL) {
      e = score_full(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, scores, L.slots, sb,
                     pool_k > 0 ? csa2::SEL_POOL : csa2::SEL_DIRECT, k, false, pool_k, s);
      ff.pool_k = pool_k;
      ff.pool = pool;
      if (pool_k > 0) {
        // the pool finish split over as many workgroups per sequence as stay
        // resident beside the attention's (one workgroup per compute unit;
        // a launch that asks for every unit waits for some of them, so three
        // quarters), each with at least 8 chunk lists
        const int G = csa2::attention_workgroups(B, H, k);
        int cus = 0;
        if ((rc0 = device_cus(&cus)) != CSA2_OK) return rc0;
        int parts = L.pool_parts_max;
        parts = std::min(parts, std::max(1, (cus * 3 / 4 - G) / B));
        parts = std::min(parts, std::max(1, (int)(L.nblk / 8)));
        ff.px = csa2::PoolExchange{(uint32_t*)(ws + L.pxh), (uint64_t*)(ws + L.pxk), (uint32_t*)(ws + L.pxn),
                                   (uint32_t*)(ws + L.pxc), L.nblk, parts};
      }
    } else {
      e = csa2::launch_score(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, pool, pool_k,
                             scores, L.slots, sb, csa2::SEL_DIRECT, k, true, 0, s);
      ff.src.cand = pool;
      ff.src.cand_stride = pool_k;
      ff.src.cand_scores = scores;
      ff.src.cand_scores_stride = L.slots;
    }
    if (e != hipSuccess) return hip_status(e, "decode_layer score");
    const size_t need_idx = L.total;
    uint8_t* fb = ws + need_idx + attention_scratch(B, H, k);
    const size_t G = (size_t)csa2::attention_workgroups(B, H, k) + (ff.pool_k > 0 ? (size_t)B : 0);
    ff.max_n = max_n;
    ff.scores = (float*)fb;
    ff.scores_stride = fp.sstride;
    ff.gscr = (uint64_t*)(fb + round_up(G * (size_t)fp.sstride * 4, 256));
    ff.gscr_stride = fp.gstride;
    ff.topk = topk;
    e = csa2::launch_attention(kv, entry_offset, n_entries, topk, k, q, B, H, softmax_scale, 1, out, lse, nullptr,
                               &ff, s);
    return hip_status(e, "decode_layer attention");
  }
  int rc = CSA2_OK;
  if (mode == CSA2_FULL) {
    rc = run_indexer(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, nullptr, 0, k, topk,
                     pool_k, pool, nullptr, ws, s);
  } else if (mode == CSA2_REINDEX) {
    rc = run_indexer(ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, pool, pool_k, k, topk, 0,
                     nullptr, nullptr, ws, s);
  }
  if (rc) return rc;
  hipError_t e = csa2::launch_attention(kv, entry_offset, n_entries, topk, k, q, B, H, softmax_scale, 1, out, lse,
                                        nullptr, nullptr, s);
  return hip_status(e, "decode_layer attention");
}
}  // namespace

// Scratch of csa2_decode_layer_noalloc: one copy per device, held until the
// process ends. Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch in *out (looked up on the
// first call on that device, with the device current); a status code.
int device_scratch(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "decode_layer_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA2_ERR_UNSUPPORTED, "decode_layer_noalloc: device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "decode_layer_noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(CSA2_ERR_HIP, "decode_layer_noalloc: hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = (uint8_t*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}
}  // namespace

int csa2_decode_layer_noalloc(int mode, const uint8_t* kv, const uint8_t* ik, const uint8_t* iks,
                              const int64_t* entry_offset, const int32_t* n_entries, int B, int64_t max_n,
                              const uint16_t* q_idx, const float* w, int Hi, int score_mode, const uint16_t* q, int H,
                              float softmax_scale, int k, int pool_k, int32_t* pool, int32_t* topk, float* out,
                              float* lse, void* stream) {
  int rc = check_decode_args(mode, kv, ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, q, H, k,
                             pool_k, pool, topk, out, lse);
  if (rc) return rc;
  // this mode's scratch: the fused plan (scoring, then the attention that
  // finishes the top-k itself) when it fits, else the plan of separate launches
  const size_t cap = (size_t)CSA2_NOALLOC_SCRATCH_BYTES;
  const size_t idx = mode == CSA2_REUSE ? 0
                     : indexer_layout(B, max_n, k, mode == CSA2_FULL ? pool_k : 0,
                                      mode == CSA2_REINDEX ? pool_k : 0).total;
  const FusedPlan fp = fused_plan(mode, B, max_n, H, k, pool_k);
  const size_t need_fused = fp.on ? idx + attention_scratch(B, H, k) + fp.bytes : 0;
  const bool fused = fp.on && need_fused <= cap;
  if (!fused && idx > cap)
    return fail(CSA2_ERR_WORKSPACE, "decode_layer_noalloc: needs %zu bytes of scratch, the static scratch holds %zu",
                idx, cap);
  uint8_t* ws = nullptr;
  rc = device_scratch(&ws);
  if (rc) return rc;
  return run_decode_layer(mode, kv, ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, q, H,
                          softmax_scale, k, pool_k, pool, topk, out, lse, ws, (hipStream_t)stream, fused);
}

}  // extern "C"

namespace {
// csa2_decode_layer, and (pre_Tq > 0) the virtual decode batch of a prefill:
// B = pre_B * pre_Tq queries of pre_B sequences, whose views (written to
// entry_offset and n_entries before they are read) pv describes.
int decode_layer_ws(int mode, const uint8_t* kv, const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                    const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx, const float* w, int Hi,
                    int score_mode, const uint16_t* q, int H, float softmax_scale, int k, int pool_k, int32_t* pool,
                    int32_t* topk, float* out, float* lse, void* workspace, size_t ws_bytes, void* stream, int pre_B,
                    int pre_Tq, const csa2::PrefillViews* pv) {
  int rc = check_decode_args(mode, kv, ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, q, H, k,
                             pool_k, pool, topk, out, lse);
  if (rc) return rc;
  const size_t need = csa2_decode_workspace_bytes(B, max_n, H, k, pool_k);
  if (!workspace || ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE, "decode_layer: workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(CSA2_ERR_ALIGN, "decode_layer: workspace must be 16-byte aligned");
  return run_decode_layer(mode, kv, ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, q, H,
                          softmax_scale, k, pool_k, pool, topk, out, lse, (uint8_t*)workspace, (hipStream_t)stream,
                          true, pre_B, pre_Tq, pv);
}
}  // namespace

extern "C" {

int csa2_decode_layer(int mode, const uint8_t* kv, const uint8_t* ik, const uint8_t* iks,
                      const int64_t* entry_offset, const int32_t* n_entries, int B, int64_t max_n,
                      const uint16_t* q_idx, const float* w, int Hi, int score_mode, const uint16_t* q, int H,
                      float softmax_scale, int k, int pool_k, int32_t* pool, int32_t* topk, float* out,
                      float* lse, void* workspace, size_t ws_bytes, void* stream) {
  return decode_layer_ws(mode, kv, ik, iks, entry_offset, n_entries, B, max_n, q_idx, w, Hi, score_mode, q, H,
                         softmax_scale, k, pool_k, pool, topk, out, lse, workspace, ws_bytes, stream, 0, 0, nullptr);
}

size_t csa2_prefill_workspace_bytes(int B, int Tq, int64_t max_n, int H, int k) {
  if (B < 1 || Tq < 1 || (int64_t)B * Tq > CSA2_MAX_BATCH) return 0;
  const int Bv = B * Tq;
  const size_t d = csa2_decode_workspace_bytes(Bv, max_n, H, k, 0);
  if (d == 0) return 0;
  return d + round_up((size_t)Bv * 8, 256) + round_up((size_t)Bv * 4, 256);
}

int csa2_prefill_layer(const uint8_t* kv, const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                       const int32_t* n_entries, int B, int64_t max_n, int m, int Tq, const int64_t* pos,
                       const uint16_t* q_idx, const float* w, int Hi, int score_mode, const uint16_t* q, int H,
                       float softmax_scale, int k, int32_t* topk, float* out, float* lse, void* workspace,
                       size_t ws_bytes, void* stream) {
  if (!pos || !entry_offset || !n_entries) return fail(CSA2_ERR_NULL, "prefill_layer: a required pointer is NULL");
  if (B < 1 || Tq < 1 || (int64_t)B * Tq > CSA2_MAX_BATCH)
    return fail(CSA2_ERR_SHAPE, "prefill_layer: need B >= 1, Tq >= 1 and B * Tq <= %d (got %d x %d)", CSA2_MAX_BATCH,
                B, Tq);
  if (m < 1 || m > CSA2_MAX_RATIO)
    return fail(CSA2_ERR_SHAPE, "prefill_layer: m must be in [1, %d] (got %d)", CSA2_MAX_RATIO, m);
  if (!aligned16(pos) || !aligned16(entry_offset) || !aligned16(n_entries))
    return fail(CSA2_ERR_ALIGN, "prefill_layer: data pointers must be 16-byte aligned");
  const int Bv = B * Tq;
  const size_t dneed = csa2_decode_workspace_bytes(Bv, max_n, H, k, 0);
  const size_t need = csa2_prefill_workspace_bytes(B, Tq, max_n, H, k);
  if (dneed == 0 || need == 0) return fail(CSA2_ERR_SHAPE, "prefill_layer: bad sizes (max_n, H or k)");
  if (!workspace || ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE, "prefill_layer: workspace needs %zu bytes (got %zu)", need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(CSA2_ERR_ALIGN, "prefill_layer: workspace must be 16-byte aligned");
  uint8_t* views = (uint8_t*)workspace + dneed;
  int64_t* eo = (int64_t*)views;
  int32_t* ne = (int32_t*)(views + round_up((size_t)Bv * 8, 256));
  const csa2::PrefillViews pv{entry_offset, n_entries, pos, m, eo, ne};
  return decode_layer_ws(CSA2_FULL, kv, ik, iks, eo, ne, Bv, max_n, q_idx, w, Hi, score_mode, q, H, softmax_scale, k,
                         0, nullptr, topk, out, lse, workspace, dneed, stream, B, Tq, &pv);
}

double csa2_bytes_per_token(const int* ratios, int n_layers, int lat_ch, int lat_blk, int lat_sbytes, int idx_ch,
                            int idx_blk, int idx_sbytes) {
  if (!ratios || n_layers < 0 || lat_ch < 0 || idx_ch < 0 || lat_blk < 0 || idx_blk < 0 || lat_sbytes < 0 ||
      idx_sbytes < 0) {
    fail(CSA2_ERR_SHAPE, "bytes_per_token: bad arguments");
    return -1.0;
  }
  double total = 0.0;
  for (int i = 0; i < n_layers; ++i) {
    if (ratios[i] < 1) {
      fail(CSA2_ERR_SHAPE, "bytes_per_token: ratio must be >= 1");
      return -1.0;
    }
    double lat = lat_ch * 0.5 + (lat_blk ? (double)lat_ch / lat_blk * lat_sbytes : 0.0);
    double idx = idx_ch * 0.5 + (idx_blk ? (double)idx_ch / idx_blk * idx_sbytes : 0.0);
    total += (lat + idx) / ratios[i];
  }
  ok();
  return total;
}

int csa2_set_profile_events(void* before_score, void* after_score) {
  if ((before_score == nullptr) != (after_score == nullptr))
    return fail(CSA2_ERR_NULL, "set_profile_events: give both events or neither");
  g_ev_before = (hipEvent_t)before_score;
  g_ev_after = (hipEvent_t)after_score;
  return ok();
}

const char* csa2_last_error(void) { return g_err; }

}  // extern "C"
