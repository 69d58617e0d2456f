// Host-visible launchers of the gfx950 kernels (internal to libcsa2fp4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Per-sequence selection state of the threshold path (k > 512). The threshold
// kernel sets it (including the candidate counter) before the select kernel
// reads it, so the workspace holds no state between calls.
struct SelState {
  uint32_t unused0;
  uint32_t unused1;
  int32_t thr_bin;        // histogram bin holding the K-th best key (-1: all selected)
  uint32_t above;         // keys in bins above thr_bin
  uint32_t ncand;         // select pass: candidates appended from thr_bin
  uint32_t pad[11];
};
static_assert(sizeof(SelState) == 64, "control block header");

constexpr int kNumBins = 4096;
constexpr int kSmallMax = 16384;
constexpr int64_t kCtrlStride = 64;   // one SelState per sequence
__host__ __device__ inline SelState* ctrl_state(uint8_t* ctrl, int b) { return (SelState*)(ctrl + b * kCtrlStride); }

hipError_t launch_cache_write(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                              const float* w_idx, int B, int64_t T, int m, const int64_t* n_tokens,
                              const int64_t* out_entry_offset, uint8_t* kv, uint8_t* ik, uint8_t* iks,
                              hipStream_t stream);
// Prefill: the decode batch of B * Tq per-query views of B sequences.
hipError_t launch_prefill_views(const int64_t* entry_offset, const int32_t* n_entries, const int64_t* pos, int m,
                                int B, int Tq, int64_t* eo, int32_t* ne, hipStream_t stream);

// Sliding window: 128 tokens per sequence, 544-byte FP8 rows.
constexpr int kSwaWindow = 128;
constexpr int kSwaRowBytes = 544;
hipError_t launch_swa_write(const uint16_t* x, int B, int64_t T, const int64_t* pos0, uint8_t* win,
                            hipStream_t stream);
hipError_t launch_swa_attention(const uint8_t* win, const int32_t* n_win, const uint16_t* q, int B, int H,
                                float tau, float* out, float* lse, hipStream_t stream);
hipError_t launch_cache_append(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                               const float* w_idx, int B, int m, uint16_t* st_lat, uint16_t* st_idx,
                               int32_t* st_count, const int64_t* entry_offset, int32_t* n_entries,
                               const int64_t* capacity, uint8_t* kv, uint8_t* ik, uint8_t* iks, int32_t* dropped,
                               hipStream_t stream);

// Selection modes of the score pass.
enum { SEL_NONE = 0, SEL_THRESHOLD = 1, SEL_DIRECT = 2, SEL_POOL = 3 };
constexpr int kScoreChunk = 1024;     // slots per score workgroup
constexpr int kScoreQmx8 = 0x100;     // score-mode flag: MXFP8 query, block-scaled FP8 x FP4 MFMA
constexpr int kSumWords = 32;         // (bin, count) pairs a workgroup may report
constexpr int kCandCap = 256;         // candidates a workgroup reports in direct mode
constexpr int kDirectMaxK = 512;      // largest k the score pass selects by itself
constexpr int kFinMaxWg = 2048;       // score workgroups per sequence whose slots the finish reads
constexpr int kFinLdsCands = 12288;   // candidates the direct finish holds in LDS
constexpr int kPoolCap = kScoreChunk;  // pool candidates a score workgroup may report (its whole chunk)
constexpr int kCandChunk = 256;      // slots per workgroup (and selection chunk) of a candidate-list direct pass

// Workspace views used by the score pass's selection (per-sequence strides).
struct SelBufs {
  uint8_t* ctrl;        // SelState per sequence (threshold path)
  uint32_t* bitmap;     // [B][bm_stride] words; the score pass clears its chunk's words
  int64_t bm_stride;
  uint64_t* hdr;        // [B][hdr_stride]: one header word per score workgroup
  int64_t hdr_stride;
  uint32_t* summ;       // [B][summ_stride] words: kSumWords (bin, count) pairs per workgroup
  int64_t summ_stride;
  uint64_t* wgc;        // [B][wgc_stride]: kCandCap candidates per workgroup (direct mode)
  int64_t wgc_stride;
  uint64_t* gscr;       // [B][gscr_stride]: gathered candidates that do not fit LDS
  int64_t gscr_stride;
  uint64_t* hdrp;       // [B][hdr_stride]: pool header per score workgroup (pool mode)
  uint64_t* wgcp;       // [B][wgcp_stride]: kPoolCap pool candidates per workgroup (pool mode)
  int64_t wgcp_stride;
  uint32_t* psync;      // [B][4]: arrival counters of a split pool finish; the pool-mode
                        // score pass sets them to zero (NULL: nothing to clear)
};

// A pool finish split over `parts` workgroups per sequence, each sweeping a
// contiguous range of the chunk lists; they exchange per-part histograms,
// per-chunk counts and the keys inside the threshold bin through these
// buffers (device-scope loads and stores) and wait for one another at two
// counters of SelBufs::psync. Workgroup bytes per sequence and part:
// kPoolXBins * 4 + kPoolXKeys * 8 + 4, plus 4 per chunk.
constexpr int kPoolXBins = 4096;       // histogram bins of the pool finish
constexpr int kPoolXKeys = 4096;       // threshold-bin keys a split finish exchanges (in total)
constexpr int kPoolMaxParts = 16;      // workgroups per sequence
constexpr int kPoolPartBudget = 256;   // pool workgroups of one launch, at most (all resident at once)
struct PoolExchange {
  uint32_t* hist;       // [B][parts][kPoolXBins]
  uint64_t* keys;       // [B][parts][kPoolXKeys]
  uint32_t* nkeys;      // [B][parts]
  uint32_t* counts;     // [B][nblk]
  int64_t nblk;
  int parts;            // 1: one workgroup per sequence, nothing exchanged
};

// What the score pass reads, for a finish that has to recompute scores; for a
// candidate list (Reindex), the list and the scores the pass stored per slot
// (a slot the list does not use holds the key 0) instead.
struct ScoreSrc {
  const uint8_t* ik;
  const uint8_t* iks;
  const int64_t* entry_offset;
  const uint16_t* q_idx;
  const float* w;
  int Hi;
  int mode;
  const int32_t* cand;          // [B][cand_stride] or NULL
  int cand_stride;
  const float* cand_scores;     // [B][cand_scores_stride]
  int64_t cand_scores_stride;
};

// store_scores: direct and pool modes may skip storing the scores (the finish
// recomputes a sequence's scores in its rare fallback); the other modes, and
// every candidate-list pass, always store. pool_k: the pool size (pool mode).
hipError_t launch_score(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                        const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                        const float* w, int Hi, int mode, const int32_t* cand, int cand_stride,
                        float* scores, int64_t sstride, const SelBufs& sb, int sel, int K,
                        bool store_scores, int pool_k, hipStream_t stream);

// The multi-query scoring pass of a prefill (direct top-k, exact scores): B
// sequences of Tq queries; eo / ne / q_idx / w / sb are per query (virtual
// sequence b * Tq + t, ne = its visible entries). The finish and attention of
// the virtual decode batch follow unchanged.
// The multi-query pass computes the views itself from the sequences' arrays
// and the token positions, uses them, and its first workgroup of each query
// group writes them to eo and ne for the launches that follow.
struct PrefillViews {
  const int64_t* entry_offset;   // [B] the sequences' first cache rows
  const int32_t* n_entries;      // [B] the sequences' entries
  const int64_t* pos;            // [B][Tq] token position of every query
  int m;                         // merge ratio
  int64_t* eo;                   // [B * Tq] out: every query's first cache row
  int32_t* ne;                   // [B * Tq] out: every query's visible entries
};
hipError_t launch_score_prefill(const uint8_t* ik, const uint8_t* iks, int B, int Tq, int64_t max_n,
                                const uint16_t* q_idx, const float* w, int Hi, int mode, const SelBufs& sb, int K,
                                const PrefillViews& pv, hipStream_t stream);

// src: non-null when the direct score pass did not store the scores, or for a
// candidate list (src->cand set).
hipError_t launch_finish(int sel, const int32_t* n_entries, int B, int64_t max_n, float* scores,
                         int64_t sstride, const SelBufs& sb, int K, int32_t* out, int out_stride,
                         const ScoreSrc* src, hipStream_t stream);

hipError_t launch_select(const float* scores, int64_t sstride, const int32_t* n_entries, int B,
                         int64_t max_n, uint8_t* ctrl, uint32_t* bitmap, int64_t bm_stride,
                         uint64_t* cbuf, int64_t cb_stride, int K, int32_t* out, int out_stride,
                         hipStream_t stream);

hipError_t launch_select_small(const float* scores, int64_t sstride, const int32_t* slot_pos,
                               int pstride, int score_by_pos, const int32_t* n_entries, int B,
                               int64_t max_n, int K, int32_t* out, int out_stride, hipStream_t stream);

// Pool finish of a pool-mode score pass, one workgroup per sequence: the best
// pool_k positions, ascending, into pool [B][pool_k]. scratch rows (scores,
// composites) per sequence serve its fallback.
hipError_t launch_pool_finish(const int32_t* n_entries, int B, int64_t max_n, const SelBufs& sb, int pool_k,
                              int32_t* pool, float* sc_rows, int64_t sc_stride, uint64_t* g_rows, int64_t g_stride,
                              const ScoreSrc& src, hipStream_t stream);

// A decode attention that derives its indices itself: every workgroup runs the
// direct top-k finish of its sequence over the lists a direct score pass left
// (scores not stored, or a candidate list's stored scores), keeps the result in
// LDS, and the first workgroup of each sequence writes the top-k to `topk`.
// scores / gscr give every workgroup rows of its own for the finish's fallback.
// With pool_k > 0 the launch has B * px.parts more workgroups, px.parts per
// sequence, that run the pool finish of a pool-mode score pass into `pool`
// (part 0 of each sequence uses the sequence's scratch rows G + b).
struct FusedFinish {
  SelBufs sb;
  ScoreSrc src;
  int64_t max_n;
  float* scores;          // [workgroups][scores_stride] (>= max_n floats per row)
  int64_t scores_stride;
  uint64_t* gscr;         // [workgroups][gscr_stride] (>= max(max_n, kFinLdsCands) per row)
  int64_t gscr_stride;
  int32_t* topk;          // [B][k]
  int pool_k;             // 0, or the pool size
  int32_t* pool;          // [B][pool_k]
  PoolExchange px;        // the split of the pool finish (px.parts >= 1)
};

// Attention: number of entry splits used for B sequences, H heads, k indices.
int attention_splits(int B, int H, int k);
int attention_workgroups(int B, int H, int k);
size_t attention_lds_bytes();
// fin: null (indices from idx) or the finish to run first (idx unused).
hipError_t launch_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                            const int32_t* idx, int k, const uint16_t* q, int B, int H, float tau,
                            int S, float* out, float* lse, float* part, const FusedFinish* fin,
                            hipStream_t stream);

}  // namespace csa2
