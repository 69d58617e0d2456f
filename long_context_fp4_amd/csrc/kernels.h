// Host-visible launchers of the gfx950 kernels (internal to libcsa2fp4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Per-sequence selection state kept in the indexer workspace (zero between calls).
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
// Per-sequence control block of the indexer workspace: SelState, then the
// histogram. The control region at the start of the workspace always holds
// CSA2_MAX_BATCH blocks, so a block's place never depends on B or max_n.
constexpr int64_t kCtrlStride = 256 + 4 * kNumBins;   // 16640 bytes
__host__ __device__ inline SelState* ctrl_state(uint8_t* ctrl, int b) { return (SelState*)(ctrl + b * kCtrlStride); }
__host__ __device__ inline uint32_t* ctrl_hist(uint8_t* ctrl, int b) { return (uint32_t*)(ctrl + b * kCtrlStride + 256); }

hipError_t launch_cache_write(const uint16_t* x_lat, const uint16_t* x_idx, const float* w_lat,
                              const float* w_idx, int B, int64_t T, int m, uint8_t* kv, uint8_t* ik,
                              uint8_t* iks, hipStream_t stream);
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
                               int64_t capacity, uint8_t* kv, uint8_t* ik, uint8_t* iks, int32_t* dropped,
                               hipStream_t stream);

// Selection modes of the score pass.
enum { SEL_NONE = 0, SEL_THRESHOLD = 1, SEL_DIRECT = 2 };
constexpr int kScoreChunk = 1024;     // slots per score workgroup
constexpr int kScoreQmx8 = 0x100;     // score-mode flag: MXFP8 query, block-scaled FP8 x FP4 MFMA
constexpr int kSumWords = 32;         // (bin, count) pairs a workgroup may report
constexpr int kCandCap = 256;         // candidates a workgroup reports in direct mode
constexpr int kDirectMaxK = 512;      // largest k the score pass selects by itself
constexpr int kFinMaxWg = 2048;       // score workgroups per sequence whose slots the finish reads
constexpr int kFinLdsCands = 12288;   // candidates the direct finish holds in LDS

// Workspace views used by the score pass's selection (per-sequence strides).
struct SelBufs {
  uint8_t* ctrl;        // control blocks (SelState + histogram), fixed places
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
};

// What the score pass reads, for a finish that has to recompute scores.
struct ScoreSrc {
  const uint8_t* ik;
  const uint8_t* iks;
  const int64_t* entry_offset;
  const uint16_t* q_idx;
  const float* w;
  int Hi;
  int mode;
};

// store_scores: direct mode may skip storing the scores (the finish recomputes
// a sequence's scores in its rare fallback); the other modes always store.
hipError_t launch_score(const uint8_t* ik, const uint8_t* iks, const int64_t* entry_offset,
                        const int32_t* n_entries, int B, int64_t max_n, const uint16_t* q_idx,
                        const float* w, int Hi, int mode, const int32_t* cand, int cand_stride,
                        float* scores, int64_t sstride, const SelBufs& sb, int sel, int K,
                        bool store_scores, hipStream_t stream);

// src: non-null when the direct score pass did not store the scores.
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

// A decode attention that derives its indices itself: every workgroup runs the
// direct top-k finish of its sequence over the lists a direct score pass left
// (scores not stored), keeps its split of the result in LDS, and the first
// workgroup of each sequence writes the top-k to `topk`. scores / gscr give
// every attention workgroup rows of its own for the finish's fallback.
struct FusedFinish {
  SelBufs sb;
  ScoreSrc src;
  int64_t max_n;
  float* scores;          // [workgroups][scores_stride] (>= max_n floats per row)
  int64_t scores_stride;
  uint64_t* gscr;         // [workgroups][gscr_stride] (>= max(max_n, kFinLdsCands) per row)
  int64_t gscr_stride;
  int32_t* topk;          // [B][k]
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
