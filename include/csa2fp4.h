/*
 * csa2fp4.h — C ABI of the FP4 compressed global KV cache and its sparse
 * decode path (CSA2-style attention), for AMD MI355X (gfx950).
 *
 * Pages this interface follows (web pages on DeepSeek-V4.1-Flash's cache):
 *   [FP4] "Le cache KV en FP4 — les 890 octets, vérifiés" (mkdocs.reaper.mx)
 *   [CS]  "DeepSeek V4.1 Flash : 890 octets de cache KV par token" (contextstudios.ai)
 *   [TF]  "DeepSeek-V4.1 Flash compresse le KV-Cache de 4 fois" (techfi24.com)
 *   [F24] "KV cache da 890 byte per token" (flash24.org)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *   never allocates, frees or retains them; it only enqueues kernels on
 *   `stream` (a hipStream_t passed as void*; NULL = the null stream). Calls
 *   return as soon as the work is enqueued and are ordered on that stream.
 * - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 * - Return value: CSA2_OK (0) or a negative CSA2_ERR_* code. On an argument
 *   error nothing is enqueued and no HIP call is made; csa2_last_error()
 *   then returns a message for the calling thread. Device-side faults surface
 *   at the caller's next synchronisation of the stream.
 * - Alignment: every data pointer must be 16-byte aligned (CSA2_ERR_ALIGN),
 *   except the E8M0 key-scale array iks, which needs 4 bytes (one entry's row),
 *   so that a cache can start at any entry of a larger buffer.
 * - Workspaces: scratch device memory of at least the size the matching
 *   *_workspace_bytes call returns. It needs no initialisation and holds no
 *   state between calls (every kernel writes what it reads), so one workspace
 *   can serve later calls of any kind and size. Calls that share a workspace
 *   must not overlap (use one stream or separate workspaces).
 * - Thread safety: the library holds no global mutable state apart from the
 *   thread-local last-error message.
 */
#ifndef CSA2FP4_H
#define CSA2FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CSA2_OK               0
#define CSA2_ERR_NULL        -1  /* a required pointer is NULL */
#define CSA2_ERR_SHAPE       -2  /* a size or count is out of range */
#define CSA2_ERR_ALIGN       -3  /* a data pointer is not 16-byte aligned */
#define CSA2_ERR_WORKSPACE   -4  /* workspace missing or smaller than required */
#define CSA2_ERR_UNSUPPORTED -5  /* a mode or option this build does not implement */
#define CSA2_ERR_HIP         -6  /* the HIP runtime reported an error at launch */

/* indexer score definitions */
#define CSA2_SCORE_DOT     0   /* S_i = q . k_i, exactly one indexer head */
#define CSA2_SCORE_RELU_W  1   /* S_i = sum_h w_h * max(0, q_h . k_i) */
/*
 * Flag OR-ed into either score mode: the quantized-query variant. Each head's
 * query is first converted to MXFP8 (per 32 channels an E8M0 scale 2^X with
 * X = floor(log2 amax) - 8, clamped to [-127, 127], -127 for a zero block;
 * values nearest-even E4M3FN of x * 2^-X, saturating at 448: the OCP MX rule
 * the keys follow as "standard MXFP4", [FP4] section "Le coût d'une entrée"),
 * and every 16 entries x 16 heads are contracted by one block-scaled FP8 x FP4
 * matrix instruction that reads the cached keys as they are. The scores are
 * those of the quantized query, up to that instruction's accumulation: within
 * each group of 8 consecutive channels, product bits more than 13 binades
 * below the group's largest product are dropped (toward zero). A faster
 * variant, not the exact path.
 */
#define CSA2_SCORE_QMX8    0x100

/* CSA2 layer modes ([CS] section "L'architecture : trois leviers contre le cache") */
#define CSA2_FULL     0   /* own indexer pass over every entry, new top-k */
#define CSA2_REINDEX  1   /* rescore the Full layer's candidate pool, new top-k */
#define CSA2_REUSE    2   /* reuse the previous layer's indices */

/* layout constants ([FP4] section "Le coût d'une entrée") */
#define CSA2_LATENT_CH           512
#define CSA2_LATENT_BLOCK        16
#define CSA2_MAIN_ROW_BYTES      288   /* 256 B of E2M1 codes + 32 B of E4M3 scales */
#define CSA2_INDEXER_CH          128
#define CSA2_INDEXER_BLOCK       32
#define CSA2_INDEXER_CODE_BYTES  64    /* E2M1 codes */
#define CSA2_INDEXER_SCALE_BYTES 4     /* E8M0 scales, kept in a separate array */

/* limits of this build */
#define CSA2_MAX_K               2048   /* top-k of a Full/Reindex layer (512 in the pages) */
#define CSA2_MAX_POOL            16384  /* hierarchical candidate pool ([CS], same section) */
#define CSA2_MAX_INDEXER_HEADS   16
#define CSA2_MAX_HEADS           128    /* query heads of the attention */
#define CSA2_MAX_RATIO           16
#define CSA2_MAX_BATCH           1024   /* sequences per indexer / decode call */

/*
 * Cache write: ratio-m merge, then FP4 packing of the latent and the indexer key.
 *
 * Follows [TF] section "Mécanismes de compression du KV-Cache" (m consecutive
 * positions fused with learned per-channel weights), [FP4] section "Le compte
 * par couche" (one entry per m tokens) and [FP4] section "Le coût d'une entrée"
 * (latent: E2M1 + one E4M3 scale per 16 channels; key: E2M1 + one E8M0 scale
 * per 32 channels).
 *
 *   x_lat  bf16 [B][T][512]   hidden latent rows of B sequences (row b*T + t = token t of
 *                             sequence b; T is the row stride, the longest sequence)
 *   x_idx  bf16 [B][T][128]   hidden indexer-key rows, same layout
 *   w_lat  f32  [m][512]      merge weights, already normalised over the m positions
 *   w_idx  f32  [m][128]
 *   n_tokens          i64 [B] or NULL: tokens of sequence b (clamped to [0, T]); NULL = T each
 *   out_entry_offset  i64 [B] or NULL: cache row of sequence b's first entry;
 *                     NULL = b * floor(T/m). With both, a ragged batch is written in one call
 *                     into one preallocated cache (the caller keeps the rows of different
 *                     sequences apart).
 *   kv     u8   [rows][288]   out: entry i of sequence b goes to row out_entry_offset[b] + i:
 *                             256 code bytes (channel 2j in the low nibble of byte j) then 32
 *                             E4M3FN scale bytes (block b covers channels 16b..16b+15)
 *   ik     u8   [rows][64]    out: indexer-key codes, same nibble order and rows
 *   iks    u8   [rows][4]     out: E8M0 scale bytes of the 4 blocks of 32 channels
 * Sequence b gets E_b = floor(n_b/m) entries; a trailing partial group is not written.
 *
 * Merge, per channel c: acc = w[0][c]*x[m*i][c], then acc = acc + w[j][c]*x[m*i+j][c]
 * for j = 1..m-1, each product and sum rounded to float32 (no fused multiply-add).
 * Latent block: s = E4M3FN(amax/6) (correctly rounded float32 division, nearest-even,
 * saturating at 448); codes = E2M1 nearest-even of the float32 quotient x/s, sign bit
 * from x; s == 0 gives all codes 0. Key block: X = floor(log2 amax) - 2, byte X+127
 * clamped to [0,254]; codes = E2M1 of x*2^-X; amax == 0 gives byte 0 and codes 0.
 * Errors: NULL pointer, B outside [1, 65535], T < 0, m outside [1, CSA2_MAX_RATIO],
 * misalignment (16 bytes; iks 4). The token counts and offsets are device data and are
 * not checked on the host: rows they name must lie inside the caller's buffers.
 */
int csa2_cache_write(const uint16_t* x_lat, const uint16_t* x_idx,
                     const float* w_lat, const float* w_idx,
                     int B, int64_t T, int m,
                     const int64_t* n_tokens, const int64_t* out_entry_offset,
                     uint8_t* kv, uint8_t* ik, uint8_t* iks, void* stream);

/*
 * Decode-time append: one new token per sequence ([FP4] section "Le compte par
 * couche": one entry per m tokens; the tokens of a group not yet complete wait
 * in a per-sequence stage, as in [CS] section "L'architecture : trois leviers
 * contre le cache", where the newest tokens are covered by the window).
 *
 *   x_lat, x_idx   bf16 [B][512], [B][128]: this step's token of each sequence
 *   w_lat, w_idx   the merge weights, as in csa2_cache_write
 *   stage_lat      bf16 [B][m-1][512], stage_idx bf16 [B][m-1][128]: in/out, the
 *                  staged tokens of each sequence's incomplete group (NULL when m == 1)
 *   stage_count    i32 [B] in/out: staged tokens, 0 <= stage_count[b] < m
 *   entry_offset   i64 [B]: first cache row of sequence b
 *   n_entries      i32 [B] in/out: entries written so far
 *   capacity       i64 [B]: cache rows reserved for sequence b (rows entry_offset[b] ..
 *                  entry_offset[b] + capacity[b] - 1); a ragged layout gives each its own
 *   kv, ik, iks    the cache (as in csa2_cache_write)
 *   dropped        i32 [B] out, or NULL: 1 where a completed group found the
 *                  sequence full (n_entries[b] >= capacity[b]) and was discarded
 * When stage_count[b] + 1 < m the token is staged at row stage_count[b] and
 * stage_count[b] grows by one. Otherwise the m - 1 staged tokens and this one
 * are merged and packed exactly as csa2_cache_write packs tokens m*i .. m*i+m-1
 * into cache row entry_offset[b] + n_entries[b]; n_entries[b] grows by one and
 * stage_count[b] returns to 0. T tokens appended one call at a time therefore
 * leave the same floor(T/m) entries as one csa2_cache_write of the T tokens,
 * and the last T mod m tokens in the stage. A stage count outside [0, m-1] is
 * taken as m - 1.
 * Errors: NULL pointer, B < 1 or B > CSA2_MAX_BATCH, m outside [1, CSA2_MAX_RATIO],
 * misalignment (16 bytes; iks 4; stage_count, n_entries, dropped 4).
 */
int csa2_cache_append(const uint16_t* x_lat, const uint16_t* x_idx,
                      const float* w_lat, const float* w_idx, int B, int m,
                      uint16_t* stage_lat, uint16_t* stage_idx, int32_t* stage_count,
                      const int64_t* entry_offset, int32_t* n_entries, const int64_t* capacity,
                      uint8_t* kv, uint8_t* ik, uint8_t* iks, int32_t* dropped, void* stream);

/*
 * Sliding-window cache ([FP4] section "La contrepartie : la fenêtre glissante":
 * each layer keeps a window in FP8 of 512 + 512/16 bytes per token; [CS] section
 * "L'architecture : trois leviers contre le cache": 128 tokens).
 *
 *   x_lat   bf16 [B][T][512]   latent rows of tokens pos0[b] .. pos0[b] + T - 1
 *   pos0    i64 [B]            position of each sequence's first row here
 *   win     u8 [B][128][544]   in/out: the ring; token t lives in row t mod 128 as 512
 *                              E4M3FN values (channel c at byte c) then 32 E8M0 scale
 *                              bytes (block b = channels 16b..16b+15)
 * Only the last min(T, 128) rows of each sequence are written (earlier ones would
 * be overwritten in the ring). Block scale: the smallest power of two 2^X with
 * amax <= 448 * 2^X (byte X + 127, clamped to [0, 254]; byte 0 and zero values
 * for an all-zero block); values: E4M3FN nearest-even of x * 2^-X with the sign
 * of x, so no value saturates. Values below 2^-110 in magnitude may flush to zero.
 * Errors: NULL pointer, B < 1, T < 0, misalignment (16 bytes).
 */
int csa2_swa_write(const uint16_t* x_lat, int B, int64_t T, const int64_t* pos0, uint8_t* win, void* stream);

/*
 * Attention over the window, merged with the sparse branch's result already in
 * out / lse (one softmax over the union of the selected entries and the window):
 * o = (e^lse o + e^lse_w o_w) / (e^lse + e^lse_w), lse = log(e^lse + e^lse_w).
 *
 *   win     the ring (see csa2_swa_write); n_win i32 [B]: valid rows 0 .. n_win[b]-1
 *           (min(tokens written, 128)); values outside [0, 128] are clamped
 *   q       bf16 [B][H][512], softmax_scale tau: as in csa2_sparse_attention
 *   out     f32 [B][H][512] in/out; lse f32 [B][H] in/out (-inf: no sparse entry)
 * Needs no workspace. Errors: NULL pointer, B < 1 or B > CSA2_MAX_BATCH, H outside
 * [1, CSA2_MAX_HEADS], misalignment (16 bytes).
 */
int csa2_swa_attention(const uint8_t* win, const int32_t* n_win, const uint16_t* q, int B, int H,
                       float softmax_scale, float* out, float* lse, void* stream);

/*
 * Indexer pass and top-k ([FP4] section "Les ingrédients": the indexer key scores
 * positions; [CS] section "L'architecture : trois leviers contre le cache": new
 * top-512 per Full layer, hierarchical pool of at most 16384 candidates; [F24]
 * section "Tre meccanismi al posto di un solo trucco": deeper layers rescore only
 * the pool).
 *
 *   ik, iks        the cache's indexer rows (see csa2_cache_write)
 *   entry_offset   i64 [B]  first cache row of sequence b
 *   n_entries      i32 [B]  entries of sequence b; positions are 0..n_entries[b]-1
 *   B, max_n       host ints; 1 <= B <= CSA2_MAX_BATCH; 0 <= max_n <= 2^26; max_n >= every n_entries[b]
 *                  (rows at positions >= max_n are not scored)
 *   q_idx          bf16 [B][Hi][128] indexer queries; w f32 [B][Hi] head weights
 *                  (NULL = all 1; ignored by CSA2_SCORE_DOT)
 *   Hi, score_mode 1 <= Hi <= 16; CSA2_SCORE_DOT needs Hi == 1; either mode may
 *                  carry CSA2_SCORE_QMX8
 *   cand           i32 [B][cand_stride] or NULL. NULL: score every entry (Full).
 *                  Otherwise score only the listed positions (Reindex). A row is
 *                  meant to list distinct positions in ascending order, as a pool
 *                  is written: an entry is used only when it lies in
 *                  [0, n_entries[b]) and is greater than every in-range entry
 *                  before it in the row; others (-1 padding, out-of-order or
 *                  repeated positions) are skipped. cand_stride <= CSA2_MAX_POOL.
 *   k              1 <= k <= CSA2_MAX_K
 *   topk           out i32 [B][k]: the k best positions by (score descending,
 *                  position ascending), written in ascending position order,
 *                  -1 padded when fewer than k candidates exist
 *   pool_k, pool   0/NULL, or 1 <= pool_k <= CSA2_MAX_POOL with pool out i32
 *                  [B][pool_k]: the best pool_k positions (same order rule, ascending,
 *                  -1 padded); topk is then chosen from the pool. Full only.
 *   scores_out     NULL, or out f32 [B][max_n] (Full) / [B][cand_stride] (Reindex):
 *                  the float32 scores, for inspection
 *   workspace      csa2_indexer_workspace_bytes(B, max_n, k, pool_k, cand_stride) bytes
 *                  (cand_stride 0 without a candidate list)
 * Selection: with k <= 512 every score workgroup keeps the keys above a local
 * cutoff and a finish merges them (the pool the same way from a second list);
 * k > 512 takes a threshold-bin pass. Both are exact.
 */
size_t csa2_indexer_workspace_bytes(int B, int64_t max_n, int k, int pool_k, int cand_stride);
int csa2_indexer_topk(const uint8_t* ik, const uint8_t* iks,
                      const int64_t* entry_offset, const int32_t* n_entries,
                      int B, int64_t max_n,
                      const uint16_t* q_idx, const float* w, int Hi, int score_mode,
                      const int32_t* cand, int cand_stride,
                      int k, int32_t* topk, int pool_k, int32_t* pool,
                      float* scores_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Sparse attention of all query heads over the dequantized latent at the selected
 * positions ([TF] section "Mécanismes de compression du KV-Cache", item 1: one
 * 512-d latent shared by keys and values across heads; [FP4] section "Les
 * ingrédients": the main-cache latent serves attention).
 *
 *   kv             the cache's main rows (see csa2_cache_write)
 *   entry_offset   i64 [B]; n_entries i32 [B] (indices >= n_entries[b] are skipped)
 *   idx            i32 [B][k] positions, -1 = skip; 1 <= k <= CSA2_MAX_K
 *   q              bf16 [B][H][512]; 1 <= H <= CSA2_MAX_HEADS
 *   softmax_scale  tau: logit = tau * (q_h . c_i)
 *   out            out f32 [B][H][512]: o_h = sum_i softmax_i * c_i (0 if no valid index)
 *   lse            out f32 [B][H] or NULL: log sum_i exp(logit_i) (-inf if none)
 *   workspace      csa2_attention_workspace_bytes(B, H, k) bytes
 */
size_t csa2_attention_workspace_bytes(int B, int H, int k);
int csa2_sparse_attention(const uint8_t* kv, const int64_t* entry_offset, const int32_t* n_entries,
                          const int32_t* idx, int k, const uint16_t* q, int B, int H,
                          float softmax_scale, float* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * One CSA2 layer of a decode step ([CS] section "L'architecture : trois leviers
 * contre le cache": Full = own indexer and new top-k; Reindex = rescoring of the
 * pool against the shared cache; Reuse = indices taken over).
 *
 *   mode CSA2_FULL:    indexer over every entry -> pool (if pool_k > 0) -> topk (out),
 *                      pool (out) -> attention
 *   mode CSA2_REINDEX: pool (in, [B][pool_k]) rescored with q_idx/w -> topk (out)
 *                      -> attention
 *   mode CSA2_REUSE:   topk (in) -> attention; q_idx, w, pool unused
 * Arguments mean what they mean in csa2_indexer_topk and csa2_sparse_attention.
 * workspace: csa2_decode_workspace_bytes(B, max_n, H, k, pool_k) bytes (one
 * buffer serves all three modes). With k <= 512 (and max_n > 16384 for a Full
 * layer) a layer is two launches: the scoring pass, then the attention, whose
 * workgroups first finish the top-k themselves (topk is still written); a Full
 * layer's pool is finished by B more workgroups of that launch. The workspace
 * then also holds scratch rows for every such workgroup (about 12 * max(max_n,
 * pool_k) bytes each), unless those would exceed 4 GiB, in which case the
 * finishes run as launches of their own.
 */
size_t csa2_decode_workspace_bytes(int B, int64_t max_n, int H, int k, int pool_k);
int csa2_decode_layer(int mode,
                      const uint8_t* kv, const uint8_t* ik, const uint8_t* iks,
                      const int64_t* entry_offset, const int32_t* n_entries,
                      int B, int64_t max_n,
                      const uint16_t* q_idx, const float* w, int Hi, int score_mode,
                      const uint16_t* q, int H, float softmax_scale,
                      int k, int pool_k, int32_t* pool, int32_t* topk,
                      float* out, float* lse,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * csa2_decode_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc). It allocates nothing: its scratch is a
 * static device array of CSA2_NOALLOC_SCRATCH_BYTES that each device the
 * library runs on holds until the process ends. Arguments, outputs and errors
 * are those of csa2_decode_layer (minus workspace and ws_bytes), with the same
 * results. The fused two-launch plan is taken when its scratch fits the array,
 * else the plan of separate indexer and attention launches; a call whose
 * indexer scratch alone exceeds the array returns CSA2_ERR_WORKSPACE before
 * any launch. The scratch needs no initialisation (every kernel writes what it
 * reads), but all calls on one device share it: calls that overlap on a device
 * (on different streams, or from different threads without ordering) race and
 * must not be made.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa2_decode_layer_noalloc(int mode,
                              const uint8_t* kv, const uint8_t* ik, const uint8_t* iks,
                              const int64_t* entry_offset, const int32_t* n_entries,
                              int B, int64_t max_n,
                              const uint16_t* q_idx, const float* w, int Hi, int score_mode,
                              const uint16_t* q, int H, float softmax_scale,
                              int k, int pool_k, int32_t* pool, int32_t* topk,
                              float* out, float* lse, void* stream);

/*
 * Multi-query (prefill) sparse attention over the same cache: Tq query tokens
 * per sequence, each with its own indexer query and its own causal top-k (the
 * layer mode Full of [CS] section "L'architecture : trois leviers contre le
 * cache", applied to every query token). Query t of sequence b, at token
 * position pos[b][t], sees the entries its token has completed: the first
 * min(n_entries[b], floor((pos + 1) / m)) of the sequence ([FP4] section "Le
 * compte par couche": one entry per m tokens; the rest is in the window).
 *
 *   pos      i64 [B][Tq] token positions (negative: no entry visible)
 *   q_idx    bf16 [B][Tq][Hi][128], w f32 [B][Tq][Hi] or NULL: indexer queries
 *   q        bf16 [B][Tq][H][512]: attention queries
 *   topk     out i32 [B][Tq][k]; out f32 [B][Tq][H][512]; lse f32 [B][Tq][H] or NULL
 * The other arguments mean what they mean in csa2_decode_layer (CSA2_FULL, no
 * pool). The queries run as one decode batch of B * Tq sequences sharing the
 * cache rows, so 1 <= B * Tq <= CSA2_MAX_BATCH.
 * workspace: csa2_prefill_workspace_bytes(B, Tq, max_n, H, k) bytes.
 */
size_t csa2_prefill_workspace_bytes(int B, int Tq, int64_t max_n, int H, int k);
int csa2_prefill_layer(const uint8_t* kv, const uint8_t* ik, const uint8_t* iks,
                       const int64_t* entry_offset, const int32_t* n_entries, int B, int64_t max_n,
                       int m, int Tq, const int64_t* pos,
                       const uint16_t* q_idx, const float* w, int Hi, int score_mode,
                       const uint16_t* q, int H, float softmax_scale, int k,
                       int32_t* topk, float* out, float* lse,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * Host-only byte accounting ([FP4] sections "Le coût d'une entrée" and "Le
 * compte par couche"): sum over layers of (entry bytes of the latent + entry
 * bytes of the key) / ratio, where an entry of ch channels with block blk and
 * sbytes scale bytes per block costs ch/2 + (ch/blk)*sbytes (blk == 0: no
 * scales). Returns a negative value on bad arguments.
 */
double csa2_bytes_per_token(const int* ratios, int n_layers,
                            int lat_ch, int lat_blk, int lat_sbytes,
                            int idx_ch, int idx_blk, int idx_sbytes);

/*
 * Measurement hook (not part of the method): two hipEvent_t handles (as void*)
 * that the next Full-pass call of this thread (csa2_indexer_topk without cand,
 * or csa2_decode_layer in CSA2_FULL mode) records on its stream immediately
 * before and after the launch of its indexer scoring kernel, so a caller can
 * time that kernel alone. One-shot: the handles are dropped by that call. Both
 * NULL clears them. The events must be created by the caller (hipEventCreate).
 */
int csa2_set_profile_events(void* before_score, void* after_score);

/* Message of the calling thread's last non-zero status ("" if none). */
const char* csa2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2FP4_H */
