/*
 * dllm.h - C ABI of the Flash-Cache per-layer denoising-step library (gfx950).
 *
 * Pages cited:
 *   [FD]  "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Fast,
 *         Memory-Efficient Diffusion LLMs" (paper summary page): sections
 *         核心方法 (core method), 方法步骤详情 (Algorithm 2, formula (2)),
 *         研究动机 (motivation), 技术新颖性 (novelty).
 *   [AIP] "Flash-dLLM 是什麼？擴散語言模型推論快 11 倍" (aiposthub explainer):
 *         Flash-Cache, selective refresh and Flash-Verify sections.
 *   [FST] Fast-dLLM article (senqingzn.com), section 并行解碼新策略 (confidence-aware
 *         parallel decoding).
 *
 * One layer of one denoising step is
 *     dllm_map_slots            logical position -> flat cache row of each query row
 *     dllm_qkv_rope_cachewrite  x W^T, rotary embedding, q out, K/V into the cache
 *     dllm_sched_attention      paged bidirectional attention + formula (2) term
 * and after the last layer of the step
 *     dllm_topk_tracked         next step's tracked positions
 * dllm_build_block_table sets up (and validates) the page table once.
 * Decode side (after the model's head): dllm_decode_commit / dllm_decode_verify,
 * or their pieces dllm_confidence_argmax, dllm_confidence_commit, dllm_verify_accept.
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller allocates and owns every buffer; the library never
 *     allocates or frees device memory and keeps no state between calls.  The
 *     *_workspace() queries report the scratch memory a call needs (a pure
 *     function of the shape arguments; 0 for most shapes); a NULL workspace is
 *     accepted when the query returns 0.  Workspace contents need no
 *     initialisation, and two calls in flight at once must not share one.
 *   - Pointers named "host" are host memory; every other pointer is device
 *     memory of the current HIP device.  All device work is enqueued on
 *     `stream` and is asynchronous unless stated; buffers must stay valid until
 *     the stream has executed the work.
 *   - Errors: the return value is the only error channel.  Argument errors the
 *     host can see return before any work is enqueued and leave every output
 *     untouched.  Device-side indices that are out of range (a page id outside
 *     the pool, a slot outside the cache) are never dereferenced: the affected
 *     key is treated as hidden, the affected row is not written.
 *   - Dtypes: DLLM_BF16 means x, W, the caches, q and o are bf16 (accumulation
 *     in fp32); DLLM_F32 means they are all fp32; DLLM_BF16_E4M3KV is DLLM_BF16
 *     with one-byte E4M3 caches (see below).
 *   - Layouts are row-major and dense.  A cache is [cache_rows, n_heads*head_dim]:
 *     one row per token slot, head h in columns h*head_dim .. h*head_dim+head_dim-1
 *     ([FD] 方法步骤详情 step 1: the flat per-layer cache of B*N_max rows).
 *     Slot s lives in physical page s / page_size.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DLLM_OK = 0,
    DLLM_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent sizes */
    DLLM_ERR_UNSUPPORTED = -2,   /* a shape or dtype this library has no kernel for */
    DLLM_ERR_OUT_OF_RANGE = -3,  /* an index outside its table, pool or cache; a duplicate slot */
    DLLM_ERR_HIP = -4            /* a HIP runtime call or launch failed */
} dllm_status;

/*
 * DLLM_BF16_E4M3KV: bf16 as DLLM_BF16 for x, W, q and o, with the K and V
 * caches held as one byte per element: OCP 8-bit float E4M3 codes (unit scale;
 * stored values rounded to nearest even, magnitudes beyond 448 saturating to
 * 448).  [FD] paper summary page, 未来方向 item (3): fused kernels over a
 * low-bit KV cache.  Accepted by dllm_qkv_rope_cachewrite(_paged) and
 * dllm_sched_attention (head_dim 128); the attention decodes codes exactly.
 */
typedef enum { DLLM_F32 = 0, DLLM_BF16 = 1, DLLM_BF16_E4M3KV = 2 } dllm_dtype;

/* Text for a status code (static storage). */
const char* dllm_status_string(int status);
/* Library ABI version, major * 100 + minor. */
int dllm_version(void);

/*
 * a0, set-up: block table over one shared page pool, and optionally the cache
 * slot of host-given query rows.  [FD] 核心方法 / 技术新颖性: a block table maps
 * each sequence's query blocks to its KV blocks; [FD] 方法步骤详情 step 1: the
 * cache is allocated once and never reallocated.
 *
 *   n_seq, page_size, pool_pages, max_pages  sizes (page_size > 0)
 *   seq_pages  host int32[n_seq]     pages taken by each sequence (<= max_pages)
 *   pool_perm  host int32[pool_pages] a permutation of 0..pool_pages-1; sequence
 *              b takes the next seq_pages[b] entries of it, in order
 *   page_table device int32[n_seq*max_pages] out: physical page of logical page j
 *              of sequence b at [b*max_pages + j], -1 past the sequence's pages
 *   n_rows, cu_q (host int32[n_seq+1]), q_logical (host int32[n_rows]), slot
 *              (device int32[n_rows]): optional (all NULL / 0 or all set); the
 *              slot of row r of sequence b is page_table[b][l/page_size]*page_size
 *              + l%page_size with l = q_logical[r]
 * Errors: INVALID_ARG for null/negative/inconsistent arguments or a cu_q that is
 * not non-decreasing from 0 to n_rows; OUT_OF_RANGE when sum(seq_pages) >
 * pool_pages, seq_pages[b] > max_pages, pool_perm is not a bijection, a logical
 * position lies beyond its sequence's pages, or two rows share one slot.
 * Blocking: returns after the copies to the device have completed.
 */
int dllm_build_block_table(int n_seq, int page_size, int pool_pages, int max_pages,
                           const int32_t* seq_pages, const int32_t* pool_perm,
                           int32_t* page_table,
                           int n_rows, const int32_t* cu_q, const int32_t* q_logical,
                           int32_t* slot, hipStream_t stream);

/*
 * a0, per step, on the device: cache slot of each query row from its logical
 * position (same formula as above).  cu_q int32[n_seq+1], q_logical int32[n_rows],
 * page_table int32[n_seq*max_pages] are device arrays; slot int32[n_rows] out.
 * A row whose logical position is negative, beyond max_pages*page_size, on a -1
 * table entry or on a page >= pool_pages gets slot -1 (the cache write then
 * skips it).  Duplicate slots are not detected here (dllm_build_block_table
 * checks host-side row sets).  Asynchronous.
 */
int dllm_map_slots(int n_seq, int n_rows, int page_size, int max_pages, int pool_pages,
                   const int32_t* cu_q, const int32_t* q_logical, const int32_t* page_table,
                   int32_t* slot, hipStream_t stream);

/*
 * a1-a3: fused QKV projection + rotary embedding + cache write.  [FD] 核心方法:
 * one kernel projects, rotates and writes K/V straight into the preallocated
 * flat cache with no intermediate tensors in memory; [FD] 研究动机: the unfused
 * four-kernel pipeline is bound by memory traffic.
 *
 *   n_rows R (>= 0), d_model (input width, multiple of 64), n_heads H, head_dim D
 *   (64 or 128; H*D a multiple of 128), rope_base > 0
 *   x        [R, d_model]           layer input rows (query rows of this step)
 *   w_qkv    [3*H*D, d_model]       out x in: rows 0..HD-1 give Q, HD..2HD-1 K,
 *                                   2HD..3HD-1 V; head h is rows h*D..h*D+D-1 of each
 *   pos      int32[R]               rotary position of each row
 *   slot     int32[R]               cache row written by each row (-1: none)
 *   q_out    [R, H*D]               out: rotated q
 *   k_cache, v_cache [cache_rows, H*D]  rows slot[r] overwritten with rotated k
 *                                   and with v; no other row is touched
 * Rotary embedding is rotate-half: for i < D/2, theta_i = rope_base^(-2i/D) and
 * the pair (t_i, t_{i+D/2}) turns by pos*theta_i.  Results are rounded once to
 * the output dtype.  Slots of one call must be pairwise distinct.
 * Errors: INVALID_ARG, UNSUPPORTED (D, H*D, d_model, dtype).
 */
size_t dllm_qkv_rope_cachewrite_workspace(dllm_dtype dt, int n_rows, int d_model, int n_heads,
                                          int head_dim);
int dllm_qkv_rope_cachewrite(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim,
                             float rope_base, const void* x, const void* w_qkv,
                             const int32_t* pos, const int32_t* slot, void* q_out,
                             void* k_cache, void* v_cache, int64_t cache_rows,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * a0-a3 in one call: dllm_qkv_rope_cachewrite where each row's cache slot is
 * formed on the device from its logical position and the block table, with
 * dllm_map_slots's rule (slot = page_table[b][l/page_size]*page_size +
 * l%page_size for row r of sequence b, l = q_logical[r]; -1, and no write,
 * for a negative or out-of-table position, a -1 entry or a page >=
 * cache_rows/page_size).  [FD] 核心方法: K/V go straight into the paged cache
 * from the projection kernel.  For bf16 row counts the weight-streaming
 * kernels take (n_rows <= 128, and the mid-size shapes up to a few hundred
 * rows) the mapping runs inside the projection kernel (no separate launch);
 * for the GEMM tilings it is a launch of its own ahead of the projection.
 *
 *   n_seq (1..1024), cu_q int32[n_seq+1], q_logical int32[n_rows],
 *   page_table int32[n_seq*max_pages] (device), page_size > 0
 *   slot     int32[n_rows]          out: the slot each row was written to (-1: none)
 *   other arguments as dllm_qkv_rope_cachewrite
 * Errors: as dllm_qkv_rope_cachewrite; INVALID_ARG for n_seq < 1, max_pages
 * < 1, page_size < 1 or a null pointer; UNSUPPORTED for n_seq > 1024.
 */
int dllm_qkv_rope_cachewrite_paged(dllm_dtype dt, int n_seq, int n_rows, int d_model, int n_heads,
                                   int head_dim, float rope_base, const void* x, const void* w_qkv,
                                   const int32_t* pos, const int32_t* cu_q, const int32_t* q_logical,
                                   const int32_t* page_table, int max_pages, int page_size,
                                   int32_t* slot, void* q_out, void* k_cache, void* v_cache,
                                   int64_t cache_rows, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * The unfused comparison arm of a1-a3 (three launches, intermediates in
 * memory), kept to measure what the fused call saves.  [FD] 研究动机: the
 * four-kernel chain (projection, rotary, cache write, attention) moves every
 * intermediate through global memory; 核心方法: the fused kernel removes that.
 * bf16 only (UNSUPPORTED otherwise).
 *
 * dllm_qkv_project: qkv_out [R, 3*H*D] = x w_qkv^T, unrotated, row r holding
 *   q | k | v (shapes and errors as dllm_qkv_rope_cachewrite).
 * dllm_rope_apply: rotate-half rotary embedding (as dllm_qkv_rope_cachewrite)
 *   of qkv's q part into q_out [R, H*D] and of its k part in place; pos
 *   int32[R].  Errors: INVALID_ARG (negative sizes, rope_base <= 0, null
 *   pointers), UNSUPPORTED (head_dim other than 64 or 128).
 * dllm_cache_write: qkv's k and v parts of row r to row slot[r] of k_cache and
 *   v_cache ([cache_rows, H*D]); rows whose slot is negative or >= cache_rows
 *   are skipped.  Errors: INVALID_ARG, UNSUPPORTED (H*D not a multiple of 8).
 * All three are asynchronous on `stream`.
 */
int dllm_qkv_project(dllm_dtype dt, int n_rows, int d_model, int n_heads, int head_dim,
                     const void* x, const void* w_qkv, void* qkv_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);
int dllm_rope_apply(dllm_dtype dt, int n_rows, int n_heads, int head_dim, float rope_base,
                    const int32_t* pos, void* qkv, void* q_out, hipStream_t stream);
int dllm_cache_write(dllm_dtype dt, int n_rows, int n_heads, int head_dim, const void* qkv,
                     const int32_t* slot, void* k_cache, void* v_cache, int64_t cache_rows,
                     hipStream_t stream);

/*
 * a4-a5: block-table scheduled bidirectional attention over the paged cache,
 * every sequence's query rows in one launch with no padding, plus one layer's
 * term of the tracked-set score.  [FD] 核心方法 / 技术新颖性: variable-length
 * query blocks aligned to their KV blocks through the block table, mixing
 * cache-phase windows and full refreshes; [FD] 方法步骤详情 step 2 (attention
 * over the full cache) and step 4 (formula (2)).
 *
 *   n_seq B, n_rows R, n_heads H, head_dim D (bf16: 128; f32: 64 or 128), page_size
 *   (16), max_kv (host upper bound of kv_len, > 0)
 *   q          [R, H*D]            rotated queries; rows of sequence b are
 *                                  cu_q[b] .. cu_q[b+1]-1 (int32[B+1], device)
 *   k_cache, v_cache [cache_rows, H*D]  written by dllm_qkv_rope_cachewrite
 *   page_table int32[B*max_pages]  as built by dllm_build_block_table
 *   kv_len     int32[B]            keys of sequence b: logical 0..kv_len[b]-1
 *   mask_bits  uint32[mask_words] or NULL (all keys visible).  If set, row i
 *              (0-based within sequence b) sees key j iff bit j%32 of word
 *              mask_off[b] + i*ceil(kv_len[b]/32) + j/32 is 1; mask_off int64[B]
 *   mass_count int32[B] or NULL    the first mass_count[b] (<= max_mass_rows <= 128)
 *              rows of sequence b are the masked-window rows of formula (2):
 *              the caller orders each sequence's rows with its window rows
 *              first (the order is otherwise free; the rows after them do not
 *              enter the score).  A count outside 0..min(max_mass_rows, rows
 *              of b) is taken as the nearest end of that range; a sequence
 *              with no score rows forms no term
 *   mass_accum float[B*H*n_cap]    per-head running score: for each head h,
 *              mass_accum[(b*H + h)*n_cap + i] += (1/(H*m_b)) * sum over the
 *              window rows of head h's probability of key i (m_b =
 *              mass_count[b]); keys i >= n_cap are not recorded.  Summed over
 *              heads (dllm_topk_tracked does) and over layers (by calling once
 *              per layer) this is formula (2)'s a_i.
 *   mass_overwrite  nonzero: store the term (= instead of +=), for the first
 *              scoring layer of a step, so the score needs no clearing between
 *              steps; entries at or past kv_len[b], and every entry of a
 *              sequence with no score rows, are then left as they were
 *   o          [R, H*D]            out: attention output
 * Scores are q.k/sqrt(D); a row that sees no key outputs zeros.  When the
 * batch has too few (sequence, head) pairs to fill the GPU, keys are split
 * over workgroups and a second kernel merges them (workspace: per split, bf16
 * partial outputs and row statistics).  Otherwise, when a score is formed
 * (bf16 paths), the workspace holds the window rows' bf16 probabilities of
 * every key tile (B*H*ceil(max_kv/64)*max_mass_rows*(128+4) bytes), so the
 * score needs no second read of K.  dllm_sched_attention_workspace reports
 * the bytes a call with these sizes needs (max_mass_rows = 0: no score; the
 * fp32 path needs none); the call checks workspace_bytes against it.
 * Errors: INVALID_ARG (also cache_rows < 16, a short workspace), UNSUPPORTED
 * (dtype/D/page_size/n_seq > 1024/max_pages > 1024/bf16 score over more than
 * 8704 keys).
 */
size_t dllm_sched_attention_workspace(dllm_dtype dt, int n_seq, int n_rows, int n_heads,
                                      int head_dim, int max_kv, int n_cap, int max_mass_rows);
int dllm_sched_attention(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim,
                         int page_size, int max_kv, const void* q, const int32_t* cu_q,
                         const void* k_cache, const void* v_cache, int64_t cache_rows,
                         const int32_t* page_table, int max_pages, const int32_t* kv_len,
                         const uint32_t* mask_bits, const int64_t* mask_off, int64_t mask_words,
                         const int32_t* mass_count, int max_mass_rows, float* mass_accum,
                         int mass_overwrite, int n_cap, void* o, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * dllm_sched_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * allocation): no workspace argument.  The scratch memory that
 * dllm_sched_attention takes from its workspace (split partials, the score's
 * window-row probabilities) comes from a static device array of
 * DLLM_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU, held from the library's
 * first use on that GPU until the process ends.  Arguments, results and
 * errors as dllm_sched_attention; a call whose workspace query
 * (dllm_sched_attention_workspace with the same sizes) exceeds the array
 * returns DLLM_ERR_UNSUPPORTED before any work is enqueued (for example a
 * batch of 32 sequences of 2048 keys with 32 score rows each needs 132 MiB),
 * and DLLM_ERR_HIP if the array's device address cannot be obtained.  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (no call needs it cleared): calls
 * that overlap on one GPU (other streams, other host threads) race on it and
 * must be serialised by the caller.
 */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dllm_sched_attention_noalloc(dllm_dtype dt, int n_seq, int n_rows, int n_heads, int head_dim,
                                 int page_size, int max_kv, const void* q, const int32_t* cu_q,
                                 const void* k_cache, const void* v_cache, int64_t cache_rows,
                                 const int32_t* page_table, int max_pages, const int32_t* kv_len,
                                 const uint32_t* mask_bits, const int64_t* mask_off, int64_t mask_words,
                                 const int32_t* mass_count, int max_mass_rows, float* mass_accum,
                                 int mass_overwrite, int n_cap, void* o, hipStream_t stream);

/*
 * a6: per-sequence top-k of the accumulated score over eligible positions.
 * [FD] 方法步骤详情 step 4: the top-k decoded tokens by formula (2), with the
 * newly decoded tokens, form the next tracked set (the caller adds the new
 * ones; `eligible` excludes them).
 *
 *   mass     float[B*H*n_cap] per-head scores as accumulated by
 *                             dllm_sched_attention; the score of position i is
 *                             the fp32 sum over h = 0..H-1 in that order (read;
 *                             zeroed afterwards if clear_mass != 0)
 *   eligible uint8[B*n_cap]   nonzero = candidate
 *   idx      int32[B*k]       out: positions, highest score first, ties to the
 *                             lower position, -1 padding
 *   val      float[B*k]       out: their scores (0 padding)
 *   count    int32[B]         out: min(k, number of candidates)
 * Limits: 1 <= k <= 256, n_cap <= 4096.
 */
int dllm_topk_tracked(int n_seq, int n_heads, int n_cap, int k, float* mass,
                      const uint8_t* eligible, int32_t* idx, float* val, int32_t* count,
                      int clear_mass, hipStream_t stream);

/*
 * Decode side, after the last layer of a step: one logits row per masked window
 * position (or per search position of a verify step).
 *
 * [FD] 方法步骤详情 step 2: the confidence of a position is the largest
 * probability of its predicted distribution, and positions whose confidence is
 * at least epsilon (0.9 in the pages) are decoded; [FST] = Fast-dLLM article,
 * 并行解碼新策略: a sequence where no position reaches epsilon decodes its most
 * confident position.  [FD] 方法步骤详情 step 3 (Flash-Verify): draft tokens
 * are accepted in position order while the draft equals the mask view's
 * predicted token and the mask view's confidence is at least gamma (0.8 in the
 * pages); the first position that fails ends acceptance for the sequence.
 *
 * Shared arguments:
 *   logits   [n_rows, row_stride] of dt (DLLM_BF16 or DLLM_F32); the first
 *            vocab entries of each row are read, which must be finite
 *   cu_rows  device int32[n_seq+1]: rows cu_rows[b] .. cu_rows[b+1]-1 belong
 *            to sequence b, in position order.  A malformed range (decreasing,
 *            or outside 0..n_rows) is clipped to 0..n_rows and, if still
 *            decreasing, treated as empty: no row outside 0..n_rows is touched.
 *   token    int32[n_rows]: the argmax token of each row (lowest id on ties)
 *   conf     float[n_rows]: its softmax probability, 1 / sum_x exp(l_x - max l),
 *            accumulated in fp32
 * Thresholds compare the fp32 confidence with the float threshold (>=).
 * Ties of the forced decode go to the lowest row.
 * The logits calls need workspace of dllm_confidence_workspace(n_rows, vocab)
 * bytes (16-byte aligned; a function of the two sizes only).
 * Errors: INVALID_ARG for null pointers, negative sizes, row_stride < vocab, a
 * dtype other than the two, or a short workspace; UNSUPPORTED when the launch
 * would exceed the grid limit.  Asynchronous.
 */
size_t dllm_confidence_workspace(int n_rows, int vocab);

/* Per row: token and conf. */
int dllm_confidence_argmax(dllm_dtype dt, int n_rows, int vocab, const void* logits, int64_t row_stride,
                           int32_t* token, float* conf, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Threshold rule on given confidences: commit uint8[n_rows] out (1 = decode
 * the row this step), n_commit int32[n_seq] out (rows committed per sequence;
 * at least 1 for a non-empty sequence). */
int dllm_confidence_commit(int n_seq, int n_rows, const int32_t* cu_rows, const float* conf, float eps,
                           uint8_t* commit, int32_t* n_commit, hipStream_t stream);

/* Verify scan on given predictions: draft int32[n_rows] (the draft view's
 * tokens), token/conf of the mask view; accept uint8[n_rows] out, n_accept
 * int32[n_seq] out (length of the accepted prefix of each sequence). */
int dllm_verify_accept(int n_seq, int n_rows, const int32_t* cu_rows, const int32_t* draft,
                       const int32_t* token, const float* conf, float gamma, uint8_t* accept,
                       int32_t* n_accept, hipStream_t stream);

/* Logits -> token, conf and the threshold rule in two launches. */
int dllm_decode_commit(dllm_dtype dt, int n_seq, int n_rows, const int32_t* cu_rows, int vocab,
                       const void* logits, int64_t row_stride, float eps, int32_t* token, float* conf,
                       uint8_t* commit, int32_t* n_commit, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Mask-view logits -> token, conf and the verify scan in two launches. */
int dllm_decode_verify(dllm_dtype dt, int n_seq, int n_rows, const int32_t* cu_rows, int vocab,
                       const void* logits, int64_t row_stride, const int32_t* draft, float gamma,
                       int32_t* token, float* conf, uint8_t* accept, int32_t* n_accept,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Tuning override, for tests and tuning runs; correct use needs none.  Forces
 * a kernel choice process-wide:
 *   knob "attn_splits": value a split count ("1" .. "1024"; capped at 16 and
 *       at the key tiles) for the bf16 dllm_sched_attention;
 *   knob "qkv_kernel": value "tiled", "gemm" or a tile shape ("g256x256",
 *       "g128x256", "g128x256o2", "g64x256", "g64x256o2", "g256x128",
 *       "g256x128o2", "g128x128", "g128x128o2") for projections of more than
 *       128 rows, where the shape allows it;
 *   value NULL or "" restores the automatic choice.
 * The first values come from the environment variables DLLM_ATTN_SPLITS and
 * DLLM_QKV_KERNEL, read once per process (at the first call that needs them
 * or at the first dllm_set_tuning).  A workspace query and the call it sizes
 * read the same stored value: change a knob only between such pairs.
 * Errors: INVALID_ARG for an unknown knob or value (nothing changes).
 */
int dllm_set_tuning(const char* knob, const char* value);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
