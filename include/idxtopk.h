/*
 * libidxtopk -- sparse-attention indexer top-k for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only; no framework types.
 *
 * Pages this interface follows:
 *   [ATOM-1473] ROCm/ATOM pull request 1473, "enable minimax m3 fp8 index cache
 *               and fuse index_score_kernel with partial_topk kernel";
 *   [SGL-37889] sgl-project/sglang pull request 37889, "[AMD] Enable GLM DSA
 *               prefill top-k to the v2 kernel";
 *   [ATOM-1282] ROCm/ATOM pull request 1282, "merge build sparse block into topk".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except `stream` is a DEVICE pointer to memory owned
 *   by the caller. The library never allocates, frees or synchronises. Each
 *   call enqueues at most two kernels on `stream` (a hipStream_t; NULL = the
 *   null stream) and returns without waiting.
 * - Strides are in elements (int64). Index, length and slot arrays are int32.
 * - fp8 data are OCP e4m3fn bytes (gfx950's native fp8). The pages name the
 *   format only as fp8 e4m3 ([SGL-37889] Reproduce: --kv-cache-dtype
 *   fp8_e4m3; [ATOM-1473] Pull request overview: FP8 index cache).
 * - Top-k semantics: for each row, the k largest values of the row's window.
 *   Equal values go to the lower key position, so -0.0 ties with +0.0.
 *   Positions are row-local until the page transform ([SGL-37889]
 *   Modifications). A row with fewer than k visible keys yields all of them,
 *   then -1 padding. The ORDER of the k entries within a row is unspecified;
 *   the SET is exact.
 * - Return value: IDXTOPK_OK, or a negative status. Every argument is checked
 *   on the host before anything is enqueued, and on error nothing is
 *   enqueued. Kernel-launch failures return IDXTOPK_ELAUNCH.
 * - Caller-owned preconditions, not checked on the device:
 *     * windows lie inside their buffers;
 *     * row_to_batch entries and page ids are valid rows / pages;
 *     * seq_lens[b] <= max_seq_len;
 *     * scales are finite and > 0;
 *     * scores are not NaN;
 *     * slots fit in int32.
 *   Out-of-range inputs are undefined behaviour.
 */
#ifndef IDXTOPK_H
#define IDXTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDXTOPK_VERSION 100 /* 1.0.0 */

/* Status codes. */
#define IDXTOPK_OK 0
#define IDXTOPK_EINVAL (-1)       /* null required pointer, negative size, bad stride */
#define IDXTOPK_EUNSUPPORTED (-2) /* valid but not implemented: dim != 128, heads, k too large */
#define IDXTOPK_EWORKSPACE (-3)   /* workspace missing or smaller than idxtopk_workspace_bytes() */
#define IDXTOPK_ELAUNCH (-4)      /* the HIP runtime refused a kernel launch */

/* Limits. */
#define IDXTOPK_DIM 128           /* index-key / query head dimension */
#define IDXTOPK_MAX_K_ROWS 8192   /* topk_rows */
#define IDXTOPK_MAX_K_FUSED 8192  /* idx_score_topk_fused */
#define IDXTOPK_MAX_K_PREFILL 2048 /* idx_score_topk_prefill */

/* flags of topk_rows and idx_score_topk_fused */
#define IDXTOPK_SORTED 1  /* each output row in descending score order, equal
                             scores by ascending row-local position, -1
                             padding last (the sorted-output variant of the
                             selection; [SGL-37889] Modifications keeps the
                             selected index row-local until the transform) */
#define IDXTOPK_MAX_TOP_BLOCKS 4096 /* block_topk */

/* Operation ids for idxtopk_workspace_bytes(). */
#define IDXTOPK_OP_TOPK_ROWS 1
#define IDXTOPK_OP_SCORE 2
#define IDXTOPK_OP_PAGE_TRANSFORM 3
#define IDXTOPK_OP_SCORE_TOPK_FUSED 4
#define IDXTOPK_OP_BLOCK_TOPK 5
#define IDXTOPK_OP_CACHE_WRITE 6
#define IDXTOPK_OP_BLOCK_TOPK_HEADS 7 /* workspace query with rows = batch * heads */
#define IDXTOPK_OP_SCORE_TOPK_PREFILL 8

/* Key element types for idx_cache_write. */
#define IDXTOPK_KEY_F32 0  /* float */
#define IDXTOPK_KEY_BF16 1 /* bfloat16, as its 16-bit pattern */

/*
 * Indexer inputs shared by idx_score_fp8, idx_score_topk_fused and block_topk.
 *
 *   q           uint8 e4m3fn [batch, heads, dim]: one query token per row, one
 *               vector per index head.
 *   q_scale     float [batch]: dequantisation scale of each query row (> 0).
 *   w           float [batch, heads]: per-row, per-head weights.
 *   kcache      uint8 e4m3fn [num_slots, dim]: the paged index-key cache.
 *   k_scale     float [num_slots]: dequantisation scale of each cached key (> 0).
 *   block_table int32 [requests, bt_stride]: physical page of each logical
 *               page of a request. Token j of row b is at slot
 *               block_table[prow, j / page_size] * page_size + j % page_size
 *               ([ATOM-1473] decode-kernel diff: page = bt_row[blk], widened
 *               to int64 before use; positions blk * BLOCK_SIZE_K + offset).
 *   row_to_batch optional int32 [batch]: prow = row_to_batch[b], the
 *               block-table row of query row b; NULL gives prow = b. Several
 *               rows may share one block-table row: multi-token decode puts
 *               each of a request's query tokens in its own row, with its own
 *               causal length in seq_lens. Same indirection as topk_rows
 *               ([SGL-37889] Modifications); the caller owns its bound.
 *   seq_lens    int32 [batch]: n_b, the number of visible keys of row b (the
 *               causal length of the decode kernel's mask in [ATOM-1473]).
 *   max_seq_len an upper bound on every seq_lens[b], used to size the grid.
 *
 * Index score of token j of row b (computed in fp32 with fp8 MFMA):
 *   S[b, j] = sum_h w[b, h] * max(0, q_scale[b] * k_scale[slot_j]
 *                                   * sum_d q[b, h, d] * kcache[slot_j, d]).
 * The pages name the index score and its fp8 operands ([ATOM-1473] Pull
 * request overview; commit "fp8 index score calculate in fp8") but do not
 * write the formula out. The weighted-ReLU head sum above is this library's
 * definition.
 *
 * Supported shapes: dim == 128; heads in {16, 32, 64, 128}; page_size >= 1.
 */

/*
 * idx_score_fp8 -- write the index score of every visible key.
 *
 * Writes scores[b * score_stride + j] for 0 <= j < seq_lens[b]. Other cells
 * are untouched. This is the unfused score kernel of [ATOM-1473] (Pull
 * request overview: the index_score_kernel whose output tensor the fused
 * kernel removes).
 * Requires max_seq_len <= score_stride.
 */
int idx_score_fp8(const uint8_t* q, const float* q_scale, const float* w,
                  const uint8_t* kcache, const float* k_scale,
                  const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                  const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                  int32_t heads, int32_t dim, int32_t max_seq_len, float* scores,
                  int64_t score_stride, void* stream);

/*
 * topk_rows -- top-k over a given fp32 score buffer, with page transform.
 *
 * [SGL-37889] Modifications, addressing table:
 *   window of row i = scores[i * score_stride + rs_i + t], 0 <= t < seq_lens[i]
 *       with rs_i = row_starts ? row_starts[i] : 0;
 *   page-table row  = row_to_batch ? row_to_batch[i] : i.
 * Both indirections are optional (NULL gives the decode layout). With
 * row_to_batch the caller owns the page-table bound. The window may start at
 * any column, and score_stride need not be a multiple of 4.
 *
 * kv_offset (optional, int32 [rows]): for a call that sees one chunk of each
 * request's KV (chunked-prefix-cache extend, the shape [SGL-37889]
 * Modifications leaves to its legacy path: the addressing plan covers the
 * whole forward, the call one chunk), the KV position of row i's window
 * column 0. A selected window position t becomes p = t + kv_offset[i]
 * (default 0) before the transform; the caller owns the page-table bound
 * of p.
 *
 * out int32 [rows, k]: for each row, the k best positions p, mapped to
 * physical slots page_table[prow * pt_stride + p / page_size] * page_size +
 * p % page_size, or the positions themselves when page_table is NULL; -1 pads
 * rows with seq_lens[i] < k. Equal scores go to the lower position.
 *
 * flags: 0, or IDXTOPK_SORTED for rows in sorted order (otherwise the order
 * within a row is unspecified); any other bit gives IDXTOPK_EINVAL.
 *
 * 1 <= k <= IDXTOPK_MAX_K_ROWS. No workspace.
 */
int topk_rows(const float* scores, int64_t score_stride, int32_t rows,
              const int32_t* seq_lens, const int32_t* row_starts, const int32_t* row_to_batch,
              const int32_t* kv_offset, const int32_t* page_table, int64_t pt_stride, int32_t page_size,
              int32_t k, int32_t* out, int32_t flags, void* stream);

/*
 * topk_page_transform -- map row-local positions to physical slots.
 *
 * out[i, t] = idx[i, t] < 0 ? -1
 *           : page_table[prow * pt_stride + idx / page_size] * page_size + idx % page_size,
 * with prow = row_to_batch ? row_to_batch[i] : i ([SGL-37889] Modifications:
 * the selected index stays row-local and the transform maps it through the
 * page table). idx and out are int32 [rows, k] and may alias.
 */
int topk_page_transform(const int32_t* idx, int32_t rows, int32_t k,
                        const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                        const int32_t* row_to_batch, int32_t* out, void* stream);

/*
 * idx_score_topk_fused -- fused decode indexer: score + top-k + page transform.
 *
 * For every row b: the top k tokens of S[b, 0:seq_lens[b]] (ties to the lower
 * position), emitted as physical slots (the block_table mapping above). The
 * score row is never written to HBM ([ATOM-1473] Pull request overview: the
 * fused kernel removes the intermediate score tensor). Chunks of each row
 * keep their candidates in a caller-provided workspace, in place of the
 * partial score and index buffers of [ATOM-1473]'s kernel launch.
 *
 * out_slots  int32 [batch, k]; -1 pads rows with seq_lens[b] < k.
 * out_scores optional float [batch, k]: the score of each emitted token
 *            (-inf for padding).
 * workspace  device memory of at least
 *            idxtopk_workspace_bytes(IDXTOPK_OP_SCORE_TOPK_FUSED, batch, k, max_seq_len)
 *            bytes, with any contents: the call reads only what it wrote
 *            itself, and no later call depends on what it leaves. Concurrent
 *            calls must not share one workspace.
 * flags      0, or IDXTOPK_SORTED (out_slots and out_scores in sorted order;
 *            otherwise the order within a row is unspecified); any other
 *            bit gives IDXTOPK_EINVAL.
 * 1 <= k <= IDXTOPK_MAX_K_FUSED.
 */
int idx_score_topk_fused(const uint8_t* q, const float* q_scale, const float* w,
                         const uint8_t* kcache, const float* k_scale,
                         const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                         const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                         int32_t heads, int32_t dim, int32_t max_seq_len, int32_t k,
                         int32_t* out_slots, float* out_scores, void* workspace,
                         size_t workspace_bytes, int32_t flags, void* stream);

/*
 * idx_score_topk_fused_noalloc -- idx_score_topk_fused with a built-in
 * workspace, for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Arguments, outputs, flags and status codes are idx_score_topk_fused's,
 * without the workspace: the call uses a workspace of
 * IDXTOPK_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on, from the first call on that GPU until the process ends. The call
 * allocates and frees nothing. The first call on a device looks up that
 * device's array (no allocation, no stream work).
 * Returns IDXTOPK_EWORKSPACE when the call would need more than that:
 * idxtopk_workspace_bytes(IDXTOPK_OP_SCORE_TOPK_FUSED, batch, k, max_seq_len)
 * > IDXTOPK_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (two streams, two threads) race and give wrong results. (The
 * array's contents never matter: each call reads only what it wrote.)
 */
#define IDXTOPK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20) /* 64 MiB per GPU */
int idx_score_topk_fused_noalloc(const uint8_t* q, const float* q_scale, const float* w,
                                 const uint8_t* kcache, const float* k_scale,
                                 const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                                 const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                                 int32_t heads, int32_t dim, int32_t max_seq_len, int32_t k,
                                 int32_t* out_slots, float* out_scores, int32_t flags, void* stream);

/*
 * idx_score_topk_prefill -- fused prefill indexer: score + top-k + page
 * transform for packed prefill rows, with no score row in HBM.
 *
 * The result is idx_score_topk_fused's (same arguments, outputs, flags and
 * status codes): for every query row b, the top k tokens of
 * S[b, 0:seq_lens[b]] (ties to the lower position) as physical slots of
 * block-table row row_to_batch[b]. The query rows of a prefill batch are
 * packed, request after request, and each keeps the top k of its causal
 * window ([SGL-37889] Motivation and Modifications: packed prefill rows
 * addressed through row_to_batch, k = 512, the selection mapped through the
 * page table); the intermediate score tensor is removed as in
 * [ATOM-1473]'s fused decode kernel (Pull request overview).
 *
 * This path is built for many rows per request: four consecutive rows that
 * name the same block-table row share every key load. Chunks of each row
 * keep the tokens above a bound taken from a sample of their own scores;
 * rows whose bound was too high are scored again in full, so every row is
 * exact.
 *
 * workspace  at least idxtopk_workspace_bytes(IDXTOPK_OP_SCORE_TOPK_PREFILL,
 *            batch, k, max_seq_len) bytes (about 8 (k + 6 sqrt(k n / 1024)
 *            + 6 n / 1024) bytes per row for n = max_seq_len, plus
 *            16 max_seq_len * 8), with any contents: the call reads only
 *            what it wrote itself. Concurrent calls must not share one
 *            workspace.
 * Supported: fp8 cache, heads 16, 32 or 64, page_size a multiple of 16,
 * 1 <= k <= IDXTOPK_MAX_K_PREFILL; others give IDXTOPK_EUNSUPPORTED.
 */
int idx_score_topk_prefill(const uint8_t* q, const float* q_scale, const float* w,
                           const uint8_t* kcache, const float* k_scale,
                           const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                           const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                           int32_t heads, int32_t dim, int32_t max_seq_len, int32_t k,
                           int32_t* out_slots, float* out_scores, void* workspace,
                           size_t workspace_bytes, int32_t flags, void* stream);

/*
 * block_topk -- block-sparse variant: block scores, top blocks, sparse list.
 *
 * Block c of row b covers tokens [c * block_size, min((c + 1) * block_size,
 * n_b)). Its score is the max of S over those tokens (the pages' "index
 * block-score kernel" in [ATOM-1473] Pull request overview, reduction read as
 * max). Keep the top_blocks best blocks, ties to the lower block id, and build
 * the sparse block list in the same call ([ATOM-1282], title: merge build
 * sparse block into topk).
 *
 * Requires block_size == page_size, so block c is physical page
 * block_table[b, c].
 * out_blocks int32 [batch, top_blocks]: physical block (page) ids; -1 pads.
 * out_slots  optional int32 [batch, top_blocks * block_size]: entry
 *            i * block_size + t is the slot of token t of the i-th emitted
 *            block, or -1 past n_b or for padded blocks.
 * workspace  at least idxtopk_workspace_bytes(IDXTOPK_OP_BLOCK_TOPK, batch,
 *            block_size, max_seq_len) bytes, with any contents (as for
 *            idx_score_topk_fused); concurrent calls must not share one.
 * 1 <= top_blocks <= IDXTOPK_MAX_TOP_BLOCKS.
 */
int block_topk(const uint8_t* q, const float* q_scale, const float* w,
               const uint8_t* kcache, const float* k_scale,
               const int32_t* block_table, int64_t bt_stride, int32_t page_size,
               const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
               int32_t heads, int32_t dim, int32_t max_seq_len, int32_t block_size,
               int32_t top_blocks,
               int32_t* out_blocks, int32_t* out_slots,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * block_topk_heads -- per-head variant of block_topk: every index head keeps
 * its own blocks.
 *
 * Head h's term of the index score, T_h[b, j] = w[b, h] * max(0, q_scale[b]
 * * k_scale[slot_j] * sum_d q[b, h, d] * kcache[slot_j, d]) (the score is
 * the sum of these over h), gives head h's block scores (the max over the
 * block's visible tokens), and the top_blocks best blocks of every (row,
 * head) are kept, ties to the lower block id ([ATOM-1473] Pull request
 * overview: the partial top-k kernel's grid runs over query rows, index
 * heads and chunks; per-head selection is this library's reading of that
 * head axis).
 *
 * out_blocks  int32 [batch, heads, top_blocks] physical block ids, -1 pads;
 * out_slots   optional int32 [batch, heads, top_blocks * block_size], laid
 *             out as block_topk's per (row, head);
 * workspace   at least idxtopk_workspace_bytes(IDXTOPK_OP_BLOCK_TOPK_HEADS,
 *             batch * heads, block_size, max_seq_len) bytes, with any
 *             contents (as for block_topk).
 * Other arguments, limits and status codes: block_topk's (fp8 cache).
 */
int block_topk_heads(const uint8_t* q, const float* q_scale, const float* w,
                     const uint8_t* kcache, const float* k_scale,
                     const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                     const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                     int32_t heads, int32_t dim, int32_t max_seq_len, int32_t block_size,
                     int32_t top_blocks, int32_t* out_blocks, int32_t* out_slots,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_cache_write -- quantize new index keys into the paged fp8 cache.
 *
 * For every token t with s = slot_mapping[t] >= 0:
 *   scale          = max_d |keys[t, d]| / 448   (fp32 division, rounded to
 *                    nearest; 1 when that is 0),
 *   kcache[s, d]   = e4m3fn(keys[t, d] / scale) (fp32 division rounded to
 *                    nearest, then the nearest e4m3fn value, ties to the
 *                    even mantissa, magnitudes above 448 saturating),
 *   k_scale[s]     = scale.
 * Tokens with a negative slot are skipped. This is the cache layout every
 * indexer entry point above reads ([ATOM-1473] Pull request overview and the
 * attention-layer diffs: the index-key cache is allocated in fp8 and written
 * with a key scale; one scale per token and the rounding are this library's
 * reading).
 *
 * keys          [tokens, key_stride] row-major, elements of key_dtype
 *               (IDXTOPK_KEY_F32 or IDXTOPK_KEY_BF16); the first dim of
 *               each row are the key. keys and key_stride must keep every
 *               row 8-byte aligned (fp32) or 4-byte aligned (bf16).
 * slot_mapping  int32 [tokens]: destination slot, or negative to skip.
 *               Non-negative slots must be distinct (two tokens writing one
 *               slot race) and below the cache's slot count.
 * kcache        uint8 e4m3fn [num_slots, dim]; k_scale float [num_slots].
 * dim == IDXTOPK_DIM. Keys must be finite. No workspace.
 */
int idx_cache_write(const void* keys, int32_t key_dtype, int64_t key_stride, int32_t tokens,
                    int32_t dim, const int32_t* slot_mapping, uint8_t* kcache, float* k_scale,
                    void* stream);

/*
 * bf16 index cache ([ATOM-1473] Pull request overview: the index cache is
 * fp8 when the KV cache is fp8 and takes the model's dtype otherwise;
 * commit "convert auto for bf16 type"). The library reads that case as bf16
 * queries and keys with no scales:
 *   S[b, j] = sum_h w[b, h] * max(0, sum_d q[b, h, d] * kcache[slot_j, d]),
 * products and sums in fp32 (v_mfma_f32_16x16x32_bf16).
 *
 * q       bf16 [batch, heads, dim], 16-byte aligned (bit patterns; any
 *         16-bit element type);
 * kcache  bf16 [num_slots, dim] (256 bytes per slot), 16-byte aligned;
 * every other argument, the outputs, workspace, flags and status codes are
 * those of the fp8 entry point of the same name without the suffix. A
 * misaligned q or kcache gives IDXTOPK_EINVAL.
 */
int idx_score_bf16(const uint16_t* q, const float* w, const uint16_t* kcache,
                   const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                   const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                   int32_t heads, int32_t dim, int32_t max_seq_len, float* scores,
                   int64_t score_stride, void* stream);

int idx_score_topk_fused_bf16(const uint16_t* q, const float* w, const uint16_t* kcache,
                              const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                              const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                              int32_t heads, int32_t dim, int32_t max_seq_len, int32_t k,
                              int32_t* out_slots, float* out_scores, void* workspace,
                              size_t workspace_bytes, int32_t flags, void* stream);

int block_topk_bf16(const uint16_t* q, const float* w, const uint16_t* kcache,
                    const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                    const int32_t* row_to_batch, const int32_t* seq_lens, int32_t batch,
                    int32_t heads, int32_t dim, int32_t max_seq_len, int32_t block_size,
                    int32_t top_blocks, int32_t* out_blocks, int32_t* out_slots,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_cache_write_bf16 -- store new index keys into the bf16 cache.
 *
 * For every token t with s = slot_mapping[t] >= 0: kcache[s, d] =
 * bf16(keys[t, d]), rounded to nearest with ties to the even pattern for
 * fp32 keys, copied as they are for bf16 keys; no scale. Tokens with a
 * negative slot are skipped.
 *
 * keys          [tokens, key_stride] row-major, elements of key_dtype
 *               (IDXTOPK_KEY_F32 or IDXTOPK_KEY_BF16); keys and every row
 *               start 16-byte aligned, else IDXTOPK_EINVAL.
 * slot_mapping  int32 [tokens], distinct non-negative slots below the
 *               cache's slot count.
 * kcache        bf16 [num_slots, dim], 16-byte aligned.
 * dim == IDXTOPK_DIM. Keys must be finite. No workspace.
 */
int idx_cache_write_bf16(const void* keys, int32_t key_dtype, int64_t key_stride, int32_t tokens,
                         int32_t dim, const int32_t* slot_mapping, uint16_t* kcache, void* stream);

/*
 * Workspace bytes an operation needs (0 when it needs none).
 * For IDXTOPK_OP_BLOCK_TOPK, pass block_size as `k`. Returns 0 for invalid
 * arguments as well.
 */
size_t idxtopk_workspace_bytes(int32_t op, int32_t rows, int32_t k, int32_t max_seq_len);

/* Human-readable text of a status code (static storage). */
const char* idxtopk_status_str(int32_t status);

/* IDXTOPK_VERSION of the loaded library. */
int32_t idxtopk_version(void);

/*
 * Checked builds. libidxtopk_checked.so is the same library built with
 * device-side checks of the caller-owned preconditions listed at the top of
 * this file and of the library's internal bounds; the kernels otherwise run
 * as in a release build and their results are the same. A failed check sets
 * its bit in a device error word:
 */
#define IDXTOPK_CHK_WINDOW 0x1         /* topk_rows: a window outside its buffer row */
#define IDXTOPK_CHK_CAND_OVERFLOW 0x2  /* topk_rows: candidate buffer overrun (internal) */
#define IDXTOPK_CHK_POSITION 0x4       /* a selected position outside its row (internal) */
#define IDXTOPK_CHK_SEQ_LEN 0x8        /* seq_lens[b] < 0 or above max_seq_len */
#define IDXTOPK_CHK_ROW_TO_BATCH 0x10  /* row_to_batch[b] < 0 */
#define IDXTOPK_CHK_PAGE_ID 0x20       /* a block-table or page-table entry < 0 */
#define IDXTOPK_CHK_CHUNK_COUNT 0x40   /* fused: chunk candidates above its tokens (internal) */
#define IDXTOPK_CHK_BLOCK 0x80         /* block top-k: a block outside the row (internal) */
#define IDXTOPK_CHK_MERGE_COUNT 0x100  /* fused merge: candidate counts inconsistent (internal) */
#define IDXTOPK_CHECKS_OFF 0x80000000u /* a release build: no checks compiled in */
/*
 * idxtopk_check_status -- the bits of every check that failed since the
 * last clear (0: none), after waiting for the current device's queued work.
 * clear != 0 zeroes the words. A release build returns IDXTOPK_CHECKS_OFF
 * without touching the device.
 */
uint32_t idxtopk_check_status(int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* IDXTOPK_H */
