/*
 * dsv4.h -- C ABI of the MI355X (gfx950) DeepSeek-V4 indexed-attention prefill
 * hot path: ratio-4 compressor -> indexer score + top-k -> fused windowed +
 * pooled sparse attention.
 *
 * Sources (page titles; sections in brackets):
 *   [P1] "perf(deepseek-v4): skip redundant all-pooled indexer scoring"
 *        (oMLX pull request 2563) [Summary, Correctness]
 *   [P2] "perf(deepseek_v4): faster exact DeepSeek-V4 prefill (wsdpa fusion +
 *        scheduler/cache amortization)" (oMLX pull request 2568)
 *        [Summary commits 1, 4, 5; Performance]
 *   [P3] "[Discussion] Tile indexed-attention scoring independently of the
 *        global prefill chunk" (ds4 issue 644) [Summary, Possible design]
 *   [P4] "perf(dflash): add opt-in exact prefill bands" (lucebox pull
 *        request 590) [q2-q4 exact prefill bands]
 *
 * Conventions shared by every entry point
 *   - Pointers named "device" are HIP device memory owned by the caller; the
 *     library never allocates, frees or keeps them.  Host structs are owned by
 *     the caller; the library only updates the fields documented below.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the library never synchronizes: device faults surface
 *     at the caller's next synchronization of that stream.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     a non-zero return nothing was enqueued, no host struct changed, and
 *     dsv4_last_error() describes the failure (thread-local string).
 *   - Positions, counts, sizes and strides are at most DSV4_MAX_EXTENT;
 *     byte sizes that would not fit a size_t are INVALID_ARG as well.
 *   - The kernels only implement the standard masks (causal window, pooled-row
 *     visibility rebuilt from positions [P2 commit 1]); they never take a mask
 *     tensor.  A caller needing another mask must use its own path.
 *   - Positions are absolute token positions counted from the start of the
 *     stream (0-based).  With pool ratio r (4 unless stated), pooled row s
 *     summarises tokens rs .. rs+r-1 and is visible to a query at position p
 *     iff r(s+1) <= p+1, i.e. s < (p+1)/r.
 *   - Calls that touch the same cache must be ordered on one stream.
 */
#ifndef DSV4_H
#define DSV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 4: dsv4_indexer_select may keep top-k candidates in its scratch (the
 * scores are not left there), and dsv4_topk_select_split takes more rows.
 * 5: dsv4_indexer_select_noalloc.
 * 6: extents above DSV4_MAX_EXTENT are rejected; dsv4_score_stride returns -1
 * for them. */
#define DSV4_ABI_VERSION 6

/* Return codes. */
#define DSV4_OK                0
#define DSV4_ERR_INVALID_ARG  -1  /* NULL pointer, negative size, position or
                                     window outside what the buffers cover     */
#define DSV4_ERR_UNSUPPORTED  -2  /* shape gate: a shape or dtype the kernels
                                     do not implement; caller may fall back    */
#define DSV4_ERR_CAPACITY     -3  /* append would pass the cache capacity      */
#define DSV4_ERR_ROW_MISMATCH -4  /* attention / indexer pooled row counts
                                     diverge [P1 Summary]                      */
#define DSV4_ERR_SCRATCH      -5  /* scratch buffer too small                  */
#define DSV4_ERR_HIP          -6  /* HIP launch error (message has details)    */

/* Storage types of a pooling cache. */
#define DSV4_BF16 1
#define DSV4_F32  2

/* Largest supported sizes (shape gate). */
#define DSV4_MAX_TOPK        4096
#define DSV4_MAX_INDEX_HEADS 64
#define DSV4_MAX_HEADS       64
#define DSV4_MAX_RATIO       256
#define DSV4_MAX_ATTN_SPLITS 64
/* Bytes of the per-GPU static score scratch of dsv4_indexer_select_noalloc. */
#define DSV4_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
/* Largest position, count, size or stride any entry point takes (a cache's
 * capacity and n_rows included): 2^40, far past any real context, so that the
 * host's index and size arithmetic cannot overflow.  Larger values are
 * INVALID_ARG. */
#define DSV4_MAX_EXTENT ((int64_t)1 << 40)

/*
 * PoolingCache of one compressor [P1 Summary, Correctness; P2 commit 4].
 * rows : device [capacity][dim] pooled rows; rows [0, n_rows) are valid.
 * rem  : device [ratio-1][dim] raw rows received but not yet pooled;
 *        rows [0, n_rem) are valid.
 * The stream position of the next raw token is ratio*n_rows + n_rem.
 * dsv4_compress updates n_rows and n_rem on success.
 * ratio: 4 for the indexer path and sparse attention, 128 for the
 * CompressedAttention mode [P2 commit 1; the ratio-128 prefill route it
 * builds on]; 2 <= ratio <= DSV4_MAX_RATIO is accepted by dsv4_compress and
 * dsv4_sparse_prefill_attn, the indexer entry points require ratio 4.
 * dtype DSV4_BF16 is the hot-path type; DSV4_F32 is accepted by
 * dsv4_compress only.
 */
typedef struct dsv4_pool_cache {
  void*   rows;
  void*   rem;
  int64_t capacity;
  int64_t n_rows;
  int32_t n_rem;
  int32_t ratio;
  int32_t dim;
  int32_t dtype;
} dsv4_pool_cache;

/*
 * Capability probe [P2 commit 5: callers probe the kernel's signature once
 * and fall back when the fused form is absent]: returns DSV4_ABI_VERSION of
 * the loaded library, so a caller built against a newer header can detect
 * an older library before calling entry points it lacks.
 */
int dsv4_abi_version(void);

/* Message describing the last failed call on this thread ("" if none). */
const char* dsv4_last_error(void);

/*
 * All-pooled decision [P1 Summary]: 1 iff 0 < n_rows <= topk, i.e. every
 * pooled row fits within index_topk and scoring can be skipped; 0 otherwise
 * (empty pools and pools larger than topk keep the full path).
 */
int dsv4_indexer_all_pooled(int64_t n_rows, int32_t topk);

/*
 * Row stride, in floats, of the score scratch for a cache holding n_rows
 * pooled rows (n_rows rounded up to a multiple of 64; 64 for n_rows <= 0;
 * -1 for n_rows above DSV4_MAX_EXTENT).
 */
int64_t dsv4_score_stride(int64_t n_rows);

/*
 * Bytes of score scratch dsv4_indexer_select needs for query-row tiles of
 * tile_rows rows against up to max_rows pooled rows [P3 Summary: scratch
 * scales with tile rows x pooled rows]: tile_rows x dsv4_score_stride(max_rows)
 * floats, plus, for narrow tiles (tile_rows <= 64) over more than 32,768
 * pooled rows, the workspace of the chunk-parallel top-k (sized for
 * DSV4_MAX_TOPK).  Writes *bytes.  0 or INVALID_ARG.
 */
int dsv4_indexer_scratch_bytes(int64_t tile_rows, int64_t max_rows, size_t* bytes);

/*
 * Pooling compressor, r = cache->ratio [P1 Correctness (ratio 4); P2 commit
 * 4].
 * x     : device [n_new][cache->dim] raw rows in cache->dtype (may be NULL
 *         iff n_new == 0).
 * The old remainder followed by x is cut into groups of r consecutive rows;
 * each whole group becomes one pooled row (mean of the r rows: float32 sum
 * taken left to right, times the float32 value of 1/r, rounded to the
 * storage type, ties to even), appended in place at cache->n_rows; the rows
 * left over become the new remainder.  Host fields n_rows / n_rem are
 * updated at enqueue time.
 * Errors: INVALID_ARG, UNSUPPORTED (ratio outside [2, DSV4_MAX_RATIO],
 * dtype), CAPACITY.
 */
int dsv4_compress(dsv4_pool_cache* cache, const void* x, int64_t n_new, void* stream);

/*
 * Indexer scores for `rows` query rows at positions q_pos0 .. q_pos0+rows-1
 * against the S = index_cache->n_rows pooled index keys [P2 Performance,
 * commit 5]:
 *     out[t][s] = sum_h w[t][h] * max(0, q[t][h][:] . key[s][:])
 * q   : device bf16 [rows][n_heads][dim], dim = index_cache->dim
 * w   : device float [rows][n_heads]
 * out : device float [rows][out_stride], columns [0, S) written.
 * fold_mask = 1: entries with s >= (q_pos0+t+1)/4 are written as -inf (the
 * pooled-ratio causal mask folded into the score epilogue [P2 commit 5]);
 * fold_mask = 0: every s < S is scored (second-pass masking is then the
 * caller's, with the same -inf sentinel).
 * Each entry is computed by one workgroup in a fixed order (fp32 products
 * of the bf16 inputs summed over dim in MFMA order, then over heads), so an
 * unmasked entry's bits depend only on q[t], w[t] and key[s]: not on rows,
 * nor on how the launch splits the rows and columns.  A row's scores are the
 * same in any tile and run to run.
 * Shape gate: bf16 ratio-4 cache, dim in {32, 64, 128}, 1 <= n_heads <= 64,
 * S <= out_stride <= 2^28 - 64 (UNSUPPORTED beyond).
 */
int dsv4_indexer_scores(const dsv4_pool_cache* index_cache, const void* q, const float* w,
                        int64_t rows, int64_t q_pos0, int32_t n_heads, int32_t fold_mask,
                        float* out, int64_t out_stride, void* stream);

/*
 * Top-k of each score row over its visible prefix [P1 Summary; P3 Possible
 * design step 3].  Row t (position q_pos0+t) considers columns
 * [0, (q_pos0+t+1)/4); it selects the min(topk, visible) largest scores,
 * equal scores going to the lower column (-0 equals +0), and writes the
 * chosen columns in ascending order followed by -1 up to topk.
 * scores  : device float [rows][stride] (finite in the visible prefix)
 * out_idx : device int32 [rows][topk]
 * n_cols bounds the visible prefix: (q_pos0+rows)/4 <= n_cols <= stride.
 */
int dsv4_topk_select(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                     int64_t n_cols, int32_t topk, int32_t* out_idx, void* stream);

/*
 * Chunk-parallel top-k for long rows (narrow-query steps: decode, draft
 * verification, short prefill bands at long context [P1 scope; P4]; and
 * whole tiles at 1M context).  Same arguments, rule and output as
 * dsv4_topk_select, bit for bit, plus a caller-owned device workspace
 * (16-byte aligned).  When the longest visible prefix spans more than one
 * 32,768-column chunk, the first row sees at least topk columns, and either
 * rows <= 64 or (topk % 4 == 0 and chunks * topk <= 32,768), every
 * (row, chunk) pair is selected by its own workgroup and a second pass
 * selects each row's top-k among the chunk winners; otherwise it runs
 * dsv4_topk_select's kernel and the workspace is unused (may be NULL).
 * dsv4_topk_split_workspace_bytes writes the workspace bytes needed (0 when
 * the two-pass path does not apply).
 * Errors: as dsv4_topk_select; INVALID_ARG (workspace NULL / misaligned when
 * needed), SCRATCH (workspace too small).
 */
int dsv4_topk_split_workspace_bytes(int64_t rows, int64_t q_pos0, int32_t topk, size_t* bytes);
int dsv4_topk_select_split(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                           int64_t n_cols, int32_t topk, int32_t* out_idx, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Whole indexer step for one prefill chunk of T query rows [P1 Summary;
 * P3 Possible design].
 *   1. Guard: index_cache->n_rows must equal n_attn_rows (ROW_MISMATCH).
 *   2. If 0 < S <= topk (all pooled): out_idx[t] = 0 .. (p+1)/4 - 1, then -1;
 *      q and w are not read (may be NULL); *out_all_pooled = 1.
 *   3. If S == 0: every slot -1, *out_all_pooled = 0.
 *   4. Otherwise, for each tile of tile_rows query rows (0 = all T), scores
 *      are written to `scratch` (folded mask) and the tile's top-k is taken,
 *      reusing the same scratch for every tile; *out_all_pooled = 0.  Over
 *      more than 32,768 pooled rows the top-k runs per 32,768-column chunk
 *      and then per row among the chunks' winners (the same result); where
 *      k is a multiple of 4 and the first query row sees at least k pooled
 *      rows, the chunks' winners are kept in the score rows themselves, so
 *      the scratch does not hold the scores after the call.  Otherwise a
 *      narrow tile (<= 64 rows) uses dsv4_topk_select_split's workspace
 *      after the scores when the scratch holds it (as
 *      dsv4_indexer_scratch_bytes sizes it).
 * q, w        : as dsv4_indexer_scores, T rows.
 * scratch     : device float, >= dsv4_indexer_scratch_bytes(tile, S) bytes
 *               (may be NULL on paths 2 and 3).
 * out_idx     : device int32 [T][topk].
 * out_all_pooled : host int32 (may be NULL).
 * The queries must lie behind the compressor frontier: q_pos0 + T <=
 * 4*S + n_rem of the index cache (compress the whole chunk first).
 */
int dsv4_indexer_select(const dsv4_pool_cache* index_cache, int64_t n_attn_rows,
                        const void* q, const float* w, int64_t T, int64_t q_pos0,
                        int32_t n_heads, int32_t topk, int32_t tile_rows,
                        float* scratch, size_t scratch_bytes,
                        int32_t* out_idx, int32_t* out_all_pooled, void* stream);

/*
 * dsv4_indexer_select for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, paths and output as
 * dsv4_indexer_select (bit for bit), without the scratch: the score scratch
 * is a static device array of DSV4_NOALLOC_SCRATCH_BYTES (32 MiB) that each
 * GPU the library runs on holds until the process ends.  The call allocates
 * and frees nothing; on a device's first call it looks the array's address
 * up (hipGetSymbolAddress, with the current device = the stream's device).
 * tile_rows = 0 takes the largest query-row tile whose scores fit the array
 * (32 MiB / (4 * dsv4_score_stride(S)) rows: 256 at 32,768 pooled rows, 32 at
 * 262,144); a tile_rows > 0 whose tile does not fit is refused with
 * DSV4_ERR_SCRATCH before anything is enqueued (also when one row does not
 * fit: more than 8,388,608 pooled rows).  The all-pooled and empty paths
 * need no scratch.
 * Every call on one GPU shares that GPU's array and leaves its last contents
 * there (nothing in it needs clearing: each tile's scores are written before
 * they are read).  Calls that overlap on one GPU -- on different streams or
 * threads, or a captured graph replayed beside another call -- race on it:
 * order them on one stream.
 */
int dsv4_indexer_select_noalloc(const dsv4_pool_cache* index_cache, int64_t n_attn_rows,
                                const void* q, const float* w, int64_t T, int64_t q_pos0,
                                int32_t n_heads, int32_t topk, int32_t tile_rows,
                                int32_t* out_idx, int32_t* out_all_pooled, void* stream);

/*
 * Fused windowed + pooled prefill attention [P2 commit 1; P3 Possible design
 * step 4].  For the query at position p = q_pos0+t and head h, with
 * r = attn_cache->ratio:
 *   keys  = raw rows at positions max(0, p-window+1) .. p
 *           + pooled rows s listed in sel_idx[t] with 0 <= s < (p+1)/r
 *             (all s < (p+1)/r when sel_idx is NULL; -1 slots are empty)
 *   out[t][h] = sum_j softmax_j(scale * q[t][h] . key_j) * key_j
 * (keys double as values and are shared by all heads).
 * q       : device bf16 [T][n_heads][head_dim]
 * raw_kv  : device bf16 [n_raw][head_dim], row i is position raw_pos0+i; it
 *           must cover [max(0, q_pos0-window+1), q_pos0+T).
 * attn_cache : bf16 pooling cache with dim == head_dim, or NULL for the
 *           window-only mode (LocalAttention: no pooled keys; sel_idx must
 *           then be NULL).  The three modes of [P2 commit 1]:
 *           LocalAttention = NULL cache; CompressedAttention = ratio-128
 *           cache, NULL sel_idx; SparseCompressedAttention = ratio-4 cache
 *           with the indexer's sel_idx (or NULL on the small-pool path).
 * sel_idx : device int32 [T][topk] or NULL.
 * out     : device bf16 [T][n_heads][head_dim].
 * q, raw_kv, out and the cache rows must be 16-byte aligned (the kernel
 * moves them in 16-byte vectors); INVALID_ARG otherwise.
 * scale <= 0 selects 1/sqrt(head_dim).
 * Shape gate: head_dim in {32, 64, 128, 256, 512}, 1 <= n_heads <= 64,
 * window >= 1, topk <= DSV4_MAX_TOPK.
 */
int dsv4_sparse_prefill_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                             int32_t head_dim, float scale,
                             const void* raw_kv, int64_t raw_pos0, int64_t n_raw,
                             int32_t window, const dsv4_pool_cache* attn_cache,
                             const int32_t* sel_idx, int32_t topk, void* out, void* stream);

/*
 * Narrow-query steps (T = 1-4 and other short query counts: decode, draft
 * verification, narrow prefill bands) [P1 scope: MTP with three draft
 * tokens; P4: exact q2-q4 prefill bands].  dsv4_sparse_prefill_attn walks each query's keys in one
 * workgroup, so a handful of queries occupies a handful of CUs; the narrow
 * variant splits each query's key tiles over n_splits workgroups and merges
 * them.  The result is the same attention (same keys, same definition), up
 * to floating-point summation order.
 *
 * Plan: *n_splits = the split count to use for T queries of at most
 * window + n_pooled_keys keys each (n_pooled_keys: topk with a selection, the
 * visible pooled rows without one, 0 for window only), about one workgroup
 * per CU in all and at least two 32-key tiles per split, at most
 * DSV4_MAX_ATTN_SPLITS; *workspace_bytes = the workspace it needs (0 when
 * *n_splits == 1).  0 or INVALID_ARG.
 */
int dsv4_sparse_attn_narrow_plan(int64_t T, int32_t n_heads, int32_t head_dim, int32_t window,
                                 int64_t n_pooled_keys, int32_t* n_splits,
                                 size_t* workspace_bytes);

/*
 * Narrow-query attention: arguments, modes and output as
 * dsv4_sparse_prefill_attn, plus
 * n_splits  : 1 .. DSV4_MAX_ATTN_SPLITS key splits per query (1 = the
 *             prefill kernel itself; the workspace is then unused).
 * workspace : device, 16-byte aligned, >= T*n_splits*n_heads*(head_dim+2)*4
 *             bytes, owned by the caller (fp32 partial outputs, then the
 *             per-head (max, sum) pairs); its contents are overwritten.
 * Each split walks a balanced range of the query's key tiles with the same
 * online softmax and leaves (m, l, O); a second kernel merges the splits:
 * out = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s, M = max m_s.
 * Errors: as dsv4_sparse_prefill_attn; UNSUPPORTED (n_splits), INVALID_ARG
 * (workspace NULL / misaligned), SCRATCH (workspace too small).
 */
int dsv4_sparse_attn_narrow(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                            int32_t head_dim, float scale,
                            const void* raw_kv, int64_t raw_pos0, int64_t n_raw,
                            int32_t window, const dsv4_pool_cache* attn_cache,
                            const int32_t* sel_idx, int32_t topk, int32_t n_splits,
                            float* workspace, size_t workspace_bytes, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_H */
