// Host side of the C ABI declared in include/dsv4.h: argument and shape
// checks (all before any enqueue), PoolingCache accounting, the all-pooled
// decision and row-count guard, the query-row tile loop over one score
// scratch, and kernel launches on the caller's stream.
//
// [P1 "perf(deepseek-v4): skip redundant all-pooled indexer scoring",
// Summary: skip scoring when every pooled row fits in index_topk, still run
// the indexer compressor, guard attention/indexer row counts, keep the full
// path for empty and large pools.  P3 "[Discussion] Tile indexed-attention
// scoring independently of the global prefill chunk", Possible design: score
// and select bounded query-row tiles that reuse one scratch.]
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "../../include/dsv4.h"
#include "dsv4_device.h"

static_assert(DSV4_MAX_ATTN_SPLITS == dsv4::kMaxAttnSplits, "split cap");
static_assert(DSV4_MAX_TOPK == dsv4::kMaxTopk, "largest k: ABI and kernels agree");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSV4_OK;
  return fail(DSV4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

int dsv4_internal_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

namespace {

// Positions, counts, sizes and strides the entry points take: 0 ..
// DSV4_MAX_EXTENT (2^40), so sums of a few of them, and their products with
// the small factors below, stay inside int64_t.
inline bool extent_ok(int64_t v) { return v >= 0 && v <= DSV4_MAX_EXTENT; }

// a * b into *out; false when the product does not fit a size_t.
inline bool mul_size(size_t a, size_t b, size_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Pool ratios accepted by the compressor and the attention: 4 (indexer and
// sparse attention) and 128 (CompressedAttention) are the pages'; any ratio
// in [2, DSV4_MAX_RATIO] follows the same definitions.  The indexer entry
// points pass need_ratio = 4: their score mask and selection fill are the
// ratio-4 rule.
int check_cache(const dsv4_pool_cache* c, const char* name, int need_ratio = 0) {
  if (!c) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL cache", name);
  if (need_ratio && c->ratio != need_ratio)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: ratio %d (only %d)", name, c->ratio, need_ratio);
  if (c->ratio < 2 || c->ratio > DSV4_MAX_RATIO)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: ratio %d", name, c->ratio);
  if (c->dtype != DSV4_BF16 && c->dtype != DSV4_F32)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: dtype %d", name, c->dtype);
  if (c->dim <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: dim %d", name, c->dim);
  if (!extent_ok(c->capacity) || c->n_rows < 0 || c->n_rows > c->capacity)
    return fail(DSV4_ERR_INVALID_ARG, "%s: n_rows %lld / capacity %lld", name,
                (long long)c->n_rows, (long long)c->capacity);
  if (c->n_rem < 0 || c->n_rem >= c->ratio)
    return fail(DSV4_ERR_INVALID_ARG, "%s: n_rem %d", name, c->n_rem);
  if (c->capacity > 0 && !c->rows) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL rows", name);
  if (!c->rem) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL remainder buffer", name);
  return DSV4_OK;
}

inline int64_t vis_rows(int64_t p, int ratio = 4) { return (p + 1) / ratio; }

// Chunk-parallel top-k (two passes) serves rows whose visible prefixes span
// more than one 32,768-column chunk and hold at least topk columns: at most
// kSplitRows of them, or any number when k is a multiple of 4 and a row has
// at most 32,768 candidates (the register kernels' two passes).  Its
// workspace is the chunk candidates' columns and scores.
constexpr int64_t kSplitRows = 64;
constexpr int64_t kTopkChunk = 32768;

size_t split_ws_bytes(int64_t rows, int64_t chunks, int32_t topk) {
  const size_t one = (static_cast<size_t>(rows) * static_cast<size_t>(chunks) *
                          static_cast<size_t>(topk) * 4 + 15) & ~static_cast<size_t>(15);
  return 2 * one;
}

bool split_applies(int64_t rows, int64_t q_pos0, int32_t topk) {
  const int64_t chunks = dsv4_topk_split_chunks(rows, q_pos0);
  return rows > 0 && chunks >= 2 && (q_pos0 + 1) / 4 >= topk &&
         (rows <= kSplitRows || (topk % 4 == 0 && chunks * topk <= kTopkChunk));
}

// The MFMA kernels read operands with 16-byte vector loads.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int dsv4_abi_version(void) { return DSV4_ABI_VERSION; }

const char* dsv4_last_error(void) { return g_err; }

int dsv4_indexer_all_pooled(int64_t n_rows, int32_t topk) {
  return (n_rows > 0 && n_rows <= topk) ? 1 : 0;
}

int64_t dsv4_score_stride(int64_t n_rows) {
  if (n_rows <= 0) return 64;
  if (n_rows > DSV4_MAX_EXTENT) return -1;
  return (n_rows + 63) / 64 * 64;
}

int dsv4_indexer_scratch_bytes(int64_t tile_rows, int64_t max_rows, size_t* bytes) {
  if (!bytes || !extent_ok(tile_rows) || !extent_ok(max_rows))
    return fail(DSV4_ERR_INVALID_ARG, "scratch_bytes: bad arguments");
  size_t n = 0;
  if (!mul_size(static_cast<size_t>(tile_rows),
                static_cast<size_t>(dsv4_score_stride(max_rows)) * sizeof(float), &n))
    return fail(DSV4_ERR_INVALID_ARG, "scratch_bytes: %lld x %lld scores overflow size_t",
                (long long)tile_rows, (long long)max_rows);
  // narrow tiles over long rows: room for the chunk-parallel top-k as well
  // (at most 64 x 2^25 chunks x DSV4_MAX_TOPK x 8 bytes: no overflow)
  if (tile_rows > 0 && tile_rows <= kSplitRows && max_rows > kTopkChunk)
    n += split_ws_bytes(tile_rows, (max_rows + kTopkChunk - 1) / kTopkChunk, DSV4_MAX_TOPK);
  *bytes = n;
  return DSV4_OK;
}

int dsv4_compress(dsv4_pool_cache* cache, const void* x, int64_t n_new, void* stream) {
  int rc = check_cache(cache, "compress");
  if (rc) return rc;
  if (!extent_ok(n_new))
    return fail(DSV4_ERR_INVALID_ARG, "compress: n_new %lld", (long long)n_new);
  if (n_new > 0 && !x) return fail(DSV4_ERR_INVALID_ARG, "compress: NULL input");
  const int64_t L = cache->n_rem + n_new;
  const int64_t groups = L / cache->ratio;
  if (cache->n_rows + groups > cache->capacity)
    return fail(DSV4_ERR_CAPACITY, "compress: %lld + %lld rows exceed capacity %lld",
                (long long)cache->n_rows, (long long)groups, (long long)cache->capacity);
  if (n_new == 0) return DSV4_OK;
  rc = hip_status(dsv4_launch_compress(cache->rows, cache->rem, cache->n_rows, cache->n_rem,
                                       cache->ratio, cache->dim, cache->dtype, x, n_new,
                                       static_cast<hipStream_t>(stream)),
                  "compress launch");
  if (rc) return rc;
  cache->n_rows += groups;
  cache->n_rem = static_cast<int32_t>(L - cache->ratio * groups);
  return DSV4_OK;
}

static int check_scores_args(const dsv4_pool_cache* ic, const void* q, const float* w,
                             int64_t rows, int64_t q_pos0, int32_t n_heads, const char* who) {
  int rc = check_cache(ic, who, 4);
  if (rc) return rc;
  if (ic->dtype != DSV4_BF16) return fail(DSV4_ERR_UNSUPPORTED, "%s: index cache must be bf16", who);
  if (ic->dim != 32 && ic->dim != 64 && ic->dim != 128)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: index dim %d not in {32,64,128}", who, ic->dim);
  if (n_heads < 1 || n_heads > DSV4_MAX_INDEX_HEADS)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: %d indexer heads", who, n_heads);
  if (!extent_ok(rows) || !extent_ok(q_pos0))
    return fail(DSV4_ERR_INVALID_ARG, "%s: rows %lld / q_pos0 %lld", who, (long long)rows,
                (long long)q_pos0);
  if (rows > 0 && (!q || !w)) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL q or w", who);
  if (rows > 0 && (!aligned16(q) || !aligned16(ic->rows)))
    return fail(DSV4_ERR_INVALID_ARG, "%s: q and cache rows must be 16-byte aligned", who);
  if (ic->n_rows > dsv4::kMaxScoreStride)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: %lld pooled rows (at most %lld)", who,
                (long long)ic->n_rows, (long long)dsv4::kMaxScoreStride);
  const int64_t frontier = 4 * ic->n_rows + ic->n_rem;
  if (q_pos0 + rows > frontier)
    return fail(DSV4_ERR_INVALID_ARG,
                "%s: queries up to position %lld are ahead of the compressor frontier %lld", who,
                (long long)(q_pos0 + rows - 1), (long long)frontier);
  return DSV4_OK;
}

int dsv4_indexer_scores(const dsv4_pool_cache* index_cache, const void* q, const float* w,
                        int64_t rows, int64_t q_pos0, int32_t n_heads, int32_t fold_mask,
                        float* out, int64_t out_stride, void* stream) {
  int rc = check_scores_args(index_cache, q, w, rows, q_pos0, n_heads, "indexer_scores");
  if (rc) return rc;
  const int64_t S = index_cache->n_rows;
  if (rows > 0 && S > 0 && !out) return fail(DSV4_ERR_INVALID_ARG, "indexer_scores: NULL out");
  if (out_stride < S) return fail(DSV4_ERR_INVALID_ARG, "indexer_scores: stride < rows of cache");
  if (out_stride > dsv4::kMaxScoreStride)
    return fail(DSV4_ERR_UNSUPPORTED, "indexer_scores: stride %lld (at most %lld)",
                (long long)out_stride, (long long)dsv4::kMaxScoreStride);
  if (rows == 0 || S == 0) return DSV4_OK;
  return hip_status(dsv4_launch_indexer_scores(q, w, index_cache->rows, rows, q_pos0, S, n_heads,
                                               index_cache->dim, fold_mask ? 1 : 0, out,
                                               out_stride, static_cast<hipStream_t>(stream)),
                    "indexer_scores launch");
}

static int check_topk_args(const char* who, const float* scores, int64_t rows, int64_t stride,
                           int64_t q_pos0, int64_t n_cols, int32_t topk,
                           const int32_t* out_idx) {
  if (!extent_ok(rows) || !extent_ok(q_pos0) || !extent_ok(n_cols) || !extent_ok(stride) ||
      stride < n_cols)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", who);
  if (topk < 1 || topk > DSV4_MAX_TOPK)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: topk %d", who, topk);
  if (rows == 0) return DSV4_OK;
  if (!out_idx) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL out", who);
  if (vis_rows(q_pos0 + rows - 1) > n_cols)
    return fail(DSV4_ERR_INVALID_ARG, "%s: visible prefix %lld exceeds %lld columns", who,
                (long long)vis_rows(q_pos0 + rows - 1), (long long)n_cols);
  if (n_cols > 0 && !scores) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL scores", who);
  return DSV4_OK;
}

int dsv4_topk_select(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                     int64_t n_cols, int32_t topk, int32_t* out_idx, void* stream) {
  int rc = check_topk_args("topk_select", scores, rows, stride, q_pos0, n_cols, topk, out_idx);
  if (rc || rows == 0) return rc;
  return hip_status(dsv4_launch_topk(scores, rows, stride, q_pos0, topk, out_idx,
                                     static_cast<hipStream_t>(stream)),
                    "topk launch");
}

int dsv4_topk_split_workspace_bytes(int64_t rows, int64_t q_pos0, int32_t topk, size_t* bytes) {
  if (!bytes || !extent_ok(rows) || !extent_ok(q_pos0) || topk < 1 || topk > DSV4_MAX_TOPK)
    return fail(DSV4_ERR_INVALID_ARG, "topk_split_workspace_bytes: bad arguments");
  *bytes = split_applies(rows, q_pos0, topk)
               ? split_ws_bytes(rows, dsv4_topk_split_chunks(rows, q_pos0), topk)
               : 0;
  return DSV4_OK;
}

// Chunk-parallel top-k when it applies (workspace checked), else the
// one-workgroup-per-row kernel.
static int launch_topk_any(const char* who, const float* scores, int64_t rows, int64_t stride,
                           int64_t q_pos0, int32_t topk, int32_t* out_idx, void* workspace,
                           size_t workspace_bytes, hipStream_t s) {
  if (!split_applies(rows, q_pos0, topk))
    return hip_status(dsv4_launch_topk(scores, rows, stride, q_pos0, topk, out_idx, s),
                      "topk launch");
  const int64_t chunks = dsv4_topk_split_chunks(rows, q_pos0);
  const size_t need = split_ws_bytes(rows, chunks, topk);
  if (!workspace || !aligned16(workspace))
    return fail(DSV4_ERR_INVALID_ARG, "%s: workspace NULL or not 16-byte aligned", who);
  if (workspace_bytes < need)
    return fail(DSV4_ERR_SCRATCH, "%s: workspace %zu bytes, need %zu", who, workspace_bytes,
                need);
  auto* cidx = static_cast<int32_t*>(workspace);
  auto* csc = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  return hip_status(dsv4_launch_topk_split(scores, rows, stride, q_pos0, topk, out_idx, cidx,
                                           csc, s),
                    "topk split launch");
}

int dsv4_topk_select_split(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                           int64_t n_cols, int32_t topk, int32_t* out_idx, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc = check_topk_args("topk_select_split", scores, rows, stride, q_pos0, n_cols, topk,
                           out_idx);
  if (rc || rows == 0) return rc;
  return launch_topk_any("topk_select_split", scores, rows, stride, q_pos0, topk, out_idx,
                         workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int dsv4_indexer_select(const dsv4_pool_cache* index_cache, int64_t n_attn_rows, const void* q,
                        const float* w, int64_t T, int64_t q_pos0, int32_t n_heads, int32_t topk,
                        int32_t tile_rows, float* scratch, size_t scratch_bytes,
                        int32_t* out_idx, int32_t* out_all_pooled, void* stream) {
  int rc = check_cache(index_cache, "indexer_select", 4);
  if (rc) return rc;
  const int64_t S = index_cache->n_rows;
  if (S != n_attn_rows)
    return fail(DSV4_ERR_ROW_MISMATCH,
                "indexer_select: index cache has %lld pooled rows, attention cache %lld",
                (long long)S, (long long)n_attn_rows);
  if (!extent_ok(T) || !extent_ok(q_pos0) || tile_rows < 0)
    return fail(DSV4_ERR_INVALID_ARG, "indexer_select: T %lld / q_pos0 %lld / tile_rows %d",
                (long long)T, (long long)q_pos0, tile_rows);
  if (topk < 1 || topk > DSV4_MAX_TOPK)
    return fail(DSV4_ERR_UNSUPPORTED, "indexer_select: topk %d", topk);
  if (T > 0 && !out_idx) return fail(DSV4_ERR_INVALID_ARG, "indexer_select: NULL out_idx");
  const int64_t frontier = 4 * S + index_cache->n_rem;
  if (q_pos0 + T > frontier)
    return fail(DSV4_ERR_INVALID_ARG,
                "indexer_select: queries up to position %lld are ahead of the compressor "
                "frontier %lld",
                (long long)(q_pos0 + T - 1), (long long)frontier);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int all_pooled = dsv4_indexer_all_pooled(S, topk);
  if (S == 0 || all_pooled) {
    if (T > 0) {
      rc = hip_status(dsv4_launch_fill_sequential(out_idx, T, q_pos0, S, topk, s),
                      "fill_sequential launch");
      if (rc) return rc;
    }
    if (out_all_pooled) *out_all_pooled = all_pooled;
    return DSV4_OK;
  }
  rc = check_scores_args(index_cache, q, w, T, q_pos0, n_heads, "indexer_select");
  if (rc) return rc;
  const int64_t tile = (tile_rows == 0 || tile_rows > T) ? T : tile_rows;
  const int64_t stride = dsv4_score_stride(S);
  const size_t need = static_cast<size_t>(tile) * static_cast<size_t>(stride) * sizeof(float);
  if (T > 0 && (!scratch || scratch_bytes < need))
    return fail(DSV4_ERR_SCRATCH, "indexer_select: scratch %zu bytes, need %zu", scratch_bytes,
                need);
  const auto* qb = static_cast<const uint16_t*>(q);
  for (int64_t t0 = 0; t0 < T; t0 += tile) {
    const int64_t rows = (T - t0) < tile ? (T - t0) : tile;
    rc = hip_status(dsv4_launch_indexer_scores(qb + t0 * n_heads * index_cache->dim,
                                               w + t0 * n_heads, index_cache->rows, rows,
                                               q_pos0 + t0, S, n_heads, index_cache->dim, 1,
                                               scratch, stride, s),
                    "indexer_scores launch");
    if (rc) return rc;
    // a narrow tile over long rows takes the chunk-parallel top-k when the
    // scratch holds its workspace after the tile's scores
    const bool split = split_applies(rows, q_pos0 + t0, topk) &&
                       scratch_bytes >= need + split_ws_bytes(rows,
                                                              dsv4_topk_split_chunks(rows, q_pos0 + t0),
                                                              topk);
    if (dsv4_topk_inplace_applies(scratch, rows, stride, q_pos0 + t0, topk))
      // long rows: two register passes, the chunks' candidates kept in the
      // tile's own score rows
      rc = hip_status(dsv4_launch_topk_inplace(scratch, rows, stride, q_pos0 + t0, topk,
                                               out_idx + t0 * topk, s),
                      "topk launch");
    else if (split)
      rc = launch_topk_any("indexer_select", scratch, rows, stride, q_pos0 + t0, topk,
                           out_idx + t0 * topk, reinterpret_cast<char*>(scratch) + need,
                           scratch_bytes - need, s);
    else
      rc = hip_status(dsv4_launch_topk(scratch, rows, stride, q_pos0 + t0, topk,
                                       out_idx + t0 * topk, s),
                      "topk launch");
    if (rc) return rc;
  }
  if (out_all_pooled) *out_all_pooled = 0;
  return DSV4_OK;
}

// Argument checks shared by the attention entry points (all before any
// enqueue).  *empty is set when there is nothing to do (T == 0).
static int check_attn_args(const char* who, const void* q, int64_t T, int64_t q_pos0,
                           int32_t n_heads, int32_t head_dim, const void* raw_kv,
                           int64_t raw_pos0, int64_t n_raw, int32_t window,
                           const dsv4_pool_cache* attn_cache, const int32_t* sel_idx,
                           int32_t topk, const void* out, bool* empty) {
  *empty = false;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: head_dim %d", who, head_dim);
  // attn_cache == NULL is the window-only (LocalAttention) mode: no pooled
  // keys, so no selection either.
  if (attn_cache) {
    int rc = check_cache(attn_cache, who);
    if (rc) return rc;
    if (attn_cache->dtype != DSV4_BF16)
      return fail(DSV4_ERR_UNSUPPORTED, "%s: attention cache must be bf16", who);
    if (attn_cache->dim != head_dim)
      return fail(DSV4_ERR_INVALID_ARG, "%s: cache dim %d != head_dim %d", who, attn_cache->dim,
                  head_dim);
  } else if (sel_idx) {
    return fail(DSV4_ERR_INVALID_ARG, "%s: selection given without a pool", who);
  }
  if (n_heads < 1 || n_heads > DSV4_MAX_HEADS)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: %d heads", who, n_heads);
  if (window < 1) return fail(DSV4_ERR_INVALID_ARG, "%s: window %d", who, window);
  if (!extent_ok(T) || !extent_ok(q_pos0) || !extent_ok(raw_pos0) || !extent_ok(n_raw))
    return fail(DSV4_ERR_INVALID_ARG, "%s: size or position outside [0, 2^40]", who);
  if (sel_idx && (topk < 1 || topk > DSV4_MAX_TOPK))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: topk %d", who, topk);
  if (T == 0) {
    *empty = true;
    return DSV4_OK;
  }
  if (!q || !raw_kv || !out) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL buffer", who);
  if (!aligned16(q) || !aligned16(raw_kv) || !aligned16(out) ||
      (attn_cache && !aligned16(attn_cache->rows)))
    return fail(DSV4_ERR_INVALID_ARG,
                "%s: q, raw_kv, out and cache rows must be 16-byte aligned", who);
  const int64_t need_lo = (q_pos0 - window + 1) > 0 ? (q_pos0 - window + 1) : 0;
  if (raw_pos0 > need_lo || raw_pos0 + n_raw < q_pos0 + T)
    return fail(DSV4_ERR_INVALID_ARG,
                "%s: raw rows [%lld, %lld) do not cover window positions [%lld, %lld)", who,
                (long long)raw_pos0, (long long)(raw_pos0 + n_raw), (long long)need_lo,
                (long long)(q_pos0 + T));
  if (attn_cache && vis_rows(q_pos0 + T - 1, attn_cache->ratio) > attn_cache->n_rows)
    return fail(DSV4_ERR_INVALID_ARG, "%s: queries see %lld pooled rows, cache holds %lld", who,
                (long long)vis_rows(q_pos0 + T - 1, attn_cache->ratio),
                (long long)attn_cache->n_rows);
  return DSV4_OK;
}

int dsv4_sparse_prefill_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                             int32_t head_dim, float scale, const void* raw_kv, int64_t raw_pos0,
                             int64_t n_raw, int32_t window, const dsv4_pool_cache* attn_cache,
                             const int32_t* sel_idx, int32_t topk, void* out, void* stream) {
  bool empty = false;
  int rc = check_attn_args("sparse_prefill_attn", q, T, q_pos0, n_heads, head_dim, raw_kv,
                           raw_pos0, n_raw, window, attn_cache, sel_idx, topk, out, &empty);
  if (rc || empty) return rc;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  return hip_status(dsv4_launch_sparse_attn(q, T, q_pos0, n_heads, head_dim, sc, raw_kv, raw_pos0,
                                            window, attn_cache ? attn_cache->rows : nullptr,
                                            attn_cache ? attn_cache->ratio : 0, sel_idx,
                                            sel_idx ? topk : 0, out, 1, nullptr, nullptr,
                                            static_cast<hipStream_t>(stream)),
                    "sparse_prefill_attn launch");
}

// Bytes of narrow-attention workspace for T queries split n_splits ways:
// fp32 O [T][n_splits][n_heads][head_dim], then (m, l) [T][n_splits][n_heads][2].
// False when the size does not fit a size_t.
static bool narrow_ws_bytes(int64_t T, int32_t n_splits, int32_t n_heads, int32_t head_dim,
                            size_t* bytes) {
  size_t n = 0;
  return mul_size(static_cast<size_t>(T), static_cast<size_t>(n_splits), &n) &&
         mul_size(n, static_cast<size_t>(n_heads), &n) &&
         mul_size(n, (static_cast<size_t>(head_dim) + 2) * sizeof(float), bytes);
}

int dsv4_sparse_attn_narrow_plan(int64_t T, int32_t n_heads, int32_t head_dim, int32_t window,
                                 int64_t n_pooled_keys, int32_t* n_splits,
                                 size_t* workspace_bytes) {
  if (!n_splits || !workspace_bytes || !extent_ok(T) || n_heads < 1 || n_heads > DSV4_MAX_HEADS ||
      head_dim < 1 || head_dim > 512 || window < 1 || !extent_ok(n_pooled_keys))
    return fail(DSV4_ERR_INVALID_ARG, "sparse_attn_narrow_plan: bad arguments");
  // About one workgroup per CU in all (256), each with at least two 32-key
  // tiles, at most DSV4_MAX_ATTN_SPLITS splits.
  const int64_t tiles = (static_cast<int64_t>(window) + n_pooled_keys + 31) / 32;
  int64_t ns = T > 0 ? (256 + T - 1) / T : 1;
  if (ns > tiles / 2) ns = tiles / 2;
  if (ns > DSV4_MAX_ATTN_SPLITS) ns = DSV4_MAX_ATTN_SPLITS;
  if (ns < 1) ns = 1;
  size_t ws = 0;
  if (ns > 1 && !narrow_ws_bytes(T, static_cast<int32_t>(ns), n_heads, head_dim, &ws))
    return fail(DSV4_ERR_INVALID_ARG, "sparse_attn_narrow_plan: workspace overflows size_t");
  *n_splits = static_cast<int32_t>(ns);
  *workspace_bytes = ws;
  return DSV4_OK;
}

int dsv4_sparse_attn_narrow(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                            int32_t head_dim, float scale, const void* raw_kv, int64_t raw_pos0,
                            int64_t n_raw, int32_t window, const dsv4_pool_cache* attn_cache,
                            const int32_t* sel_idx, int32_t topk, int32_t n_splits,
                            float* workspace, size_t workspace_bytes, void* out, void* stream) {
  bool empty = false;
  int rc = check_attn_args("sparse_attn_narrow", q, T, q_pos0, n_heads, head_dim, raw_kv,
                           raw_pos0, n_raw, window, attn_cache, sel_idx, topk, out, &empty);
  if (rc) return rc;
  if (n_splits < 1 || n_splits > DSV4_MAX_ATTN_SPLITS)
    return fail(DSV4_ERR_UNSUPPORTED, "sparse_attn_narrow: %d splits", n_splits);
  if (empty) return DSV4_OK;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (n_splits > 1) {
    size_t need = 0;
    if (!narrow_ws_bytes(T, n_splits, n_heads, head_dim, &need))
      return fail(DSV4_ERR_INVALID_ARG, "sparse_attn_narrow: workspace overflows size_t");
    if (!workspace || !aligned16(workspace))
      return fail(DSV4_ERR_INVALID_ARG, "sparse_attn_narrow: workspace NULL or not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(DSV4_ERR_SCRATCH, "sparse_attn_narrow: workspace %zu bytes, need %zu",
                  workspace_bytes, need);
    part_o = workspace;
    part_ml = workspace + static_cast<size_t>(T) * n_splits * n_heads * head_dim;
  }
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = hip_status(dsv4_launch_sparse_attn(q, T, q_pos0, n_heads, head_dim, sc, raw_kv, raw_pos0,
                                          window, attn_cache ? attn_cache->rows : nullptr,
                                          attn_cache ? attn_cache->ratio : 0, sel_idx,
                                          sel_idx ? topk : 0, out, n_splits, part_o, part_ml, s),
                  "sparse_attn_narrow launch");
  if (rc || n_splits == 1) return rc;
  return hip_status(dsv4_launch_attn_combine(part_o, part_ml, T, n_splits, n_heads, head_dim, out, s),
                    "sparse_attn_narrow combine launch");
}

}  // extern "C"
