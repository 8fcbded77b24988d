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
  if (c->capacity < 0 || c->n_rows < 0 || c->n_rows > c->capacity)
    return fail(DSV4_ERR_INVALID_ARG, "%s: n_rows %lld / capacity %lld", name,
                (long long)c->n_rows, (long long)c->capacity);
  if (c->n_rem < 0 || c->n_rem >= c->ratio)
    return fail(DSV4_ERR_INVALID_ARG, "%s: n_rem %d", name, c->n_rem);
  if (c->capacity > 0 && !c->rows) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL rows", name);
  if (!c->rem) return fail(DSV4_ERR_INVALID_ARG, "%s: NULL remainder buffer", name);
  return DSV4_OK;
}

inline int64_t vis_rows(int64_t p, int ratio = 4) { return (p + 1) / ratio; }

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
  return (n_rows + 63) / 64 * 64;
}

int dsv4_indexer_scratch_bytes(int64_t tile_rows, int64_t max_rows, size_t* bytes) {
  if (!bytes || tile_rows < 0 || max_rows < 0)
    return fail(DSV4_ERR_INVALID_ARG, "scratch_bytes: bad arguments");
  *bytes = static_cast<size_t>(tile_rows) * static_cast<size_t>(dsv4_score_stride(max_rows)) *
           sizeof(float);
  return DSV4_OK;
}

int dsv4_compress(dsv4_pool_cache* cache, const void* x, int64_t n_new, void* stream) {
  int rc = check_cache(cache, "compress");
  if (rc) return rc;
  if (n_new < 0) return fail(DSV4_ERR_INVALID_ARG, "compress: n_new %lld", (long long)n_new);
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
  if (rows < 0 || q_pos0 < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: rows/q_pos0 negative", who);
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

int dsv4_topk_select(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                     int64_t n_cols, int32_t topk, int32_t* out_idx, void* stream) {
  if (rows < 0 || q_pos0 < 0 || n_cols < 0 || stride < n_cols)
    return fail(DSV4_ERR_INVALID_ARG, "topk_select: bad sizes");
  if (topk < 1 || topk > DSV4_MAX_TOPK)
    return fail(DSV4_ERR_UNSUPPORTED, "topk_select: topk %d", topk);
  if (rows == 0) return DSV4_OK;
  if (!out_idx) return fail(DSV4_ERR_INVALID_ARG, "topk_select: NULL out");
  if (vis_rows(q_pos0 + rows - 1) > n_cols)
    return fail(DSV4_ERR_INVALID_ARG, "topk_select: visible prefix %lld exceeds %lld columns",
                (long long)vis_rows(q_pos0 + rows - 1), (long long)n_cols);
  if (n_cols > 0 && !scores) return fail(DSV4_ERR_INVALID_ARG, "topk_select: NULL scores");
  return hip_status(dsv4_launch_topk(scores, rows, stride, q_pos0, topk, out_idx,
                                     static_cast<hipStream_t>(stream)),
                    "topk launch");
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
  if (T < 0 || q_pos0 < 0 || tile_rows < 0)
    return fail(DSV4_ERR_INVALID_ARG, "indexer_select: negative size");
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
    rc = hip_status(dsv4_launch_topk(scratch, rows, stride, q_pos0 + t0, topk,
                                     out_idx + t0 * topk, s),
                    "topk launch");
    if (rc) return rc;
  }
  if (out_all_pooled) *out_all_pooled = 0;
  return DSV4_OK;
}

int dsv4_sparse_prefill_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                             int32_t head_dim, float scale, const void* raw_kv, int64_t raw_pos0,
                             int64_t n_raw, int32_t window, const dsv4_pool_cache* attn_cache,
                             const int32_t* sel_idx, int32_t topk, void* out, void* stream) {
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(DSV4_ERR_UNSUPPORTED, "sparse_prefill_attn: head_dim %d", head_dim);
  // attn_cache == NULL is the window-only (LocalAttention) mode: no pooled
  // keys, so no selection either.
  if (attn_cache) {
    int rc = check_cache(attn_cache, "sparse_prefill_attn");
    if (rc) return rc;
    if (attn_cache->dtype != DSV4_BF16)
      return fail(DSV4_ERR_UNSUPPORTED, "sparse_prefill_attn: attention cache must be bf16");
    if (attn_cache->dim != head_dim)
      return fail(DSV4_ERR_INVALID_ARG, "sparse_prefill_attn: cache dim %d != head_dim %d",
                  attn_cache->dim, head_dim);
  } else if (sel_idx) {
    return fail(DSV4_ERR_INVALID_ARG, "sparse_prefill_attn: selection given without a pool");
  }
  if (n_heads < 1 || n_heads > DSV4_MAX_HEADS)
    return fail(DSV4_ERR_UNSUPPORTED, "sparse_prefill_attn: %d heads", n_heads);
  if (window < 1) return fail(DSV4_ERR_INVALID_ARG, "sparse_prefill_attn: window %d", window);
  if (T < 0 || q_pos0 < 0 || raw_pos0 < 0 || n_raw < 0)
    return fail(DSV4_ERR_INVALID_ARG, "sparse_prefill_attn: negative size");
  if (sel_idx && (topk < 1 || topk > DSV4_MAX_TOPK))
    return fail(DSV4_ERR_UNSUPPORTED, "sparse_prefill_attn: topk %d", topk);
  if (T == 0) return DSV4_OK;
  if (!q || !raw_kv || !out) return fail(DSV4_ERR_INVALID_ARG, "sparse_prefill_attn: NULL buffer");
  if (!aligned16(q) || !aligned16(raw_kv) || (attn_cache && !aligned16(attn_cache->rows)))
    return fail(DSV4_ERR_INVALID_ARG,
                "sparse_prefill_attn: q, raw_kv and cache rows must be 16-byte aligned");
  const int64_t need_lo = (q_pos0 - window + 1) > 0 ? (q_pos0 - window + 1) : 0;
  if (raw_pos0 > need_lo || raw_pos0 + n_raw < q_pos0 + T)
    return fail(DSV4_ERR_INVALID_ARG,
                "sparse_prefill_attn: raw rows [%lld, %lld) do not cover window positions "
                "[%lld, %lld)",
                (long long)raw_pos0, (long long)(raw_pos0 + n_raw), (long long)need_lo,
                (long long)(q_pos0 + T));
  const int ratio = attn_cache ? attn_cache->ratio : 0;
  if (attn_cache && vis_rows(q_pos0 + T - 1, ratio) > attn_cache->n_rows)
    return fail(DSV4_ERR_INVALID_ARG,
                "sparse_prefill_attn: queries see %lld pooled rows, cache holds %lld",
                (long long)vis_rows(q_pos0 + T - 1, ratio), (long long)attn_cache->n_rows);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  return hip_status(dsv4_launch_sparse_attn(q, T, q_pos0, n_heads, head_dim, sc, raw_kv, raw_pos0,
                                            window, attn_cache ? attn_cache->rows : nullptr,
                                            ratio, sel_idx,
                                            sel_idx ? topk : 0, out,
                                            static_cast<hipStream_t>(stream)),
                    "sparse_prefill_attn launch");
}

}  // extern "C"
