/* Host-side sweep of every entry point of include/dsv4.h, meant to run with
 * the library's host code built under AddressSanitizer and
 * UndefinedBehaviorSanitizer (see tests/test_host_sanitize.py).
 *
 * Each entry point is called many times with arguments drawn from tables of
 * boundary and extreme values (negative, zero, small, around the kernels'
 * limits, around DSV4_MAX_EXTENT, up to INT64_MAX), NULL / aligned /
 * misaligned pointers and cache structs with arbitrary fields.  Nothing here
 * may reach a GPU: the program refuses to run where one is visible, and
 * without one every launch fails cleanly with DSV4_ERR_HIP.  Device pointers
 * are never dereferenced on the host, so the fake addresses below are safe.
 *
 * Checked beside what the sanitizers catch:
 *   - every return code is DSV4_OK or a documented error code;
 *   - on an error the caller's structs and out-flags are unchanged and
 *     dsv4_last_error() is a non-empty NUL-terminated string;
 *   - the size queries honour their documented limits and never shrink as
 *     the pooled row count grows;
 *   - every launching entry point passed all of its checks at least once
 *     (reaching the launch, which fails here) and was refused at least once.
 * Exit status 0 iff every check holds; 77 when a GPU is visible (skipped). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <unistd.h>

#include "dsv4.h"

static int failures = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      if (failures < 20)                                                     \
        fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);    \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

/* xorshift64*: a seeded draw for the argument tables */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t draw(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
#define PICK(table) (table[draw() % (sizeof(table) / sizeof(table[0]))])

static const int64_t I64[] = {INT64_MIN, INT64_MIN + 1, -4096, -1, 0, 1, 2, 3, 4, 15, 16,
                              63, 64, 65, 127, 128, 512, 1023, 1024, 2047, 2048, 4096, 4097,
                              32767, 32768, 32769, 262144, (int64_t)1 << 28, (int64_t)1 << 31,
                              DSV4_MAX_EXTENT - 1, DSV4_MAX_EXTENT, DSV4_MAX_EXTENT + 1,
                              (int64_t)1 << 62, INT64_MAX - 64, INT64_MAX - 63, INT64_MAX - 1,
                              INT64_MAX};
static const int32_t I32[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 8, 16, 31, 32, 33, 64, 65, 127,
                              128, 129, 256, 257, 512, 2048, 4095, 4096, 4097, 5160, 65536,
                              INT32_MAX - 1, INT32_MAX};
static const size_t SZ[] = {0, 1, 15, 16, 4096, (size_t)1 << 20, (size_t)1 << 30,
                            (size_t)1 << 40, SIZE_MAX / 2, SIZE_MAX};
static void* const PTR[] = {NULL, (void*)0x10000, (void*)0x10008, (void*)0x7f0000000000};

/* return codes seen per launching entry point: seen[entry][-rc] */
enum { E_COMPRESS, E_SCORES, E_SELECT, E_NOALLOC, E_TOPK, E_TOPK_SPLIT, E_ATTN, E_NARROW,
       E_COUNT };
static const char* const entry_name[E_COUNT] = {
    "compress", "indexer_scores", "indexer_select", "indexer_select_noalloc", "topk_select",
    "topk_select_split", "sparse_prefill_attn", "sparse_attn_narrow"};
static long seen[E_COUNT][7];

/* a documented code, and on an error a message; counted for `entry` (-1: a
 * size query, not counted) */
static void check_rc(int entry, int rc) {
  CHECK(rc == DSV4_OK || rc == DSV4_ERR_INVALID_ARG || rc == DSV4_ERR_UNSUPPORTED ||
        rc == DSV4_ERR_CAPACITY || rc == DSV4_ERR_ROW_MISMATCH || rc == DSV4_ERR_SCRATCH ||
        rc == DSV4_ERR_HIP);
  if (entry >= 0 && rc <= 0 && rc >= -6) ++seen[entry][-rc];
  if (rc == DSV4_OK) return;
  const char* e = dsv4_last_error();
  CHECK(e != NULL);
  if (e) {
    size_t n = 0;
    while (n < 4096 && e[n]) ++n;
    CHECK(n > 0 && n < 4096);
  }
}

static void random_cache(dsv4_pool_cache* c) {
  c->rows = PICK(PTR);
  c->rem = PICK(PTR);
  c->capacity = PICK(I64);
  c->n_rows = PICK(I64);
  c->n_rem = PICK(I32);
  c->ratio = (draw() & 1) ? 4 : PICK(I32);
  c->dim = PICK(I32);
  c->dtype = (int32_t)(draw() % 4);
}

/* a cache that passes the struct checks, so the sweep reaches the checks
 * behind them */
static void plausible_cache(dsv4_pool_cache* c, int32_t dim) {
  c->rows = (void*)0x10000;
  c->rem = (void*)0x20000;
  c->capacity = PICK(I64);
  if (c->capacity < 0) c->capacity = -(c->capacity + 1);
  if (c->capacity > DSV4_MAX_EXTENT && (draw() & 1)) c->capacity = DSV4_MAX_EXTENT;
  c->n_rows = (draw() & 1) ? c->capacity : (int64_t)(draw() % 40000);
  if (c->n_rows > c->capacity) c->n_rows = c->capacity;
  c->n_rem = (int32_t)(draw() % 4);
  c->ratio = 4;
  c->dim = dim;
  c->dtype = DSV4_BF16;
}

static dsv4_pool_cache any_cache(int32_t dim) {
  dsv4_pool_cache c;
  memset(&c, 0, sizeof(c));
  if (draw() % 3 == 0) random_cache(&c);
  else plausible_cache(&c, dim);
  return c;
}

static void sweep_size_queries(int n) {
  for (int i = 0; i < n; ++i) {
    const int64_t a = PICK(I64), b = PICK(I64);
    const int32_t k = PICK(I32);
    (void)dsv4_indexer_all_pooled(a, k);
    const int64_t s = dsv4_score_stride(a);
    if (a <= 0) CHECK(s == 64);
    else if (a <= DSV4_MAX_EXTENT) CHECK(s >= a && s % 64 == 0 && s - a < 64);
    else CHECK(s == -1);

    size_t bytes = 12345, bytes2 = 0;
    int rc = dsv4_indexer_scratch_bytes(a, b, &bytes);
    check_rc(-1, rc);
    if (a > DSV4_MAX_EXTENT || b > DSV4_MAX_EXTENT || a < 0 || b < 0)
      CHECK(rc == DSV4_ERR_INVALID_ARG);
    if (rc == DSV4_OK && b < DSV4_MAX_EXTENT && dsv4_indexer_scratch_bytes(a, b + 1, &bytes2) == DSV4_OK)
      CHECK(bytes2 >= bytes); /* more pooled rows never need less scratch */
    CHECK(dsv4_indexer_scratch_bytes(a, b, NULL) == DSV4_ERR_INVALID_ARG);

    rc = dsv4_topk_split_workspace_bytes(a, b, k, &bytes);
    check_rc(-1, rc);

    int32_t ns = -7;
    rc = dsv4_sparse_attn_narrow_plan(a, PICK(I32), PICK(I32), PICK(I32), b, &ns, &bytes);
    check_rc(-1, rc);
    if (rc == DSV4_OK) CHECK(ns >= 1 && ns <= DSV4_MAX_ATTN_SPLITS);
    else CHECK(ns == -7);
    CHECK(dsv4_sparse_attn_narrow_plan(a, 64, 512, 128, b, NULL, &bytes) == DSV4_ERR_INVALID_ARG);
  }
}

static void sweep_compress(int n) {
  for (int i = 0; i < n; ++i) {
    dsv4_pool_cache c = any_cache((draw() & 1) ? 128 : 512);
    if (draw() % 4 == 0) c.dtype = DSV4_F32;
    const dsv4_pool_cache before = c;
    const int rc = dsv4_compress((draw() % 8) ? &c : NULL, PICK(PTR), PICK(I64), NULL);
    check_rc(E_COMPRESS, rc);
    if (rc != DSV4_OK) CHECK(memcmp(&c, &before, sizeof(c)) == 0);
  }
}

static void sweep_indexer(int n) {
  for (int i = 0; i < n; ++i) {
    const int32_t dims[] = {32, 64, 128, 96, PICK(I32)};
    dsv4_pool_cache c = any_cache(dims[draw() % 5]);
    const dsv4_pool_cache before = c;
    int rc = dsv4_indexer_scores((draw() % 8) ? &c : NULL, PICK(PTR), (const float*)PICK(PTR),
                                 PICK(I64), PICK(I64), PICK(I32), (int32_t)(draw() & 1),
                                 (float*)PICK(PTR), PICK(I64), NULL);
    check_rc(E_SCORES, rc);
    CHECK(memcmp(&c, &before, sizeof(c)) == 0);

    int32_t all_pooled = -7;
    const int64_t n_attn = (draw() % 4) ? c.n_rows : PICK(I64);
    rc = dsv4_indexer_select((draw() % 8) ? &c : NULL, n_attn, PICK(PTR), (const float*)PICK(PTR),
                             PICK(I64), PICK(I64), PICK(I32), PICK(I32), PICK(I32),
                             (float*)PICK(PTR), PICK(SZ), (int32_t*)PICK(PTR),
                             (draw() & 1) ? &all_pooled : NULL, NULL);
    check_rc(E_SELECT, rc);
    if (rc != DSV4_OK && rc != DSV4_ERR_HIP) CHECK(all_pooled == -7);
    CHECK(memcmp(&c, &before, sizeof(c)) == 0);

    all_pooled = -7;
    rc = dsv4_indexer_select_noalloc((draw() % 8) ? &c : NULL, n_attn, PICK(PTR),
                                     (const float*)PICK(PTR), PICK(I64), PICK(I64), PICK(I32),
                                     PICK(I32), PICK(I32), (int32_t*)PICK(PTR),
                                     (draw() & 1) ? &all_pooled : NULL, NULL);
    check_rc(E_NOALLOC, rc);
    if (rc != DSV4_OK && rc != DSV4_ERR_HIP) CHECK(all_pooled == -7);
    CHECK(memcmp(&c, &before, sizeof(c)) == 0);
  }
}

static void sweep_topk(int n) {
  for (int i = 0; i < n; ++i) {
    int rc = dsv4_topk_select((const float*)PICK(PTR), PICK(I64), PICK(I64), PICK(I64), PICK(I64),
                              PICK(I32), (int32_t*)PICK(PTR), NULL);
    check_rc(E_TOPK, rc);
    rc = dsv4_topk_select_split((const float*)PICK(PTR), PICK(I64), PICK(I64), PICK(I64),
                                PICK(I64), PICK(I32), (int32_t*)PICK(PTR), PICK(PTR), PICK(SZ),
                                NULL);
    check_rc(E_TOPK_SPLIT, rc);
  }
}

/* attention arguments: either drawn from the tables, or consistent ones
 * (raw rows covering the window, a pool holding the visible rows) with one
 * field at a time left to the tables, so the later checks are reached too */
typedef struct {
  int64_t T, q_pos0, raw_pos0, n_raw;
  int32_t n_heads, window, topk, n_splits;
  size_t ws_bytes;
} attn_args;

static attn_args any_attn_args(dsv4_pool_cache* c) {
  attn_args a;
  if (draw() & 1) {
    a.T = PICK(I64);
    a.q_pos0 = PICK(I64);
    a.raw_pos0 = PICK(I64);
    a.n_raw = PICK(I64);
    a.n_heads = PICK(I32);
    a.window = PICK(I32);
    a.topk = PICK(I32);
    a.n_splits = PICK(I32);
    a.ws_bytes = PICK(SZ);
    return a;
  }
  a.T = 1 + (int64_t)(draw() % 4096);
  a.q_pos0 = (int64_t)(draw() % 1000000);
  a.window = (draw() & 1) ? 128 : 1 + (int32_t)(draw() % 300);
  a.raw_pos0 = a.q_pos0 - a.window + 1 > 0 ? a.q_pos0 - a.window + 1 : 0;
  a.raw_pos0 -= a.raw_pos0 > 0 ? (int64_t)(draw() % 2) : 0;
  a.n_raw = a.q_pos0 + a.T - a.raw_pos0 + (int64_t)(draw() % 3) - 1;
  a.n_heads = 1 + (int32_t)(draw() % 64);
  a.topk = 1 + (int32_t)(draw() % DSV4_MAX_TOPK);
  a.n_splits = 1 + (int32_t)(draw() % DSV4_MAX_ATTN_SPLITS);
  a.ws_bytes = (size_t)a.T * (size_t)a.n_splits * (size_t)a.n_heads * 514u * 4u;
  if (c->ratio >= 2 && c->ratio <= DSV4_MAX_RATIO) {
    const int64_t vis = (a.q_pos0 + a.T) / c->ratio;
    if (c->capacity < vis && c->capacity >= 0 && (draw() & 1)) c->capacity = vis;
    if (c->capacity >= vis && (draw() & 1)) c->n_rows = vis;
  }
  switch (draw() % 8) {  /* one field from the tables */
    case 0: a.T = PICK(I64); break;
    case 1: a.q_pos0 = PICK(I64); break;
    case 2: a.raw_pos0 = PICK(I64); break;
    case 3: a.n_raw = PICK(I64); break;
    case 4: a.window = PICK(I32); break;
    case 5: a.n_splits = PICK(I32); break;
    case 6: a.ws_bytes = PICK(SZ); break;
    default: break;
  }
  return a;
}

static void sweep_attention(int n) {
  for (int i = 0; i < n; ++i) {
    const int32_t dims[] = {32, 64, 128, 256, 512, PICK(I32)};
    const int32_t hd = dims[draw() % 6];
    dsv4_pool_cache c = any_cache(hd);
    if (draw() % 4 == 0) c.ratio = (draw() & 1) ? 128 : PICK(I32);
    const attn_args a = any_attn_args(&c);
    const dsv4_pool_cache before = c;
    const dsv4_pool_cache* cp = (draw() % 4) ? &c : NULL;
    const int32_t* sel = (cp && (draw() % 4)) ? (const int32_t*)0x30000 : (const int32_t*)PICK(PTR);
    void* const q = (draw() % 8) ? (void*)0x40000 : PICK(PTR);
    void* const raw = (draw() % 8) ? (void*)0x50000 : PICK(PTR);
    void* const out = (draw() % 8) ? (void*)0x60000 : PICK(PTR);
    float* const ws = (draw() % 8) ? (float*)0x70000 : (float*)PICK(PTR);
    const float scales[] = {0.f, -1.f, 0.0441941738f, 1e30f};
    int rc = dsv4_sparse_prefill_attn(q, a.T, a.q_pos0, a.n_heads, hd, scales[draw() % 4], raw,
                                      a.raw_pos0, a.n_raw, a.window, cp, sel, a.topk, out, NULL);
    check_rc(E_ATTN, rc);
    CHECK(memcmp(&c, &before, sizeof(c)) == 0);
    rc = dsv4_sparse_attn_narrow(q, a.T, a.q_pos0, a.n_heads, hd, scales[draw() % 4], raw,
                                 a.raw_pos0, a.n_raw, a.window, cp, sel, a.topk, a.n_splits, ws,
                                 a.ws_bytes, out, NULL);
    check_rc(E_NARROW, rc);
    CHECK(memcmp(&c, &before, sizeof(c)) == 0);
  }
}

int main(void) {
  if (access("/dev/kfd", F_OK) == 0) {
    printf("host_sanitize_check: skipped (a GPU is visible)\n");
    return 77;
  }
  CHECK(dsv4_abi_version() == DSV4_ABI_VERSION);
  sweep_size_queries(20000);
  sweep_compress(20000);
  sweep_indexer(20000);
  sweep_topk(20000);
  sweep_attention(20000);
  for (int e = 0; e < E_COUNT; ++e) {
    printf("%-24s ok %6ld  invalid %6ld  unsupported %6ld  capacity %5ld  rows %5ld  "
           "scratch %5ld  launch %5ld\n",
           entry_name[e], seen[e][0], seen[e][1], seen[e][2], seen[e][3], seen[e][4], seen[e][5],
           seen[e][6]);
    CHECK(seen[e][-DSV4_ERR_HIP] > 0);
    CHECK(seen[e][-DSV4_ERR_INVALID_ARG] > 0);
  }
  if (failures == 0) printf("host_sanitize_check: ok\n");
  else fprintf(stderr, "host_sanitize_check: %d failed checks\n", failures);
  return failures == 0 ? 0 : 1;
}
