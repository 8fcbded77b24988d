/* Plain C99 client of include/dsv4.h: host-only calls and argument checks
 * (nothing here reaches a GPU; every call either needs no device or fails
 * validation before any enqueue).  Exit status 0 iff every check holds. */
#include <stdio.h>
#include <string.h>

#include "dsv4.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  size_t bytes = 0;
  dsv4_pool_cache c;
  int32_t ns = 0;
  CHECK(dsv4_abi_version() == DSV4_ABI_VERSION);
  CHECK(dsv4_indexer_all_pooled(0, 8) == 0);
  CHECK(dsv4_indexer_all_pooled(8, 8) == 1);
  CHECK(dsv4_indexer_all_pooled(9, 8) == 0);
  CHECK(dsv4_score_stride(65) == 128);
  CHECK(dsv4_indexer_scratch_bytes(1024, 262144, &bytes) == DSV4_OK);
  CHECK(bytes == (size_t)1 << 30);
  CHECK(dsv4_indexer_scratch_bytes(-1, 10, &bytes) == DSV4_ERR_INVALID_ARG);
  CHECK(strlen(dsv4_last_error()) > 0);
  CHECK(dsv4_topk_split_workspace_bytes(1, (1 << 20) - 4, 2048, &bytes) == DSV4_OK);
  CHECK(bytes == (size_t)2 * 8 * 2048 * 4);
  CHECK(dsv4_sparse_attn_narrow_plan(1, 64, 512, 128, 2048, &ns, &bytes) == DSV4_OK);
  CHECK(ns == 34 && bytes == (size_t)34 * 64 * 514 * 4);

  /* a cache struct with a NULL remainder buffer is rejected before any enqueue */
  memset(&c, 0, sizeof(c));
  c.capacity = 16;
  c.ratio = 4;
  c.dim = 128;
  c.dtype = DSV4_BF16;
  c.rows = (void*)0x1000;
  c.rem = NULL;
  CHECK(dsv4_compress(&c, (const void*)0x1000, 4, NULL) == DSV4_ERR_INVALID_ARG);
  CHECK(c.n_rows == 0 && c.n_rem == 0);
  c.rem = (void*)0x1000;
  c.ratio = DSV4_MAX_RATIO + 1;
  CHECK(dsv4_compress(&c, (const void*)0x1000, 4, NULL) == DSV4_ERR_UNSUPPORTED);
  /* window-only attention with a selection is an argument error */
  CHECK(dsv4_sparse_prefill_attn((const void*)0x1000, 4, 100, 64, 512, 0.0f, (const void*)0x1000, 0,
                                 104, 128, NULL, (const int32_t*)0x1000, 16, (void*)0x1000,
                                 NULL) == DSV4_ERR_INVALID_ARG);
  if (failures == 0) printf("abi_check: ok\n");
  return failures == 0 ? 0 : 1;
}
