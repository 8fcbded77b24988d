// dsv4_indexer_select_noalloc: the whole indexer step (dsv4_indexer_select)
// for callers that cannot allocate device memory -- code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc.  The score
// scratch is a file-scope device array of DSV4_NOALLOC_SCRATCH_BYTES, one per
// GPU, held until the process ends; the call itself allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and every use below goes through that address.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/dsv4.h"
#include "dsv4_device.h"

static __device__ __align__(256) unsigned char scratch[DSV4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// device's first call, then reused).
int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return dsv4_internal_fail(DSV4_ERR_HIP, "indexer_select_noalloc: hipGetDevice: %s",
                              hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dsv4_internal_fail(DSV4_ERR_UNSUPPORTED, "indexer_select_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dsv4_internal_fail(DSV4_ERR_HIP,
                                "indexer_select_noalloc: hipGetSymbolAddress: %s",
                                hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DSV4_OK;
}

}  // namespace

extern "C" int dsv4_indexer_select_noalloc(const dsv4_pool_cache* index_cache,
                                           int64_t n_attn_rows, const void* q, const float* w,
                                           int64_t T, int64_t q_pos0, int32_t n_heads,
                                           int32_t topk, int32_t tile_rows, int32_t* out_idx,
                                           int32_t* out_all_pooled, void* stream) {
  if (!index_cache)
    return dsv4_internal_fail(DSV4_ERR_INVALID_ARG, "indexer_select_noalloc: NULL cache");
  if (T < 0 || tile_rows < 0)
    return dsv4_internal_fail(DSV4_ERR_INVALID_ARG, "indexer_select_noalloc: negative size");
  const int64_t S = index_cache->n_rows;
  // the full path (the others need no scratch); a pool count outside
  // [0, DSV4_MAX_EXTENT] takes no scratch and fails the cache checks below
  const bool scores = T > 0 && S > topk && S <= DSV4_MAX_EXTENT;
  const size_t row_bytes =
      scores ? static_cast<size_t>(dsv4_score_stride(S)) * sizeof(float) : sizeof(float);
  const size_t cap = DSV4_NOALLOC_SCRATCH_BYTES;
  const int64_t fit = static_cast<int64_t>(cap / row_bytes);  // score rows the array holds
  int64_t tile = (tile_rows == 0 || tile_rows > T) ? T : tile_rows;
  if (scores && tile_rows == 0 && fit < tile) tile = fit;
  if (scores && (tile < 1 || tile > fit))
    return dsv4_internal_fail(DSV4_ERR_SCRATCH,
                              "indexer_select_noalloc: a %lld-row tile of %lld pooled rows does "
                              "not fit the static scratch of %zu bytes (%lld rows of them do)",
                              static_cast<long long>(tile < 1 ? 1 : tile),
                              static_cast<long long>(S), cap, static_cast<long long>(fit));
  void* p = nullptr;
  if (scores) {
    const int rc = device_scratch(&p);
    if (rc) return rc;
  }
  return dsv4_indexer_select(index_cache, n_attn_rows, q, w, T, q_pos0, n_heads, topk,
                             scores ? static_cast<int32_t>(tile) : 0, static_cast<float*>(p),
                             scores ? cap : 0, out_idx, out_all_pooled, stream);
}
