// Pooling compressor (ratio 4 for the indexer and sparse attention, ratio
// 128 for the CompressedAttention mode) with in-place append and remainder
// carry, and the all-pooled sequential selection fill.
//
// Compressor [P1 "perf(deepseek-v4): skip redundant all-pooled indexer
// scoring", Correctness: 10 tokens -> 2 pooled rows + 2-token remainder;
// P2 "perf(deepseek_v4): faster exact DeepSeek-V4 prefill", commit 4: pooled
// rows appended in place; commit 1 and the ratio-128 prefill routing it
// builds on].  Each pooled row is the mean of r consecutive raw rows of (old
// remainder ++ new rows): float32 sum left to right, times 1/r (exact for a
// power of two), rounded to the storage type with ties to even.  Contraction
// is off so the sum order and roundings are exactly that; the loads of a
// group are issued eight at a time ahead of the adds, which stay in order.
//
// Memory traffic is one read of each raw element and one write per pooled
// element; the kernel is HBM/launch bound and tiny (a 2,048-token chunk of
// 512-wide bf16 rows is 2 MiB in, 0.5 MiB out at ratio 4).
//
// Remainder hazard: only group 0 can read the old remainder, and the thread
// that pools column c of group 0 is the one that writes column c of the new
// remainder, after its read; no other thread touches the remainder.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {  // bf16 storage
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};

template <typename T>
__global__ void __launch_bounds__(256) compress_kernel(T* __restrict__ rows, T* __restrict__ rem,
                                                       int64_t n_rows, int n_rem, int dim,
                                                       const T* __restrict__ x, int64_t n_new,
                                                       int ratio, float inv_ratio, int64_t groups,
                                                       int64_t work_groups) {
#pragma clang fp contract(off)
  const int64_t total = work_groups * dim;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / dim;  // group
    const int c = static_cast<int>(i - j * dim);
    if (j < groups) {
      auto elem = [&](int64_t e) -> float {  // element e of (rem ++ x)
        return (e < n_rem) ? Elem<T>::load(rem + e * dim + c)
                           : Elem<T>::load(x + (e - n_rem) * dim + c);
      };
      const int64_t e0 = static_cast<int64_t>(ratio) * j;
      float acc = elem(e0);
      int r = 1;
      for (; r + 8 <= ratio; r += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = elem(e0 + r + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = acc + v[u];
      }
      for (; r < ratio; ++r) acc = acc + elem(e0 + r);
      Elem<T>::store(rows + (n_rows + j) * dim + c, acc * inv_ratio);
    }
    if (j == 0) {
      // New remainder = (rem ++ x)[ratio*groups, n_rem + n_new).
      const int64_t L = n_rem + n_new;
      const int64_t new_len = L - ratio * groups;
      for (int64_t r = 0; r < new_len; ++r) {
        const int64_t e = ratio * groups + r;
        if (e < n_rem) continue;  // only when groups == 0: already in place
        rem[r * dim + c] = x[(e - n_rem) * dim + c];
      }
    }
  }
}

__global__ void __launch_bounds__(256) fill_sequential_kernel(int32_t* __restrict__ out, int64_t T,
                                                              int64_t q_pos0, int64_t S, int topk) {
  const int64_t total = T * topk;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / topk;
    const int j = static_cast<int>(i - t * topk);
    int64_t v = visible_rows(q_pos0 + t);
    if (v > S) v = S;
    out[i] = (j < v) ? j : -1;
  }
}

inline unsigned grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g);
}

}  // namespace

hipError_t dsv4_launch_compress(void* rows, void* rem, int64_t n_rows, int32_t n_rem,
                                int32_t ratio, int32_t dim, int32_t dtype, const void* x,
                                int64_t n_new, hipStream_t s) {
  if (ratio < 1) return hipErrorInvalidValue;
  const int64_t L = n_rem + n_new;
  const int64_t groups = L / ratio;
  const float inv = 1.0f / static_cast<float>(ratio);
  const int64_t work_groups = groups > 0 ? groups : 1;
  const unsigned grid = grid_for(work_groups * dim);
  if (dtype == 1) {
    hipLaunchKernelGGL(compress_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<uint16_t*>(rows), static_cast<uint16_t*>(rem), n_rows, n_rem,
                       dim, static_cast<const uint16_t*>(x), n_new, ratio, inv, groups,
                       work_groups);
  } else {
    hipLaunchKernelGGL(compress_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<float*>(rows), static_cast<float*>(rem), n_rows, n_rem, dim,
                       static_cast<const float*>(x), n_new, ratio, inv, groups, work_groups);
  }
  return hipGetLastError();
}

hipError_t dsv4_launch_fill_sequential(int32_t* out, int64_t T, int64_t q_pos0, int64_t S,
                                       int32_t topk, hipStream_t s) {
  const unsigned grid = grid_for(T * topk);
  hipLaunchKernelGGL(fill_sequential_kernel, dim3(grid), dim3(256), 0, s, out, T, q_pos0, S,
                     topk);
  return hipGetLastError();
}
