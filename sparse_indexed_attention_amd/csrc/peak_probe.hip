// Ceiling probes for the benchmark (libdsv4_probe.so, not part of the C ABI
// of the hot path): what this MI355X reaches on plain MFMA and copy work, so
// kernel rates can be set beside a measured ceiling as well as the spec one.
//
//   dsv4_probe_mfma  -- a register-resident loop of v_mfma_f32_32x32x16_bf16
//                       (the score kernel's instruction) over varied non-zero
//                       bf16 operands, four independent accumulator chains
//                       per wave, two waves per SIMD on every CU.  Wave 0 of
//                       workgroup 0 also stamps the shader clock counter
//                       (s_memtime) and the 100 MHz real-time counter
//                       (s_memrealtime) at its start and end, giving the
//                       engine clock under MFMA load.
//   dsv4_probe_copy  -- a 16-byte-per-lane grid-stride copy (reads n bytes,
//                       writes n bytes).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lcg(uint32_t& x) {
  x = x * 1664525u + 1013904223u;
  return x;
}

// bf16 in [-1, -0.5) U [0.5, 1): never zero, mantissa bits varied.
__device__ __forceinline__ __bf16 rand_bf16(uint32_t& x) {
  const uint32_t r = lcg(x);
  const uint32_t bits = 0x3f000000u | ((r >> 9) & 0x7f0000u) | (r & 0x80000000u);
  return __builtin_bit_cast(__bf16, static_cast<uint16_t>(bits >> 16));
}

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* out,
                                                        unsigned long long* stamps) {
  uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[j][e] = rand_bf16(seed);
      b[j][e] = rand_bf16(seed);
    }
  const bool stamp = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (stamp) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  f32x16_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = f32x16_t{};
  for (int i = 0; i < iters; ++i) {
    // four rounds with rotated B operands: every chain sees changing inputs
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + r) & 3], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (stamp) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    stamps[0] = t1 - t0;
    stamps[1] = r1 - r0;
  }
}

__global__ void __launch_bounds__(256) copy_kernel(const u32x4_t* __restrict__ src,
                                                   u32x4_t* __restrict__ dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

// MFMA FLOPs one call performs: workgroups * 4 waves * iters * 16 MFMAs * 32,768.
double dsv4_probe_mfma_flops(int workgroups, int iters) {
  return static_cast<double>(workgroups) * 4.0 * iters * 16.0 * 32768.0;
}

// out: device float [workgroups * 256]; stamps: device uint64 [2] (shader
// clock ticks, 100 MHz ticks of workgroup 0's wave 0).  Returns a hipError_t.
int dsv4_probe_mfma(int workgroups, int iters, float* out, unsigned long long* stamps,
                    void* stream) {
  if (workgroups < 1 || iters < 1 || !out || !stamps) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out, stamps);
  return hipGetLastError();
}

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned).
int dsv4_probe_copy(const void* src, void* dst, size_t bytes, int workgroups, void* stream) {
  if (!src || !dst || (bytes & 15u) || workgroups < 1 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), bytes / 16);
  return hipGetLastError();
}

}  // extern "C"
