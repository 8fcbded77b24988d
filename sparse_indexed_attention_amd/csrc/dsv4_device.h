// Device-side helpers shared by the gfx950 kernels: bf16 storage conversions,
// MFMA operand types, order-preserving float keys and launch wrappers'
// declarations.  Host validation lives in dsv4_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest, ties to even.  NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16x2 (low half = a), round to nearest even, using
// gfx950's v_cvt_pk_bf16_f32 (what a __bf16 conversion lowers to).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// float -> bf16 bits with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Order-preserving unsigned key of a float: a < b  <=>  key(a) < key(b) for
// non-NaN inputs; -0 and +0 map to the same key (adding +0 turns -0 into +0
// and leaves every other non-NaN value unchanged).  Negative floats have all
// bits flipped, non-negative ones only the sign bit; no non-NaN float maps
// to key 0.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  const uint32_t neg = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
  return u ^ (neg | 0x80000000u);
}

// max(x, 0) on the float's bits: one integer max, no NaN canonicalisation.
// Equal to fmaxf(x, 0) for every non-NaN x (-0 gives +0).
__device__ __forceinline__ float relu_bits(float x) {
  const int32_t i = __float_as_int(x);
  return __int_as_float(i > 0 ? i : 0);
}

// Largest score-row stride (floats) the score kernel accepts: two rows of it
// must fit a 32-bit buffer range.
// Most key splits of one query in the narrow-query attention (one wave
// merges their states).
constexpr int kMaxAttnSplits = 64;
// Largest k of a selection (the ABI's DSV4_MAX_TOPK).
constexpr int kMaxTopk = 4096;
constexpr int64_t kMaxScoreStride = (int64_t(1) << 28) - 64;

// Pooled rows visible to a query at absolute position p (ratio 4).
__device__ __forceinline__ int64_t visible_rows(int64_t p) { return (p + 1) >> 2; }
// The same rule for a pool of any ratio r >= 1: floor((p+1)/r); r == 0 means
// no pool (the window-only mode), so nothing is visible.
__device__ __forceinline__ int64_t visible_rows(int64_t p, int ratio) {
  return ratio > 0 ? (p + 1) / ratio : 0;
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane L of the wave writes lds_wave_base + 16*L.
// Issued as inline asm so the compiler neither reorders it nor adds its own
// conservative vmcnt(0) waits for it; callers wait with s_waitcnt vmcnt before
// the barrier that publishes the data.  The LDS address goes in m0 as an
// operand, so the compiler sets m0 itself and knows it is in use.  Issued after the compiler's own loads,
// these can only make the compiler's in-order vmcnt waits stricter.
// The compiler does not insert hazard wait states across an inline-asm
// boundary, so the asm carries its own s_nop 4 (five wait states): an SALU
// write of m0 needs one before a load into LDS reads it, and a VALU write of
// an SGPR (v_readlane / v_readfirstlane making the base or m0) needs five
// before a vector-memory instruction reads that SGPR.
__device__ __forceinline__ void global_to_lds16(const void* g, const void* lds_wave_base) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_wave_base));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Same, addressed as a wave-uniform 64-bit base (SGPR pair) plus a 32-bit
// per-lane byte offset (the saddr form of the instruction).
__device__ __forceinline__ void global_to_lds16_s(const void* sbase, uint32_t voff,
                                                  const void* lds_wave_base) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_wave_base));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// 4 bytes per lane (global_load_lds_dword): lane L of the wave writes
// lds_wave_base + 4*L; lanes masked off by exec write nothing.
__device__ __forceinline__ void global_to_lds4(const void* g, const void* lds_wave_base) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_wave_base));
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Whether `blocks` workgroups of `threads` work-items fit one dispatch along
// x: the dispatch packet counts work-items in 32 bits, so a larger count
// would otherwise be cut short when it becomes a grid size.
inline bool dispatch_fits(int64_t blocks, int64_t threads) {
  return blocks >= 1 && threads >= 1 && blocks <= int64_t(0xFFFFFFFF) / threads;
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with the other counters open,
// and lgkmcnt(0) with the others open.
constexpr int kWaitVm0 = 0x0F70;
__device__ __forceinline__ constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

}  // namespace dsv4

// Records a failure in the library's thread-local error string (read by
// dsv4_last_error) and returns `code`.
int dsv4_internal_fail(int code, const char* fmt, ...);

// Launch wrappers (defined next to their kernels).  All return hipError_t of
// the launch; argument checks happen before they are called.
hipError_t dsv4_launch_compress(void* rows, void* rem, int64_t n_rows, int32_t n_rem,
                                int32_t ratio, int32_t dim, int32_t dtype, const void* x,
                                int64_t n_new, hipStream_t s);
hipError_t dsv4_launch_fill_sequential(int32_t* out, int64_t T, int64_t q_pos0, int64_t S,
                                       int32_t topk, hipStream_t s);
hipError_t dsv4_launch_indexer_scores(const void* q, const float* w, const void* keys,
                                      int64_t rows, int64_t q_pos0, int64_t S, int32_t n_heads,
                                      int32_t dim, int32_t fold_mask, float* out,
                                      int64_t out_stride, hipStream_t s);
hipError_t dsv4_launch_topk(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                            int32_t topk, int32_t* out_idx, hipStream_t s);
// Top-k of long rows (2 to 8 chunks of 32,768 columns, k a multiple of 4,
// every row showing at least k columns, row starts 16-byte aligned) that
// reuses the score rows as its workspace: each chunk's candidates overwrite
// the chunk's first 2 k floats.  The scores are not preserved.
bool dsv4_topk_inplace_applies(const float* scores, int64_t rows, int64_t stride,
                               int64_t q_pos0, int32_t topk);
hipError_t dsv4_launch_topk_inplace(float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                                    int32_t topk, int32_t* out_idx, hipStream_t s);
// Chunk-parallel top-k of a few long rows (two passes; see topk.hip): the
// number of 32,768-column chunks of the longest row, and the launch, which
// needs cand_idx / cand_score of rows * chunks * topk entries each.
int64_t dsv4_topk_split_chunks(int64_t rows, int64_t q_pos0);
hipError_t dsv4_launch_topk_split(const float* scores, int64_t rows, int64_t stride,
                                  int64_t q_pos0, int32_t topk, int32_t* out_idx,
                                  int32_t* cand_idx, float* cand_score, hipStream_t s);
hipError_t dsv4_launch_sparse_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                                   int32_t head_dim, float scale, const void* raw_kv,
                                   int64_t raw_pos0, int32_t window, const void* pooled,
                                   int32_t ratio, const int32_t* sel_idx, int32_t topk,
                                   void* out, int32_t nsplit, float* part_o, float* part_ml,
                                   hipStream_t s);
// The H = 64, D = 512 kernel (attn_h64.hip); scale_log2 = scale * log2(e).
// It takes selections of at most 5,160 slots (its LDS holds the row).
bool dsv4_attn_h64_fits(int32_t topk);
hipError_t dsv4_launch_sparse_attn_h64(const void* q, int64_t T, int64_t q_pos0, float scale_log2,
                                       const void* raw_kv, int64_t raw_pos0, int32_t window,
                                       const void* pooled, int32_t ratio, const int32_t* sel_idx,
                                       int32_t topk, void* out, int32_t nsplit, float* part_o,
                                       float* part_ml, hipStream_t s);
hipError_t dsv4_launch_attn_combine(const float* part_o, const float* part_ml, int64_t T,
                                    int32_t nsplit, int32_t n_heads, int32_t head_dim, void* out,
                                    hipStream_t s);
