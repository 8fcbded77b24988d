// Indexer score with the pooled-ratio causal mask folded into the epilogue,
// bf16 MFMA on gfx950.
//
//   score[t][s] = sum_h w[t][h] * max(0, q[t][h][:] . key[s][:])      s <  vis(t)
//               = -inf                                                  s >= vis(t)
//
// [P2 "perf(deepseek_v4): faster exact DeepSeek-V4 prefill", Performance:
// the DSA indexer scores every visible pooled row, FLOP-bound; commit 5: the
// pooled-ratio causal mask folded into the score kernel epilogue with the
// same sentinel as a second-pass mask.]
//
// Mapping onto CDNA4.  This is a dense contraction (per query: a 64x128 by
// 128xS product), so it runs on v_mfma_f32_32x32x16_bf16:
//   * M = indexer heads (one or two 32-row tiles), K = index dim, N = pooled
//     rows.  Each wave owns one query; its q block (heads x dim, bf16) stays
//     in VGPRs for the whole sweep over its column range, as do its head
//     weights.
//   * Pooled index keys are staged through LDS in 64-row tiles shared by the
//     8 waves (8 queries) of a workgroup; each key byte fetched from L2 feeds
//     8 queries' MFMAs.  Rows are padded by 16 bytes so the 16-byte B-operand
//     reads of 16 consecutive rows fall in distinct banks.
//   * The contraction index is permuted identically in A and B: lane half kb
//     holds dims [kb*D/2, kb*D/2 + D/2), so every lane reads one contiguous
//     run of D bytes from its q row and its key row.
//   * Epilogue in the accumulator layout: each lane holds 16 head rows of one
//     column per M tile; ReLU and the weight are one max + one fma per
//     element, the lane sums its rows, and one v_permlane32_swap adds the
//     other lane half.  The mask compares the column with the query's visible
//     count; fully masked column tiles are written as -inf without MFMA work.
//   * Grid: the workgroups are dealt round-robin to the 8 XCDs; a workgroup's
//     column split is chosen from blockIdx % 8 so each XCD sweeps one eighth
//     of the key rows, which then stays resident in that XCD's L2.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kWaves = 8;     // queries per workgroup (one per wave)
constexpr int kThreads = kWaves * 64;
constexpr int kTileCols = 64; // key rows per LDS tile

template <int KSTEPS, int MT>
__global__ void __launch_bounds__(kThreads)
indexer_score_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                     const uint16_t* __restrict__ keys, int64_t rows, int64_t q_pos0, int64_t S,
                     int n_heads, int fold_mask, float* __restrict__ out, int64_t out_stride,
                     int splits_per_xcd, int64_t cols_per_split) {
  constexpr int D = KSTEPS * 16;
  constexpr int PITCH = D + 8;               // uint16 per LDS row (16 B pad)
  constexpr int CHUNKS = kTileCols * D / 8;  // 16-byte chunks per tile
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kTileCols * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = lane >> 5;
  const int ln = lane & 31;

  const int g = blockIdx.x;
  const int xcd = g & 7;
  const int r = g >> 3;
  const int cs = xcd * splits_per_xcd + (r % splits_per_xcd);
  const int64_t qb = r / splits_per_xcd;
  const int64_t col_begin = (int64_t)cs * cols_per_split;
  int64_t col_end = col_begin + cols_per_split;
  if (col_end > S) col_end = S;
  if (col_begin >= col_end) return;  // whole workgroup: no barrier reached yet

  const int64_t t = qb * kWaves + wave;
  const bool tvalid = t < rows;
  int64_t t_last = qb * kWaves + (kWaves - 1);
  if (t_last > rows - 1) t_last = rows - 1;
  int64_t vis_t = S, vis_max = S;
  if (fold_mask) {
    vis_t = tvalid ? visible_rows(q_pos0 + t) : 0;
    if (vis_t > S) vis_t = S;
    vis_max = visible_rows(q_pos0 + t_last);
    if (vis_max > S) vis_max = S;
  }
  int64_t compute_end = col_end < vis_max ? col_end : vis_max;
  if (compute_end < col_begin) compute_end = col_begin;

  // ---- per-wave operands held in registers for the whole sweep
  bf16x8_t afrag[MT][KSTEPS];
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = mt * 32 + ln;
    const bool hv = tvalid && head < n_heads;
    const uint16_t* qp = q + ((t * n_heads + head) * (int64_t)D + kb * (D / 2));
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      if (hv) {
        afrag[mt][j] = *reinterpret_cast<const bf16x8_t*>(qp + j * 8);
      } else {
        afrag[mt][j] = bf16x8_t{};
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = mt * 32 + 8 * (i >> 2) + 4 * kb + (i & 3);
      wv[mt][i] = (tvalid && hh < n_heads) ? w[t * n_heads + hh] : 0.f;
    }
  }

  // ---- sweep column tiles that some query of this workgroup can see
  const int64_t n_tiles = (compute_end - col_begin + kTileCols - 1) / kTileCols;
  constexpr int PER_THREAD = (CHUNKS + kThreads - 1) / kThreads;
  u32x4_t pre[PER_THREAD];

  auto load_tile = [&](int64_t c0) {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int ci = tid + k * kThreads;
      pre[k] = u32x4_t{0u, 0u, 0u, 0u};
      if (ci < CHUNKS) {
        const int rr = ci / (D / 8);
        const int c8 = ci - rr * (D / 8);
        const int64_t col = c0 + rr;
        if (col < compute_end)
          pre[k] = *reinterpret_cast<const u32x4_t*>(keys + col * D + c8 * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int ci = tid + k * kThreads;
      if (ci < CHUNKS) {
        const int rr = ci / (D / 8);
        const int c8 = ci - rr * (D / 8);
        *reinterpret_cast<u32x4_t*>(&ktile[rr * PITCH + c8 * 8]) = pre[k];
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(col_begin);
    store_tile();
  }
  __syncthreads();

  float* orow = out + t * out_stride;
  for (int64_t it = 0; it < n_tiles; ++it) {
    const int64_t c0 = col_begin + it * kTileCols;
    if (it + 1 < n_tiles) load_tile(c0 + kTileCols);  // in flight during MFMA work

    if (tvalid) {
#pragma unroll
      for (int sub = 0; sub < kTileCols / 32; ++sub) {
        const int64_t s0 = c0 + sub * 32;
        const int64_t col = s0 + ln;
        if (s0 >= col_end) break;
        if (s0 >= vis_t) {  // whole 32-column block masked for this query
          if (kb == 0 && col < col_end) orow[col] = -INFINITY;
          continue;
        }
        bf16x8_t bfrag[KSTEPS];
        const uint16_t* kp = &ktile[(sub * 32 + ln) * PITCH + kb * (D / 2)];
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) bfrag[j] = *reinterpret_cast<const bf16x8_t*>(kp + j * 8);
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x16_t acc = {};
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mt][j], bfrag[j], acc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) part = fmaf(wv[mt][i], fmaxf(acc[i], 0.f), part);
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                         __float_as_uint(part), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (kb == 0 && col < col_end) orow[col] = (col < vis_t) ? tot : -INFINITY;
      }
    }
    __syncthreads();
    if (it + 1 < n_tiles) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- columns no query of this workgroup can see: sentinel only
  if (tvalid) {
    for (int64_t col = compute_end + lane; col < col_end; col += 64) orow[col] = -INFINITY;
  }
}

template <int KSTEPS, int MT>
hipError_t launch_t(const void* q, const float* w, const void* keys, int64_t rows,
                    int64_t q_pos0, int64_t S, int n_heads, int fold_mask, float* out,
                    int64_t out_stride, hipStream_t s) {
  const int64_t nqb = (rows + kWaves - 1) / kWaves;
  // Column splits: a multiple of 8 (one group per XCD), enough workgroups to
  // fill 256 CUs several times, and at least one 64-column tile per split.
  int64_t per_xcd = (2048 + 8 * nqb - 1) / (8 * nqb);
  int64_t max_per_xcd = S / (8 * kTileCols);
  if (max_per_xcd < 1) max_per_xcd = 1;
  if (per_xcd > max_per_xcd) per_xcd = max_per_xcd;
  if (per_xcd < 1) per_xcd = 1;
  const int64_t splits = 8 * per_xcd;
  int64_t cps = (S + splits - 1) / splits;
  cps = (cps + kTileCols - 1) / kTileCols * kTileCols;
  const int64_t grid = splits * nqb;
  hipLaunchKernelGGL((indexer_score_kernel<KSTEPS, MT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(q), w,
                     static_cast<const uint16_t*>(keys), rows, q_pos0, S, n_heads, fold_mask,
                     out, out_stride, static_cast<int>(per_xcd), cps);
  return hipGetLastError();
}

}  // namespace

hipError_t dsv4_launch_indexer_scores(const void* q, const float* w, const void* keys,
                                      int64_t rows, int64_t q_pos0, int64_t S, int32_t n_heads,
                                      int32_t dim, int32_t fold_mask, float* out,
                                      int64_t out_stride, hipStream_t s) {
  const bool two = n_heads > 32;
  switch (dim) {
    case 32:
      return two ? launch_t<2, 2>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s)
                 : launch_t<2, 1>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s);
    case 64:
      return two ? launch_t<4, 2>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s)
                 : launch_t<4, 1>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s);
    case 128:
      return two ? launch_t<8, 2>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s)
                 : launch_t<8, 1>(q, w, keys, rows, q_pos0, S, n_heads, fold_mask, out, out_stride, s);
    default:
      return hipErrorInvalidValue;
  }
}
