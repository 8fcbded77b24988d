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
//     rows.  Each wave owns two queries; their q blocks (heads x dim, bf16)
//     stay in VGPRs for the whole sweep over the workgroup's column range, so
//     every key fragment read from LDS feeds both queries' MFMAs.
//   * Pooled index keys are gathered 64 rows at a time straight into LDS with
//     global_load_lds_dwordx4 (no VGPRs hold data in flight), three LDS stages
//     deep with one barrier per tile; 16-byte chunk c of row r sits at slot
//     c ^ (r & 15), so the B-operand reads (32 rows, one chunk) are free of
//     bank conflicts.
//   * The contraction index is permuted identically in A and B: lane half kb
//     holds dims [kb*D/2, kb*D/2 + D/2), so every lane reads one contiguous
//     run of D bytes from its q rows.
//   * Epilogue in the accumulator layout: each lane holds 16 head rows of one
//     column per M tile; ReLU and the weight are one max + one fma per
//     element (weights read from LDS), the lane sums its rows, and one
//     v_permlane32_swap both finishes the head sum and leaves query 0's
//     column in lanes 0-31 and query 1's in lanes 32-63 for a single store.
//     The mask compares the column with the query's visible count; column
//     blocks no query of the wave can see are written as -inf without MFMA
//     work.
//   * Four-wave workgroups, two per CU: their barriers are independent, so one
//     workgroup's epilogue VALU work overlaps the other's MFMAs.
//   * Grid: workgroups are dealt round-robin to the 8 XCDs; a workgroup's
//     column split is chosen from blockIdx % 8 so each XCD sweeps one eighth
//     of the key rows, which then stays resident in that XCD's L2.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 2;                 // queries per wave
constexpr int kQB = kWaves * kQW;      // queries per workgroup
constexpr int kTileCols = 64;          // key rows per LDS tile
constexpr int kStages = 3;

template <int KSTEPS, int MT>
__global__ void __launch_bounds__(kThreads, 2)
indexer_score_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                     const uint16_t* __restrict__ keys, int64_t rows, int64_t q_pos0, int64_t S,
                     int n_heads, int fold_mask, float* __restrict__ out, int64_t out_stride,
                     int splits_per_xcd, int64_t cols_per_split) {
  constexpr int D = KSTEPS * 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
  constexpr int RPI = 64 / CPR;              // key rows per DMA instruction
  constexpr int INSTS = kTileCols / RPI;     // DMA instructions per tile
  constexpr int PER_WAVE = INSTS / kWaves;   // ... per wave
  static_assert(INSTS % kWaves == 0 && PER_WAVE >= 1 && PER_WAVE <= 15, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kStages][kTileCols * D];
  __shared__ __attribute__((aligned(16))) float w_lds[kQB][64];

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

  const int64_t t0 = qb * kQB + wave * kQW;  // this wave's queries t0, t0+1
  int64_t vis[kQW];
  bool tval[kQW];
#pragma unroll
  for (int qi = 0; qi < kQW; ++qi) {
    tval[qi] = t0 + qi < rows;
    int64_t v = S;
    if (fold_mask) {
      v = tval[qi] ? visible_rows(q_pos0 + t0 + qi) : 0;
      if (v > S) v = S;
    }
    vis[qi] = tval[qi] ? v : 0;
  }
  const int64_t vis_wave = vis[0] > vis[1] ? vis[0] : vis[1];
  int64_t t_last = qb * kQB + (kQB - 1);
  if (t_last > rows - 1) t_last = rows - 1;
  int64_t vis_max = S;
  if (fold_mask) {
    vis_max = visible_rows(q_pos0 + t_last);
    if (vis_max > S) vis_max = S;
  }
  int64_t compute_end = col_end < vis_max ? col_end : vis_max;
  if (compute_end < col_begin) compute_end = col_begin;

  // ---- head weights of the workgroup's queries -> LDS (0 for missing heads)
  for (int i = tid; i < kQB * 64; i += kThreads) {
    const int ql = i >> 6, h = i & 63;
    const int64_t tq = qb * kQB + ql;
    w_lds[ql][h] = (tq < rows && h < n_heads) ? w[tq * n_heads + h] : 0.f;
  }

  // ---- the wave's q blocks, held in registers for the whole sweep
  bf16x8_t afrag[kQW][MT][KSTEPS];
#pragma unroll
  for (int qi = 0; qi < kQW; ++qi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int head = mt * 32 + ln;
      const bool hv = tval[qi] && head < n_heads;
      const uint16_t* qp = q + (((t0 + qi) * n_heads + head) * (int64_t)D + kb * (D / 2));
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        afrag[qi][mt][j] = hv ? *reinterpret_cast<const bf16x8_t*>(qp + j * 8) : bf16x8_t{};
    }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only tile DMAs in flight from here

  const int64_t n_tiles = (compute_end - col_begin + kTileCols - 1) / kTileCols;
  auto issue_tile = [&](int64_t it, int buf) {
    const int64_t c0 = col_begin + it * kTileCols;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int inst = wave * PER_WAVE + k;
      const int row = inst * RPI + lane / CPR;
      const int slot = lane % CPR;
      int64_t col = c0 + row;
      if (col >= compute_end) col = col_begin;  // any valid row; never stored
      global_to_lds16(keys + col * D + (slot ^ (row & SWZ)) * 8, &ktile[buf][inst * RPI * D]);
    }
  };

  if (n_tiles > 0) issue_tile(0, 0);
  if (n_tiles > 1) issue_tile(1, 1);

  float* orow = out + (t0 + kb) * out_stride;
  const bool lane_tval = kb == 0 ? tval[0] : tval[1];
  const int64_t lane_vis = kb == 0 ? vis[0] : vis[1];

  for (int64_t it = 0; it < n_tiles; ++it) {
    const int buf = static_cast<int>(it % kStages);
    if (it + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0F70 | PER_WAVE);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();  // publishes tile `it`, retires tile it-1 (its stage takes it+2)
    if (it + 2 < n_tiles) issue_tile(it + 2, static_cast<int>((it + 2) % kStages));
    const int64_t c0 = col_begin + it * kTileCols;
    const uint16_t* tb = ktile[buf];
#pragma unroll
    for (int sub = 0; sub < kTileCols / 32; ++sub) {
      const int64_t s0 = c0 + sub * 32;
      if (s0 >= col_end) break;
      const int64_t col = s0 + ln;
      if (s0 >= vis_wave) {  // neither query of the wave sees this block
        if (lane_tval && col < col_end) orow[col] = -INFINITY;
        continue;
      }
      const int row = sub * 32 + ln;
      bf16x8_t bfrag[KSTEPS];
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        const int chunk = kb * KSTEPS + j;
        bfrag[j] = *reinterpret_cast<const bf16x8_t*>(tb + row * D + ((chunk ^ (row & SWZ)) * 8));
      }
      float part[kQW];
#pragma unroll
      for (int qi = 0; qi < kQW; ++qi) {
        part[qi] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x16_t acc = {};
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[qi][mt][j], bfrag[j], acc, 0, 0, 0);
          // accumulator element i holds head mt*32 + 8*(i/4) + 4*kb + i%4
          const float* wp = &w_lds[wave * kQW + qi][mt * 32 + 4 * kb];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(wp + 8 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              part[qi] = fmaf(wv[i], fmaxf(acc[4 * g4 + i], 0.f), part[qi]);
          }
        }
      }
      // lanes 0-31 <- query 0 (both halves summed), lanes 32-63 <- query 1
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                       __float_as_uint(part[1]), false, false);
      const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (lane_tval && col < col_end) orow[col] = (col < lane_vis) ? tot : -INFINITY;
    }
  }

  // ---- columns no query of this workgroup can see: sentinel only
#pragma unroll
  for (int qi = 0; qi < kQW; ++qi) {
    if (!tval[qi]) continue;
    float* orq = out + (t0 + qi) * out_stride;
    for (int64_t col = compute_end + lane; col < col_end; col += 64) orq[col] = -INFINITY;
  }
}

template <int KSTEPS, int MT>
hipError_t launch_t(const void* q, const float* w, const void* keys, int64_t rows,
                    int64_t q_pos0, int64_t S, int n_heads, int fold_mask, float* out,
                    int64_t out_stride, hipStream_t s) {
  const int64_t nqb = (rows + kQB - 1) / kQB;
  // Column splits: a multiple of 8 (one group per XCD), enough workgroups to
  // fill 256 CUs several times, and at least one tile per split.
  int64_t per_xcd = (4096 + 8 * nqb - 1) / (8 * nqb);
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
