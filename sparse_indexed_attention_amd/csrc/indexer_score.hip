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
//     bank conflicts.  The tile loop is unrolled over the three stages so each
//     B-fragment address is a per-lane offset plus an immediate.
//   * The contraction index is permuted identically in A and B: lane half kb
//     holds dims [kb*D/2, kb*D/2 + D/2), so every lane reads one contiguous
//     run of D bytes from its q rows.
//   * Epilogue in the accumulator layout: each lane holds 16 head rows of one
//     column per M tile; ReLU is one integer max on the float bits and the
//     weight one fma per element, with the weight broadcast across the
//     16-lane row by DPP from a single register per chain (no LDS traffic
//     for weights).  The lane sums its rows, and one v_permlane32_swap both
//     finishes the head sum and leaves query 0's column in lanes 0-31 and
//     query 1's in lanes 32-63 for a single store.  The mask compares the
//     column with the query's visible count.
//   * Software pipeline: a 32-column block runs 2*MT accumulation chains of
//     KSTEPS MFMAs; the epilogue of each chain is issued under the next
//     chain's MFMAs (after the first two of them, which cover the wait for
//     its accumulator), and the last chain's epilogue plus the block's store
//     move into the next block (across the tile barrier), so the matrix pipe
//     has independent work beside every epilogue.  The block body has no branches:
//     stores go through a buffer resource whose range check drops lanes whose
//     column or query is out of range.
//   * Four-wave workgroups, two per CU: their barriers are independent, so one
//     workgroup's epilogue VALU work overlaps the other's MFMAs.
//   * Grid: workgroups are dealt round-robin to the 8 XCDs, and blockIdx % 8
//     picks the XCD's share, one of query groups x column groups = 8.  XCD x
//     takes query group x / cgroups (every qgroups-th query block) and column
//     group x % cgroups (that fraction of the key rows, which stays in the
//     XCD's 4 MiB L2 while the XCD works through it), so each query block's
//     q is fetched by cgroups XCDs and each key row by qgroups.  The launch
//     picks cgroups to balance those two fetches.  Score rows are written
//     non-temporal so the stream of output does not evict the keys from L2.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 2;                 // queries per wave
constexpr int kQB = kWaves * kQW;      // queries per workgroup
constexpr int kTileCols = 64;          // key rows per LDS tile
constexpr int kStages = 3;
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond any buffer range used here

// part += w[row base + I] * x, where the weight comes from lane I of the
// lane's 16-lane row (DPP row_newbcast on the fma's first operand).  The
// weight register is written once before the column loop, so the DPP
// source never follows a VALU write of it.
template <int I>
__device__ __forceinline__ void fmac_row_bcast(float& part, float w, float x) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(part)
      : "v"(w), "v"(x), "n"(I));
}

// part += sum_i w_i * max(0, acc[i]) over the 16 accumulator elements.
template <int... I>
__device__ __forceinline__ void weighted_relu_sum(const f32x16_t& acc, float w, float& part,
                                                  std::integer_sequence<int, I...>) {
  (fmac_row_bcast<I>(part, w, relu_bits(acc[I])), ...);
}

template <int KSTEPS, int MT>
__global__ void __launch_bounds__(kThreads, 2)
indexer_score_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                     const uint16_t* __restrict__ keys, int64_t rows, int64_t q_pos0, int64_t S,
                     int n_heads, int fold_mask, float* __restrict__ out, int64_t out_stride,
                     int cgroups, int splits_per_cg, int64_t cols_per_split) {
  constexpr int D = KSTEPS * 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
  constexpr int RPI = 64 / CPR;              // key rows per DMA instruction
  constexpr int INSTS = kTileCols / RPI;     // DMA instructions per tile
  constexpr int PER_WAVE = INSTS / kWaves;   // ... per wave
  constexpr int NCH = kQW * MT;              // accumulation chains per 32-column block
  static_assert(INSTS % kWaves == 0 && PER_WAVE >= 1 && PER_WAVE <= 15, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kStages][kTileCols * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: SGPR addressing
  const int kb = lane >> 5;
  const int ln = lane & 31;

  const int g = blockIdx.x;
  const int xcd = g & 7;
  const int r = g >> 3;
  const int qgroups = 8 / cgroups;
  const int cs = (xcd % cgroups) * splits_per_cg + (r % splits_per_cg);
  const int64_t qb = xcd / cgroups + static_cast<int64_t>(qgroups) * (r / splits_per_cg);
  if (qb * kQB >= rows) return;  // whole workgroup: no barrier reached yet
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
  int64_t t_last = qb * kQB + (kQB - 1);
  if (t_last > rows - 1) t_last = rows - 1;
  int64_t vis_max = S;
  if (fold_mask) {
    vis_max = visible_rows(q_pos0 + t_last);
    if (vis_max > S) vis_max = S;
  }
  int64_t compute_end = col_end < vis_max ? col_end : vis_max;
  if (compute_end < col_begin) compute_end = col_begin;

  // ---- head weights, one register per chain: lane L holds the weight of
  // accumulator element L % 16 for its lane half (head mt*32 + 8*((L%16)/4)
  // + 4*(L/32) + L%4), broadcast to the 16-lane row by the epilogue's DPP.
  float wreg[kQW][MT];
#pragma unroll
  for (int qi = 0; qi < kQW; ++qi)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 32 + 8 * ((lane & 15) >> 2) + 4 * kb + (lane & 3);
      wreg[qi][mt] = (tval[qi] && h < n_heads) ? w[(t0 + qi) * n_heads + h] : 0.f;
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
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // only tile DMAs in flight from here

  const int64_t n_tiles = (compute_end - col_begin + kTileCols - 1) / kTileCols;
  // DMA lane offsets: instruction k of this wave moves rows dma_row(k) ..,
  // this lane one 16-byte chunk of row dma_row(k) (swizzled slot).
  uint32_t dma_off[PER_WAVE];
#pragma unroll
  for (int k = 0; k < PER_WAVE; ++k) {
    const int row = (wave * PER_WAVE + k) * RPI + lane / CPR;
    dma_off[k] = static_cast<uint32_t>((row * D + ((lane % CPR) ^ (row & SWZ)) * 8) * 2);
  }
  auto issue_tile = [&](int64_t it, int buf) {
    const int64_t c0 = col_begin + it * kTileCols;
    const uint16_t* tbase = keys + c0 * D;
    const int64_t n_ok = compute_end - c0;  // rows of this tile that exist (>= 1)
    if (n_ok >= kTileCols) {
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k)
        global_to_lds16_s(tbase, dma_off[k], &ktile[buf][(wave * PER_WAVE + k) * RPI * D]);
    } else {
      // last tile of the range: rows past the end re-read row 0 of the tile
      // (valid memory; their scores are never kept)
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k) {
        const int row = (wave * PER_WAVE + k) * RPI + lane / CPR;
        const uint32_t off = row < n_ok ? dma_off[k] : dma_off[k] - row * D * 2;
        global_to_lds16_s(tbase, off, &ktile[buf][(wave * PER_WAVE + k) * RPI * D]);
      }
    }
  };

  if (n_tiles > 0) issue_tile(0, 0);
  if (n_tiles > 1) issue_tile(1, 1);

  // Output: the wave's valid query rows from column col_begin on, as one
  // buffer range; lane half kb stores query t0+kb.  Offsets past the range
  // (invalid query, column >= col_end) are dropped by the range check.
  // Columns are handled relative to col_begin in 32 bits.
  const int n_valid_q = tval[1] ? 2 : (tval[0] ? 1 : 0);
  float* obase = out + (n_valid_q > 0 ? t0 * out_stride + col_begin : 0);
  const int64_t n_bytes = n_valid_q > 0 ? (n_valid_q * out_stride - col_begin) * 4 : 0;
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(obase, 0, static_cast<int>(n_bytes), 0x00020000);
  const int32_t rel_end = static_cast<int32_t>(col_end - col_begin);
  int64_t lv = (kb == 0 ? vis[0] : vis[1]) - col_begin;
  if (lv < 0) lv = 0;
  if (lv > rel_end) lv = rel_end;
  const int32_t lane_vis = static_cast<int32_t>(lv);
  const uint32_t lane_row_off = static_cast<uint32_t>(kb * out_stride * 4);

  // Byte offset of B fragment j inside a tile for this lane (row ln of the
  // first 32-row block; chunk kb*KSTEPS + j sits at slot chunk ^ (ln & SWZ)).
  uint32_t boff[KSTEPS];
#pragma unroll
  for (int j = 0; j < KSTEPS; ++j)
    boff[j] = static_cast<uint32_t>((ln * D + (((kb * KSTEPS + j) ^ (ln & SWZ)) * 8)) * 2);

  // ---- pipeline state carried from one 32-column block to the next
  f32x16_t acc_c = {};              // last chain of the previous block
  float part_c[kQW] = {0.f, 0.f};   // the previous block's per-query partial sums
  int32_t col_c = rel_end;          // the previous block's column (rel_end: nothing to store)

  // ReLU + weight of one chain's accumulator, added into `part`.
  auto epilogue = [&](const f32x16_t& acc, int chain, float& part) {
    weighted_relu_sum(acc, wreg[chain / MT][chain % MT], part,
                      std::make_integer_sequence<int, 16>{});
    // Empty volatile asm on the result: instruction selection keeps the
    // epilogue inside this chain's scheduling region instead of sinking it
    // towards its use at the end of the block.
    asm volatile("" : "+v"(part));
  };
  // Head sum across the lane halves, mask, store of one finished block.
  auto store_block = [&](float p0, float p1, int32_t col) {
    // lanes 0-31 <- query 0 (both halves summed), lanes 32-63 <- query 1
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1),
                                                     false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float v = col < lane_vis ? tot : -INFINITY;
    const uint32_t off =
        col < rel_end ? lane_row_off + static_cast<uint32_t>(col) * 4u : kDropOffset;
    // non-temporal (cache policy nt): the output streams past L2
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), orsrc, static_cast<int>(off), 0, 2);
  };

  // One 32-column block at LDS byte address tb (first row of the block).
  auto block = [&](const char* tb, int32_t s0) {
    bf16x8_t bfrag[KSTEPS];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) bfrag[j] = *reinterpret_cast<const bf16x8_t*>(tb + boff[j]);
    float part[kQW] = {0.f, 0.f};
    f32x16_t prev = acc_c;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int qi = c / MT, mt = c % MT;
      f32x16_t acc = {};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[qi][mt][j], bfrag[j], acc, 0, 0, 0);
      if (c == 0) {
        // finish the previous block under this chain's MFMAs
        epilogue(prev, NCH - 1, part_c[kQW - 1]);
        store_block(part_c[0], part_c[1], col_c);
      } else {
        epilogue(prev, c - 1, part[(c - 1) / MT]);
      }
      prev = acc;
      if (c >= 1) {
        // Issue order of this region (masks: 0x008 MFMA, 0x002 VALU): two of
        // this chain's MFMAs first, while the previous chain's accumulator
        // settles, then its epilogue spread five VALU to an MFMA over the
        // other six.  Left to itself the scheduler opens the region with the
        // epilogue, whose first reads wait on that accumulator with the
        // matrix pipe idle.
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
        for (int g = 0; g < KSTEPS - 2; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
      }
      // one chain's MFMAs beside one epilogue: keeps two accumulators live
      __builtin_amdgcn_sched_barrier(0);
    }
    acc_c = prev;
    part_c[0] = part[0];
    part_c[1] = part[1];
    col_c = s0 + ln;
  };

  // Wait for tile `it`'s DMA.  vmcnt also counts stores, and retires in
  // issue order, so the wait names the number of vector memory ops issued
  // after that DMA: the next tile's DMA (if any) plus one store per 32-column
  // block of each of the (up to two) tile steps since.  Extra ops in between
  // only make the wait stricter.
  auto wait_tile = [&](int64_t it) {
    constexpr int kStoresPerTile = kTileCols / 32;
    const bool next = it + 1 < n_tiles;
    if (it == 0) {
      if (next) __builtin_amdgcn_s_waitcnt(wait_vmcnt(PER_WAVE));
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    } else if (it == 1) {
      if (next) __builtin_amdgcn_s_waitcnt(wait_vmcnt(PER_WAVE + kStoresPerTile));
      else __builtin_amdgcn_s_waitcnt(wait_vmcnt(kStoresPerTile));
    } else {
      if (next) __builtin_amdgcn_s_waitcnt(wait_vmcnt(PER_WAVE + 2 * kStoresPerTile));
      else __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kStoresPerTile));
    }
  };

  // One tile; the stage is a compile-time constant.
  auto tile_step = [&](int64_t it, auto stage_c) {
    constexpr int buf = decltype(stage_c)::value;
    wait_tile(it);
    __syncthreads();  // publishes tile `it`, retires tile it-1 (its stage takes it+2)
    if (it + 2 < n_tiles) issue_tile(it + 2, (buf + 2) % kStages);
    const int32_t c0 = static_cast<int32_t>(it * kTileCols);  // relative to col_begin
    const char* tb = reinterpret_cast<const char*>(ktile[buf]);
#pragma unroll
    for (int sub = 0; sub < kTileCols / 32; ++sub) block(tb + sub * 32 * D * 2, c0 + sub * 32);
  };
  for (int64_t it = 0; it < n_tiles; it += kStages) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_tiles) tile_step(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 < n_tiles) tile_step(it + 2, std::integral_constant<int, 2>{});
  }
  // drain: the last block's final chain
  epilogue(acc_c, NCH - 1, part_c[kQW - 1]);
  store_block(part_c[0], part_c[1], col_c);

  // ---- columns past the computed tiles (none of the workgroup's queries
  // sees them): sentinel only
  const int64_t tail = col_begin + n_tiles * kTileCols;
#pragma unroll
  for (int qi = 0; qi < kQW; ++qi) {
    if (!tval[qi]) continue;
    float* orq = out + (t0 + qi) * out_stride;
    for (int64_t col = tail + lane; col < col_end; col += 64) orq[col] = -INFINITY;
  }
}

template <int KSTEPS, int MT>
hipError_t launch_t(const void* q, const float* w, const void* keys, int64_t rows,
                    int64_t q_pos0, int64_t S, int n_heads, int fold_mask, float* out,
                    int64_t out_stride, hipStream_t s) {
  const int64_t nqb = (rows + kQB - 1) / kQB;
  const int64_t tiles = (S + kTileCols - 1) / kTileCols;
  // Column splits over the whole key range: as few as fill one round of two
  // workgroups per CU (512), and at most 256 tiles (16,384 key rows) each.
  // Every workgroup stages its 8 queries (128 KiB at 64 heads x 128) before
  // its first tile, so longer splits amortise that; a second round would
  // load new queries into the L2 that holds the keys and fetch the keys
  // again (at 128K, 2,048 rows: 106 MB per launch in one round, 154 MB in 8,
  // same time).  Past 256 tiles per split, rounds even out the CUs instead
  // (at 1M context one round of 512 takes 4% longer than 4,096 workgroups).
  int64_t sp = std::max<int64_t>((512 + nqb - 1) / nqb, (tiles + 255) / 256);
  sp = std::min<int64_t>(sp, tiles);
  if (sp < 1) sp = 1;
  // XCD shares: query groups x column groups = 8 (see the kernel comment).
  // An XCD reads S / cgroups key rows and nqb * cgroups / 8 query blocks, so
  // key bytes + query bytes is least near cgroups^2 = S / (nqb * n_heads);
  // take the power of two nearest that, at most 8 and at most sp.
  int cgroups = 8;
  while (cgroups > 1 &&
         (cgroups > sp || static_cast<int64_t>(cgroups) * cgroups * nqb * n_heads > 2 * S))
    cgroups >>= 1;
  const int64_t qgroups = 8 / cgroups;
  const int64_t nqb_g = (nqb + qgroups - 1) / qgroups;  // query blocks per query group
  int64_t per_cg = (sp + cgroups - 1) / cgroups;
  int64_t max_per_cg = S / (static_cast<int64_t>(cgroups) * kTileCols);
  if (max_per_cg < 1) max_per_cg = 1;
  if (per_cg > max_per_cg) per_cg = max_per_cg;
  const int64_t splits = cgroups * per_cg;
  int64_t cps = (S + splits - 1) / splits;
  cps = (cps + kTileCols - 1) / kTileCols * kTileCols;
  const int64_t grid = 8 * per_cg * nqb_g;
  if (!dispatch_fits(grid, kThreads)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((indexer_score_kernel<KSTEPS, MT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(q), w,
                     static_cast<const uint16_t*>(keys), rows, q_pos0, S, n_heads, fold_mask,
                     out, out_stride, cgroups, static_cast<int>(per_cg), cps);
  return hipGetLastError();
}

}  // namespace

hipError_t dsv4_launch_indexer_scores(const void* q, const float* w, const void* keys,
                                      int64_t rows, int64_t q_pos0, int64_t S, int32_t n_heads,
                                      int32_t dim, int32_t fold_mask, float* out,
                                      int64_t out_stride, hipStream_t s) {
  // The epilogue addresses two output rows through one 32-bit buffer range.
  if (out_stride > kMaxScoreStride) return hipErrorInvalidValue;
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
