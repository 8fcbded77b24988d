// Exact per-row top-k over the visible prefix of a score row.
//
// [P1 "perf(deepseek-v4): skip redundant all-pooled indexer scoring", Summary:
// top-k selection of index_topk pooled rows; P3 "[Discussion] Tile
// indexed-attention scoring independently of the global prefill chunk",
// Possible design step 3: top-k of a score tile into the compact selection.]
// Selection rule (readings): the min(k, visible) largest scores, equal scores
// to the lower column (-0 == +0), chosen columns written in ascending order,
// then -1.
//
// HBM-bound: every visible score is read once.  Two kernels:
//   * topk_reg_kernel (below, after topk_kernel) keeps a row's keys in
//     registers: rows of up to 32,768 columns whose starts are 16-byte
//     aligned, and, in two passes, longer rows;
//   * topk_kernel stages rows through LDS: longer rows when there is no
//     workspace for two passes, and any stride.
// topk_kernel's design:
//   * Persistent workgroups (one per CU, 16 waves) walk a list of work items,
//     an item being a row or, for rows longer than one chunk, a chunk of a
//     row.  The next item is copied from HBM into an LDS row buffer with
//     global_load_lds_dwordx4 while the current item is processed, so HBM
//     reads overlap all the compute below.  Thread t holds columns
//     [PER*t, PER*t + PER) of the item in registers as order-preserving 32-bit
//     keys; their max and min are reduced while the keys are made.
//   * Threshold: MSB-first radix select with 11-bit digits starting at the
//     highest bit in which the item's max and min keys differ (all keys share
//     the bits above it).  One LDS histogram (2,048 bins) locates the digit of
//     the k-th key; the keys of that bin (usually a few dozen) are then copied
//     to an LDS list and one wave finishes the remaining bits with ballot
//     counts, without further workgroup barriers.  A bin too large for the
//     list takes further histogram passes instead.  The result is the exact
//     threshold key T and the number of T-valued keys still needed.
//   * Ordered emission: each thread counts its keys > T and == T (packed in
//     one word), one block scan turns the counts into offsets, and each chosen
//     key lands at (#greater before it) + min(#equal before it, needed
//     equal): ascending output, ties to the lower column.
//   * Wave-level scans and reductions use DPP row shifts and row broadcasts
//     (no LDS round trips).
//   * Long rows: a tournament over chunks.  The running top-k (at most k keys
//     and columns, ascending) stays in LDS and precedes the next chunk in the
//     same ordered selection; the top-k of (carry ++ chunk) is the top-k of
//     everything seen so far.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;                    // 11-bit digits
constexpr int kCandCap = 1024;                 // keys of one bin finished without more passes
constexpr int kRankCap = 256;                  // ... by direct ranking (else bit by bit)
constexpr int64_t kSplitChunk = 32 * kThreads; // columns of one single-chunk item

// DPP move with 0 in lanes whose source is outside the pattern.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 within each
// 16-lane row, then lane 15 into rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_or0<0x111, 0xF>(x);
  x += dpp_or0<0x112, 0xF>(x);
  x += dpp_or0<0x114, 0xF>(x);
  x += dpp_or0<0x118, 0xF>(x);
  x += dpp_or0<0x142, 0xA>(x);
  x += dpp_or0<0x143, 0xC>(x);
  return x;
}

// Maximum over the 64 lanes (same pattern; lane 63 ends with the result).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_or0<0x111, 0xF>(x));
  x = max(x, dpp_or0<0x112, 0xF>(x));
  x = max(x, dpp_or0<0x114, 0xF>(x));
  x = max(x, dpp_or0<0x118, 0xF>(x));
  x = max(x, dpp_or0<0x142, 0xA>(x));
  x = max(x, dpp_or0<0x143, 0xC>(x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Exclusive scan over the workgroup in thread order (one barrier); `scr`
// holds kWaves entries.  *total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scr,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) scr[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t x = scr[w];
    before += (w < wave) ? x : 0u;
    all += x;
  }
  *total = all;
  return before + incl - v;
}

struct Item {
  int64_t row, base;
  int n;         // columns of this item
  bool first, last;
};

// Work item `it` of workgroup g.  Normally rows g, g + G, ..., each row's
// chunks in order (a tournament over them).  SPLIT (first pass of the
// chunk-parallel top-k): items g, g + G, ... of the rows x chunks grid, each
// chunk selected on its own into output row row * chunks_per_row + chunk.
// A row's visible prefix is fixed_n columns when fixed_n >= 0 (second pass:
// the candidate lists), else the causal prefix of its position.
template <int kChunk, bool SPLIT>
__device__ __forceinline__ bool item_of(int64_t it, int64_t rows, int64_t q_pos0, int64_t g,
                                        int64_t G, int chunks_per_row, int64_t fixed_n,
                                        Item* o) {
  int64_t row;
  int ch;
  if (SPLIT) {
    const int64_t id = g + it * G;
    row = id / chunks_per_row;
    ch = static_cast<int>(id - row * chunks_per_row);
  } else {
    const int64_t r_local = it / chunks_per_row;
    ch = static_cast<int>(it - r_local * chunks_per_row);
    row = g + r_local * G;
  }
  if (row >= rows) return false;
  const int64_t vis = fixed_n >= 0 ? fixed_n : visible_rows(q_pos0 + row);
  const int64_t base = static_cast<int64_t>(ch) * kChunk;
  o->row = row;
  o->base = base;
  int64_t n = vis - base;
  if (n > kChunk) n = kChunk;
  if (n < 0) n = 0;
  o->n = static_cast<int>(n);
  o->first = SPLIT || ch == 0;
  o->last = SPLIT || (ch == chunks_per_row - 1) || (base + kChunk >= vis);
  return true;
}

// LDS slot of 16-byte chunk c of an item.  Within each 1 KiB block (64
// chunks) the chunk index is XOR-permuted so that thread t, reading chunk v of
// its own 128-byte run (chunk 8t + v), never shares a bank group with the 15
// other lanes of its 16-lane phase: low 3 bits v ^ (t & 7), bit 3 flipped on
// odd blocks.
__device__ __forceinline__ int chunk_slot(int c) {
  const int i = c >> 6, lp = c & 63, a = lp >> 3;
  return i * 64 + 8 * (a ^ (i & 1)) + ((lp & 7) ^ a);
}

// Copy the 16-byte chunks covering item columns [0, n) to LDS `buf` in the
// chunk_slot order.  A partial last chunk is copied whole: rows are allocated
// `stride` floats with stride % 4 == 0, so its columns past n are in bounds
// (their values are never used).  Wave w issues the 1 KiB blocks w, w + 16,
// ...; lane L of block i writes slot 64i + L and fetches the chunk that maps
// there; a lane whose chunk lies past the last one re-reads the block's first
// chunk (always valid) and its bytes are never used.
// `half` selects every other block of the wave (0: w, w + 32, ...; 1: w + 16,
// w + 48, ...), so an item can be issued in two parts.
__device__ __forceinline__ void issue_item(const float* src, int n, float* buf, int wave,
                                           int half) {
  const int n4 = (n + 3) & ~3;
  const int lane = threadIdx.x & 63;
  for (int i = wave + half * kWaves; i * 256 < n4; i += 2 * kWaves) {
    const int a = ((lane >> 3) & 7) ^ (i & 1);
    const int lp = 8 * a + ((lane & 7) ^ a);
    const int e = i * 256 + 4 * lp;
    global_to_lds16(src + (e + 4 <= n4 ? e : i * 256), buf + i * 256);
  }
}

// PER: columns per thread (chunk = PER * 1,024 columns).  DMA: rows start on
// 16-byte boundaries, so items are copied with LDS DMA ahead of their use;
// otherwise each item is loaded synchronously.
// Chunk-parallel top-k of a few long rows, in two passes over this kernel:
//   SPLIT: every (row, chunk) item is selected on its own; output row
//     row * chunks_per_row + chunk of out_idx gets the chunk's chosen
//     columns (ascending, -1 padded) and the same row of cand_score their
//     scores (-inf padded);
//   then, with fixed_n = chunks_per_row * topk and remap = those columns:
//     the top-k of each row's candidate scores, the chosen positions mapped
//     back to columns through remap (same layout as the scores).
// Exact: the top-k of a union under the total order (score desc, column
// asc) is the top-k of the union of each part's top-k, and a row's
// candidates lie in column order (chunks in order, each ascending, pads
// last and never chosen while every row shows at least topk columns).
enum TopkPass { kRows = 0, kSplit = 1, kMerge = 2 };

template <int CPT, int PER, bool DMA, int PASS>
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ scores, int64_t rows, int64_t stride, int64_t q_pos0,
            int topk, int chunks_per_row, int32_t* __restrict__ out_idx, int64_t fixed_n,
            const int32_t* __restrict__ remap, float* __restrict__ cand_score) {
  constexpr bool SPLIT = PASS == kSplit;
  constexpr int KMAX = CPT > 0 ? CPT * kThreads : 1;
  constexpr int kPer = PER;
  constexpr int kChunk = PER * kThreads;
  constexpr int kCE = kCandCap / 64;  // list entries per lane of the finishing wave
  // Histogram + candidate list while the threshold is found, then the item's
  // output row staged for one coalesced copy (top-k <= 2,048 for CPT == 2,
  // which keeps that variant inside 160 KiB of LDS).
  // With a single chunk per row (CPT == 0) the output row has its own area
  // and is copied out at the start of the next item, after the end-of-item
  // barrier; otherwise it reuses the work area.
  constexpr bool kSepOut = CPT == 0;
  constexpr int kWork = kSepOut ? kBins + kCandCap : (CPT == 2 ? kBins + kCandCap : 4096);
  static_assert(kWork >= kBins + kCandCap, "work area");
  __shared__ __attribute__((aligned(16))) float rowbuf[kChunk];
  __shared__ __attribute__((aligned(16))) uint32_t work[kWork];
  __shared__ int32_t out_sep[kSepOut ? 4096 : 1];
  uint32_t* const hist = work;
  uint32_t* const cand = work + kBins;
  int32_t* const obuf = kSepOut ? out_sep : reinterpret_cast<int32_t*>(work);
  Item pend;  // item whose staged output awaits its copy (kSepOut)
  bool have_pend = false;
  int pend_need = 0;
  auto copy_out = [&](const Item& itm, int nsel) {
    // output row: the row, or (row, chunk) in the chunk-parallel pass
    const int64_t orow = SPLIT ? itm.row * chunks_per_row + itm.base / kChunk : itm.row;
    int32_t* d = out_idx + orow * static_cast<int64_t>(topk);
    if (SPLIT) {
      float* ds = cand_score + orow * static_cast<int64_t>(topk);
      const float* sr = scores + itm.row * stride;
      for (int j = static_cast<int>(threadIdx.x); j < topk; j += kThreads) {
        const int32_t col = j < nsel ? obuf[j] : -1;
        d[j] = col;
        ds[j] = col >= 0 ? sr[col] : -INFINITY;
      }
    } else if (PASS == kMerge) {
      const int32_t* rm = remap + itm.row * stride;
      for (int j = static_cast<int>(threadIdx.x); j < topk; j += kThreads)
        d[j] = j < nsel ? rm[obuf[j]] : -1;
    } else {
      for (int j = static_cast<int>(threadIdx.x); j < topk; j += kThreads)
        d[j] = j < nsel ? obuf[j] : -1;
    }
  };
  __shared__ uint32_t scr[2][kWaves];
  __shared__ uint32_t s_red[4][kWaves];
  __shared__ uint32_t s_bin, s_cum, s_cnt, s_ncand, s_T, s_rem;
  __shared__ uint32_t ckey[KMAX];
  __shared__ int32_t cidx[KMAX];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x, G = gridDim.x;

  uint32_t key[kPer];
  Item cur, nx;
  int64_t it = 0;
  if (!item_of<kChunk, SPLIT>(it, rows, q_pos0, g, G, chunks_per_row,
                              PASS == kMerge ? fixed_n : -1, &cur))
    return;
  if (DMA) {
    issue_item(scores + cur.row * stride + cur.base, cur.n, rowbuf, wave, 0);
    issue_item(scores + cur.row * stride + cur.base, cur.n, rowbuf, wave, 1);
  }
  int c = 0;  // carry entries of the current row

  while (true) {
    if (!DMA) {
      const float* src = scores + cur.row * stride + cur.base;
      for (int e = tid; e < cur.n; e += kThreads) rowbuf[e] = src[e];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of the item landed
    __syncthreads();                       // ... and every other wave's
    // Only the wave holding the item's end has columns past it; every other
    // wave skips the validity tests (uniform branches on wave_full).
    const bool wave_full = (wave * 64 + 63) * kPer + kPer <= cur.n;
    const int lim = cur.n - tid * kPer;  // valid columns of this thread (if < kPer)
    {
      // keys; 0 marks a column past the item's end (no float maps to key 0).
      // Every thread reads its PER columns with vector reads (always inside
      // the row buffer); only the wave holding the item's end masks them.
      const int e0 = tid * kPer;
#pragma unroll
      for (int v = 0; v < kPer / 4; ++v) {
        const int slot = DMA ? chunk_slot((e0 >> 2) + v) : (e0 >> 2) + v;
        const float4 x = *reinterpret_cast<const float4*>(&rowbuf[4 * slot]);
        key[4 * v] = float_key(x.x);
        key[4 * v + 1] = float_key(x.y);
        key[4 * v + 2] = float_key(x.z);
        key[4 * v + 3] = float_key(x.w);
      }
      // the item's key range, reduced per wave now (published by the barrier
      // below); min over valid keys is max over their complements
      uint32_t kmax = 0u, nmin = 0u;
      if (wave_full) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          kmax = max(kmax, key[j]);
          nmin = max(nmin, ~key[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          key[j] = j < lim ? key[j] : 0u;
          kmax = max(kmax, key[j]);
          nmin = max(nmin, j < lim ? ~key[j] : 0u);
        }
      }
      kmax = wave_max(kmax);
      nmin = wave_max(nmin);
      if (lane == 0) { s_red[0][wave] = kmax; s_red[1][wave] = nmin; }
      // the first histogram pass's table, cleared ahead of the barrier
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
      if (tid == 0) s_ncand = 0u;
    }
    const bool have_next =
        item_of<kChunk, SPLIT>(it + 1, rows, q_pos0, g, G, chunks_per_row,
                               PASS == kMerge ? fixed_n : -1, &nx);
    __syncthreads();  // every thread has its keys: the row buffer takes the next item
    if (DMA && have_next) issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf, wave, 0);
    bool second_half = DMA && have_next;  // the rest of the next item's copy, issued later
    if (kSepOut && have_pend) {
      copy_out(pend, pend_need);  // the previous item's staged row
      have_pend = false;
    }
    if (cur.first) c = 0;
    // chunk slots past a shorter row's end carry no work (uniform branch)
    if (!cur.first && cur.n == 0) {
      if (second_half) issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf, wave, 1);
      if (!have_next) break;
      cur = nx;
      ++it;
      continue;
    }

    const int n = cur.n;
    // carry (previous chunks' running top-k), CPT entries per thread, in order
    uint32_t ck[CPT > 0 ? CPT : 1];
    int32_t ci[CPT > 0 ? CPT : 1];
    int cv = 0;
    if (CPT > 0) {
      cv = c - tid * CPT;
      cv = cv < 0 ? 0 : (cv > CPT ? CPT : cv);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        ck[j] = j < cv ? ckey[tid * CPT + j] : 0u;
        ci[j] = j < cv ? cidx[tid * CPT + j] : -1;
      }
    }
    const int E = c + n;
    const int need = E < topk ? E : topk;
    uint32_t T = 0u, need_eq = 0u;  // need == E: every valid key (> 0) is chosen
    if (second_half && !(need < E)) {
      issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf, wave, 1);
      second_half = false;
    }

    if (need < E) {
      if (CPT > 0) {
        uint32_t kmax = 0u, nmin = 0u;
#pragma unroll
        for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j) {
          kmax = max(kmax, ck[j]);
          nmin = max(nmin, ck[j] ? ~ck[j] : 0u);
        }
        kmax = wave_max(kmax);
        nmin = wave_max(nmin);
        if (lane == 0) { s_red[2][wave] = kmax; s_red[3][wave] = nmin; }
        __syncthreads();
      }
      uint32_t mx = 0u, nmn = 0u;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mx = max(mx, s_red[0][w]);
        nmn = max(nmn, s_red[1][w]);
        if (CPT > 0) { mx = max(mx, s_red[2][w]); nmn = max(nmn, s_red[3][w]); }
      }
      const uint32_t mn = ~nmn;

      uint32_t remaining = static_cast<uint32_t>(need);
      uint32_t prefix, mask;
      int shift;
      if (mx == mn) {
        prefix = mx;
        mask = 0xffffffffu;
        shift = 0;
      } else {
        const int hb = 31 - __builtin_clz(mx ^ mn);
        mask = (hb == 31) ? 0u : ~((2u << hb) - 1u);
        prefix = mx & mask;
        shift = hb + 1;
      }
      bool first_pass = true;
      while (shift > 0) {
        const int dbits = shift < 11 ? shift : 11;
        shift -= dbits;
        const uint32_t dmask = (1u << dbits) - 1u;
        if (!first_pass) {
          for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
          if (tid == 0) s_ncand = 0u;
          __syncthreads();
        }
        // every valid key shares the max/min prefix, so the first pass counts
        // all of them
        if (first_pass && wave_full) {
#pragma unroll
          for (int j = 0; j < kPer; ++j) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
        } else {
#pragma unroll
          for (int j = 0; j < kPer; ++j)
            if (j < lim && (first_pass || (key[j] & mask) == prefix))
              atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
        }
#pragma unroll
        for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
          if (j < cv && (first_pass || (ck[j] & mask) == prefix))
            atomicAdd(&hist[(ck[j] >> shift) & dmask], 1u);
        first_pass = false;
        __syncthreads();
        if (second_half) {
          issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf, wave, 1);
          second_half = false;
        }
        if (wave == 0) {
          // lane l owns bins 32l .. 32l+31 as 8 groups of 4; suffix sums over
          // lanes locate the lane, then the group, then the bin
          uint32_t gs[8];
          uint32_t own = 0;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const u32x4_t q4 = *reinterpret_cast<const u32x4_t*>(&hist[32 * lane + 4 * v]);
            gs[v] = q4[0] + q4[1] + q4[2] + q4[3];
            own += gs[v];
          }
          // bins of lanes >= this one: the total minus the exclusive prefix
          const uint32_t pre = wave_incl_scan(own);
          const uint32_t all =
              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pre), 63));
          const uint32_t incl = all - pre + own;
          const uint32_t above = incl - own;
          if (above < remaining && remaining <= incl) {
            uint32_t cum = above;
            int gv = 0;
#pragma unroll
            for (int v = 7; v >= 0; --v) {
              if (cum + gs[v] >= remaining) { gv = v; break; }
              cum += gs[v];
            }
            const u32x4_t q4 = *reinterpret_cast<const u32x4_t*>(&hist[32 * lane + 4 * gv]);
            int b = 0;
#pragma unroll
            for (int v = 3; v >= 0; --v) {
              if (cum + q4[v] >= remaining) { b = v; break; }
              cum += q4[v];
            }
            s_bin = static_cast<uint32_t>(32 * lane + 4 * gv + b);
            s_cum = cum;
            s_cnt = q4[b];
          }
        }
        __syncthreads();
        remaining -= s_cum;
        prefix |= s_bin << shift;
        mask |= dmask << shift;
        const uint32_t in_bin = s_cnt;  // keys sharing the digits so far; remaining <= in_bin
        if (shift > 0 && in_bin <= static_cast<uint32_t>(kCandCap)) {
          // ---- finish: list the bin's keys, one wave resolves the low bits
          uint32_t mk = 0;
#pragma unroll
          for (int j = 0; j < kPer; ++j)
            mk |= static_cast<uint32_t>((key[j] & mask) == prefix) << j;
          if (!wave_full) mk &= lim >= kPer ? 0xffffffffu : (lim > 0 ? (1u << lim) - 1u : 0u);
          uint32_t mc = 0;
#pragma unroll
          for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
            mc |= static_cast<uint32_t>(j < cv && (ck[j] & mask) == prefix) << j;
          const uint32_t cnt = __popc(mk) + __popc(mc);
          if (cnt) {
            uint32_t pos = atomicAdd(&s_ncand, cnt);
            // the matches number exactly in_bin <= kCandCap; the guard only
            // keeps the writes inside the list
#pragma unroll
            for (int j = 0; j < kPer; ++j)
              if (((mk >> j) & 1u) && pos < kCandCap) cand[pos++] = key[j];
#pragma unroll
            for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
              if (((mc >> j) & 1u) && pos < kCandCap) cand[pos++] = ck[j];
          }
          __syncthreads();
          if (in_bin <= static_cast<uint32_t>(kRankCap)) {
            // thread i ranks list entry i against the whole list (broadcast
            // reads); the entry with #greater < remaining <= #greater-or-equal
            // is the threshold (equal entries write equal values)
            if (static_cast<uint32_t>(tid) < in_bin) {
              const uint32_t x = cand[tid];
              uint32_t gt = 0, ge = 0;
              for (uint32_t m4 = 0; m4 < in_bin; m4 += 4) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&cand[m4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const bool ok = m4 + i < in_bin;
                  gt += ok && v[i] > x;
                  ge += ok && v[i] >= x;
                }
              }
              if (gt < remaining && remaining <= ge) { s_T = x; s_rem = remaining - gt; }
            }
          } else if (wave == 0) {
            // larger lists: one wave settles the low bits one at a time with
            // ballot counts
            uint32_t x[kCE];
            uint32_t alive = 0u;  // bit e: entry lane + 64e is still a candidate
#pragma unroll
            for (int e = 0; e < kCE; ++e) {
              const uint32_t idx = static_cast<uint32_t>(lane + 64 * e);
              x[e] = idx < in_bin ? cand[idx] : 0u;
              alive |= static_cast<uint32_t>(idx < in_bin) << e;
            }
            uint32_t pfx = prefix, rem = remaining;
            for (int b = shift - 1; b >= 0; --b) {
              uint32_t ones = 0u;  // alive entries with bit b set
              uint32_t c1 = 0u;
#pragma unroll
              for (int e = 0; e < kCE; ++e) {
                if (64u * e >= in_bin) continue;  // uniform (a break would stop the unrolling)
                const bool one = ((alive >> e) & 1u) && ((x[e] >> b) & 1u);
                ones |= static_cast<uint32_t>(one) << e;
                c1 += static_cast<uint32_t>(__popcll(__ballot(one)));
              }
              if (c1 >= rem) {
                pfx |= 1u << b;
                alive = ones;
              } else {
                rem -= c1;
                alive &= ~ones;
              }
            }
            if (lane == 0) { s_T = pfx; s_rem = rem; }
          }
          __syncthreads();
          prefix = s_T;
          remaining = s_rem;
          shift = 0;
        }
      }
      T = prefix;
      need_eq = remaining;
    }
    // every path issues the rest of the next item's copy before the emission
    // (an item whose keys are all equal skips the histogram loop above)
    if (second_half) {
      issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf, wave, 1);
      second_half = false;
    }

    // ---- ordered emission: carry entries first, then the chunk, thread order
    uint32_t c_gt = 0, c_eq = 0;
#pragma unroll
    for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
      if (j < cv) { c_gt += ck[j] > T; c_eq += ck[j] == T; }
    uint32_t gtm = 0, eqm = 0;  // this thread's keys > T / == T, bit j = column j
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      gtm |= static_cast<uint32_t>(key[j] > T) << j;
      eqm |= static_cast<uint32_t>(key[j] == T) << j;  // key 0 only equals T = 0 (need_eq = 0)
    }
    // counts packed as (greater | equal << 16): each total is at most
    // carry + chunk < 65,536
    uint32_t tot_c = 0, tot_k;
    uint32_t cb = 0;
    if (CPT > 0) cb = block_exclusive_scan(c_gt | (c_eq << 16), scr[0], &tot_c);
    const uint32_t kb = block_exclusive_scan(
        static_cast<uint32_t>(__popc(gtm)) | (static_cast<uint32_t>(__popc(eqm)) << 16), scr[1],
        &tot_k);
    const uint32_t kgt_b = (kb & 0xffffu) + (tot_c & 0xffffu);
    const uint32_t keq_b = (kb >> 16) + (tot_c >> 16);
    const bool to_out = (CPT == 0) || cur.last;
    if (CPT > 0) {
      // carry entries (at most CPT per thread)
      uint32_t gtb = cb & 0xffffu, eqb = cb >> 16;
#pragma unroll
      for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j) {
        if (j < cv) {
          const bool gt = ck[j] > T, eq = ck[j] == T;
          if (gt || (eq && eqb < need_eq)) {
            const uint32_t pos = gtb + (eqb < need_eq ? eqb : need_eq);
            if (to_out) obuf[pos] = ci[j];
            else { ckey[pos] = ck[j]; cidx[pos] = ci[j]; }
          }
          gtb += gt;
          eqb += eq;
        }
      }
    }
    const int32_t col0 = static_cast<int32_t>(cur.base) + tid * kPer;
    if (to_out) {
      // walk only the chosen columns: positions come from popcounts of the masks
      uint32_t m = gtm | eqm;
      while (m) {
        const int j = __builtin_ctz(m);
        m &= m - 1u;
        const uint32_t low = (1u << j) - 1u;
        const bool gt = (gtm >> j) & 1u;
        const uint32_t eqb = keq_b + __popc(eqm & low);
        if (gt || eqb < need_eq) {
          obuf[kgt_b + __popc(gtm & low) + (eqb < need_eq ? eqb : need_eq)] = col0 + j;
        } else {
          m &= gtm;  // later equal keys rank even lower
        }
      }
    } else {
      uint32_t gtb = kgt_b, eqb = keq_b;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool gt = key[j] > T, eq = key[j] == T;
        if (gt || (eq && eqb < need_eq)) {
          const uint32_t pos = gtb + (eqb < need_eq ? eqb : need_eq);
          ckey[pos] = key[j];  // every thread read its carry entries before the scans' barriers
          cidx[pos] = col0 + j;
        }
        gtb += gt;
        eqb += eq;
      }
    }
    c = need;
    if (to_out) {
      // the row's min(k, visible) choices (need of them) are staged in LDS;
      // they are copied out coalesced and padded with -1 once every thread's
      // writes are in: after the next barrier (kSepOut: at the next item)
      if (kSepOut) {
        pend = cur;
        have_pend = true;
        pend_need = need;
      } else {
        __syncthreads();
        copy_out(cur, need);
      }
    }
    __syncthreads();  // LDS tables / carry reused by the next item
    if (!have_next) {
      if (kSepOut && have_pend) copy_out(pend, pend_need);
      break;
    }
    cur = nx;
    ++it;
  }
}

// ---------------------------------------------------------------------------
// Rows held in registers (at most 32,768 visible columns): one wave per row
// up to 64 * KPL <= 4,096 columns (kShortWaves rows per workgroup, no
// workgroup barriers), else NW = 2, 4 or 8 waves of 4,096 columns each; few
// rows of 2,049 - 16,384 columns take 2, 4 or 8 waves of 2,048.  The same
// selection rule as above:
//   * lane L holds the float4 at columns 256v + 4L .. 256v + 4L + 3 of its
//     wave's block for v = 0 .. KPL/4 - 1 (each load instruction reads 1 KiB
//     contiguous), as keys key[4v + i]; columns past the visible prefix get
//     key 0, and only the steps v that reach past it test for that (a
//     wave-uniform branch);
//   * threshold: MSB-first radix select with 11-bit digits over a 2,048-bin
//     LDS histogram (private to the wave, or shared by the row's waves and
//     double-buffered), from the highest bit in which the row's keys differ
//     (OR of the keys and of their complements); once the bin holding the
//     k-th key has at most 64 keys they are listed, one per lane, and ballot
//     counts settle the remaining bits one at a time.  Waves of one row
//     exchange the ORs, list counts and chosen counts through LDS; every
//     wave searches the same table, so all take the same branches;
//   * list building and ordered emission give each key its place with one
//     packed wave scan per three steps (10-bit per-step counts), and every
//     key makes one unconditional LDS write, to its slot or to a slot of its
//     own lane that is never read (no per-key branches).  When every key
//     equal to the threshold T is chosen (the usual case) the choice is
//     simply key >= T; otherwise equal keys go to the lower columns.  The
//     chosen columns, ascending, are then copied to the output row, padded
//     with -1 to k.
// Longer rows run two passes of the same kernel (see RegPass below).
constexpr int kShortWaves = 4;  // waves (rows in flight) per workgroup

// Orders this wave's earlier LDS accesses before its later ones, across lanes.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// OR over the 64 lanes (row shifts and broadcasts as in wave_incl_scan).
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x |= dpp_or0<0x111, 0xF>(x);
  x |= dpp_or0<0x112, 0xF>(x);
  x |= dpp_or0<0x114, 0xF>(x);
  x |= dpp_or0<0x118, 0xF>(x);
  x |= dpp_or0<0x142, 0xA>(x);
  x |= dpp_or0<0x143, 0xC>(x);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Exclusive prefix over the lanes of a packed count, and the wave's total.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t x, uint32_t* total) {
  const uint32_t incl = wave_incl_scan(x);
  *total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  return incl - x;
}

// Writes the 4-key steps v0 .. v0+2 (those below kSteps) of this lane in
// column order: key j is "taken" when take(j); taken keys land at
// dst[base + (taken keys before them)] and the others at dst[spare];
// base advances by the step group's total.  One wave scan of three 10-bit
// counts (at most 4 per lane and step, 256 per wave) serves the group.
template <int kSteps, typename Take, typename Val, typename Dst>
__device__ __forceinline__ void place_group(int v0, uint32_t& base, uint32_t spare, Take take,
                                            Val val, Dst* dst) {
  uint32_t packed = 0u;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (v0 + s < kSteps) {
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) c += take(4 * (v0 + s) + i);
      packed |= c << (10 * s);
    }
  }
  uint32_t tot;
  const uint32_t ex = wave_excl_scan(packed, &tot);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (v0 + s < kSteps) {
      uint32_t pos = base + ((ex >> (10 * s)) & 1023u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (v0 + s) + i;
        const bool t = take(j);
        dst[t ? pos : spare] = val(j);
        pos += t;
      }
      base += (tot >> (10 * s)) & 1023u;
    }
  }
}

// The register kernel's passes:
//   kRegRows:  each row's top-k of its visible prefix (the per-row selection);
//   kRegChunk: each (row, chunk) pair, a chunk being kRegChunkCols columns of
//              the row's visible prefix, on its own: its chosen scores and
//              (row) columns in column order, padded with -inf / -1 to k;
//   kRegMerge: each row's top-k of the n2 candidates of its chunks (in chunk
//              order, so in column order), mapped back to columns.
// Exact for the same reason as the two-pass top-k above: the top-k of a
// union under (score desc, column asc) is the top-k of the parts' top-k,
// and the padding is never chosen while the row shows at least k columns.
enum RegPass { kRegRows = 0, kRegChunk = 1, kRegMerge = 2 };
constexpr int kRegChunkCols = 8 * 64 * 64;  // one chunk: 8 waves of 4,096 columns

struct RegArgs {
  const float* scores;  // kRegRows, kRegChunk: score rows; kRegMerge: candidate scores
  int64_t rows, stride, q_pos0;
  int topk, cap, words;
  int32_t* out_idx;     // kRegRows, kRegMerge
  // kRegChunk: chunks per row.  The candidates of (row, chunk) go to
  // cand_score / cand_col + (row * cpr + chunk) * topk; with cand_score null,
  // into the chunk's own first 2 topk floats instead (its scores, then its
  // columns as int32), which the chunk no longer needs once selected.
  int cpr;
  float* cand_score;
  int32_t* cand_col;
  // kRegMerge: n2 candidates per row; candidate c sits at float
  // (c / topk) * cstride + c % topk of its row (cstride == topk: contiguous),
  // and its column at the same offset of col_base + row * col_stride.
  int n2;
  int cstride;
  const int32_t* col_base;
  int64_t col_stride;
  uint32_t kmagic;  // floor(2^32 / topk) + 1: c / topk == mulhi(c, kmagic) for c < 2^20
};

template <int KPL, int NW, int PASS>
__global__ void __launch_bounds__(64 * (NW == 1 ? kShortWaves : NW), 4)
topk_reg_kernel(const RegArgs a) {
  static_assert(PASS != kRegChunk || (NW == 8 && KPL == 64), "a chunk is 8 waves of 4,096 columns");
  const float* const __restrict__ scores = a.scores;
  const int64_t rows = a.rows, stride = a.stride, q_pos0 = a.q_pos0;
  const int topk = a.topk, cap = a.cap, words = a.words;
  int32_t* const __restrict__ out_idx = a.out_idx;
  static_assert(KPL % 4 == 0 && KPL <= 64, "keys per lane");
  static_assert(NW == 1 || KPL == 64 || KPL == 32,
                "rows of several waves hold 4,096 or 2,048 columns per wave");
  constexpr int kSteps = KPL / 4;
  constexpr int kRowsPerWG = NW == 1 ? kShortWaves : 1;
  constexpr int kCols = 64 * KPL;  // columns of one wave
  // per row: the histogram (two of kBins words when several waves share the
  // row, so that one can be cleared while the other is read) while the
  // threshold is found, then the chosen columns (cap of them, 16-bit) + one
  // spare slot per lane
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_all[];
  __shared__ uint32_t cand_all[kRowsPerWG * NW][128];  // per wave: bin list + spare slots
  __shared__ uint32_t xch[4][NW];                       // cross-wave exchange (NW > 1)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rslot = NW == 1 ? wave : 0;  // row of this wave within the workgroup
  const int wr = NW == 1 ? 0 : wave;     // part of the row held by this wave
  // item: a row, or (kRegChunk) a (row, chunk) pair per workgroup
  const int64_t item = PASS == kRegChunk ? static_cast<int64_t>(blockIdx.x)
                                         : static_cast<int64_t>(blockIdx.x) * kRowsPerWG + rslot;
  const int64_t row = PASS == kRegChunk ? item / a.cpr : item;
  const int64_t chunk = PASS == kRegChunk ? item - row * a.cpr : 0;
  if (row >= rows) return;  // NW > 1: the whole workgroup (one item)
  uint32_t* const row_lds = lds_all + rslot * words;
  uint16_t* const ob = reinterpret_cast<uint16_t*>(row_lds);
  uint32_t* const cand = cand_all[wave];
  int vis;  // the item's columns
  if (PASS == kRegChunk) {
    const int64_t v = visible_rows(q_pos0 + row) - chunk * kRegChunkCols;
    vis = static_cast<int>(v < 0 ? 0 : (v > kRegChunkCols ? kRegChunkCols : v));
  } else if (PASS == kRegMerge) {
    vis = a.n2;
  } else {
    vis = static_cast<int>(visible_rows(q_pos0 + row));
  }
  const float* const rsrc = scores + row * stride + chunk * kRegChunkCols;
  // float offset of item column c from rsrc (kRegMerge: candidate c's score);
  // with topk % 4 == 0 four candidates c .. c+3 (c % 4 == 0) are adjacent
  auto addr = [&](int c) -> int {
    if (PASS != kRegMerge) return c;
    const uint32_t qd = __umulhi(static_cast<uint32_t>(c), a.kmagic);
    return static_cast<int>(qd) * a.cstride + (c - static_cast<int>(qd) * topk);
  };
  const int need = vis < topk ? vis : topk;  // <= cap
  const int col0 = wr * kCols;
  const int nthr = 64 * NW, tid_r = 64 * wr + lane;  // threads of the row, and this one
  int32_t* const dst = out_idx + row * static_cast<int64_t>(topk);
  auto row_sync = [&]() {
    if (NW == 1) wave_lds_sync();
    else __syncthreads();
  };
  // Output of the chunk and merge passes: slot j < nsel holds item column
  // idx(j); the other slots up to k are padding.
  auto write_out = [&](int nsel, auto idx) {
    if constexpr (PASS == kRegMerge) {
      const int32_t* cb = a.col_base + row * a.col_stride;
      for (int j = tid_r; j < topk; j += nthr) dst[j] = j < nsel ? cb[addr(idx(j))] : -1;
    } else if constexpr (PASS == kRegChunk) {
      // every thread reads its slots' scores first: written in place, they
      // overwrite the chunk's first columns
      constexpr int kPer = (kMaxTopk + 64 * NW - 1) / (64 * NW);
      float sv[kPer];
      int32_t cv[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int j = tid_r + u * nthr;
        const int c = j < nsel ? idx(j) : -1;
        sv[u] = c >= 0 ? rsrc[c] : -INFINITY;
        cv[u] = c >= 0 ? static_cast<int32_t>(chunk * kRegChunkCols + c) : -1;
      }
      __syncthreads();
      float* const os = a.cand_score ? a.cand_score + item * topk : const_cast<float*>(rsrc);
      int32_t* const oc = a.cand_score ? a.cand_col + item * topk
                                       : reinterpret_cast<int32_t*>(const_cast<float*>(rsrc) + topk);
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int j = tid_r + u * nthr;
        if (j < topk) { os[j] = sv[u]; oc[j] = cv[u]; }
      }
    }
  };
  auto clear_hist = [&](uint32_t* h) {  // the row's threads clear kBins words
#pragma unroll
    for (int v = 0; v < kBins / (256 * NW); ++v)
      *reinterpret_cast<u32x4_t*>(&h[4 * (tid_r + nthr * v)]) = u32x4_t{0u, 0u, 0u, 0u};
  };
  auto hist_of = [&](int pass) { return row_lds + (NW > 1 ? (pass & 1) * kBins : 0); };

  if (need < vis) {
    const float* src = rsrc;
    // loads: lanes past the prefix re-read its last float4 (rows hold
    // `stride` >= vis floats with stride % 4 == 0, so that float4 is in
    // bounds); their keys are cleared below.  A wave wholly past the prefix
    // loads nothing.
    const int clast = (vis - 1) & ~3;
    float4 x[kSteps];
    if (col0 < vis) {
#pragma unroll
      for (int v = 0; v < kSteps; ++v) {
        const int c = col0 + 256 * v + 4 * lane;
        x[v] = *reinterpret_cast<const float4*>(src + addr(c < clast ? c : clast));
      }
    } else {
#pragma unroll
      for (int v = 0; v < kSteps; ++v) x[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    uint32_t key[KPL];
    uint32_t kor = 0u, nor = 0u;  // OR of the valid keys, and of their complements
#pragma unroll
    for (int v = 0; v < kSteps; ++v) {
      uint32_t k0 = float_key(x[v].x), k1 = float_key(x[v].y);
      uint32_t k2 = float_key(x[v].z), k3 = float_key(x[v].w);
      if (col0 + 256 * v + 256 > vis) {  // uniform: this step reaches past the prefix
        const int c = col0 + 256 * v + 4 * lane;
        k0 = c < vis ? k0 : 0u;
        k1 = c + 1 < vis ? k1 : 0u;
        k2 = c + 2 < vis ? k2 : 0u;
        k3 = c + 3 < vis ? k3 : 0u;
        nor |= (k0 ? ~k0 : 0u) | (k1 ? ~k1 : 0u) | (k2 ? ~k2 : 0u) | (k3 ? ~k3 : 0u);
      } else {
        nor |= ~k0 | ~k1 | ~k2 | ~k3;
      }
      kor |= k0 | k1 | k2 | k3;
      key[4 * v] = k0;
      key[4 * v + 1] = k1;
      key[4 * v + 2] = k2;
      key[4 * v + 3] = k3;
    }
    kor = wave_or(kor);
    nor = wave_or(nor);
    if (NW > 1) {
      if (lane == 0) { xch[0][wr] = kor; xch[1][wr] = nor; }
      clear_hist(hist_of(0));
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NW; ++w) { kor |= xch[0][w]; nor |= xch[1][w]; }
    }
    const uint32_t diff = kor & nor;  // bits in which the valid keys differ
    uint32_t remaining = static_cast<uint32_t>(need);
    uint32_t prefix, mask, n_eq;
    int shift;
    if (diff == 0u) {  // one value
      prefix = kor;
      mask = 0xffffffffu;
      shift = 0;
      n_eq = static_cast<uint32_t>(vis);
    } else {
      const int hb = 31 - __builtin_clz(diff);
      mask = (hb == 31) ? 0u : ~((2u << hb) - 1u);
      prefix = kor & mask;
      shift = hb + 1;
      n_eq = 0u;
    }
    // Every decision below depends only on values the row's waves share, so
    // all of them take the same branches and reach the same barriers.
    int pass = 0;
    while (shift > 0) {
      // the keys pass through an empty asm, so that per-key tests are made in
      // each pass rather than hoisted out of this loop as 64 lane masks
#pragma unroll
      for (int j = 0; j < KPL; ++j) asm volatile("" : "+v"(key[j]));
      const int dbits = shift < 11 ? shift : 11;
      shift -= dbits;
      const uint32_t dmask = (1u << dbits) - 1u;
      uint32_t* const hist = hist_of(pass);
      if (NW == 1) {
        clear_hist(hist);
        wave_lds_sync();
      } else if (pass > 0) {
        __syncthreads();  // this pass's table was cleared during the previous pass
      }
#pragma unroll
      for (int v = 0; v < kSteps; ++v) {
        // the first pass counts every valid key (all share the prefix)
        if (pass == 0 && col0 + 256 * v + 256 <= vis) {
#pragma unroll
          for (int i = 0; i < 4; ++i) atomicAdd(&hist[(key[4 * v + i] >> shift) & dmask], 1u);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k = key[4 * v + i];
            if (k && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
          }
        }
      }
      row_sync();  // every count is in
      // the other table is no longer read by anyone: clear it for the next pass
      if (NW > 1) clear_hist(hist_of(pass + 1));
      // lane l owns bins 32l .. 32l + 31 as 8 groups of 4; keys in higher
      // lanes' bins are larger.  The lane holding the k-th key is found by a
      // wave scan, then (in every lane, for its own bins) the group and bin.
      // Every wave of the row does this on the same table.
      uint32_t gs[8];
      uint32_t own = 0u;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const u32x4_t q4 = *reinterpret_cast<const u32x4_t*>(&hist[32 * lane + 4 * v]);
        gs[v] = q4[0] + q4[1] + q4[2] + q4[3];
        own += gs[v];
      }
      const uint32_t pre = wave_incl_scan(own);
      const uint32_t all =
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pre), 63));
      const uint32_t above = all - pre;
      uint32_t cum = above;
      int gv = 0;
      bool found = false;
#pragma unroll
      for (int v = 7; v >= 0; --v) {
        const bool f = !found && cum + gs[v] >= remaining;
        gv = f ? v : gv;
        cum += (found || f) ? 0u : gs[v];
        found = found || f;
      }
      const u32x4_t q4 = *reinterpret_cast<const u32x4_t*>(&hist[32 * lane + 4 * gv]);
      uint32_t b = 0u, cnt = q4[0];
      found = false;
#pragma unroll
      for (int i = 3; i >= 1; --i) {
        const bool f = !found && cum + q4[i] >= remaining;
        b = f ? static_cast<uint32_t>(i) : b;
        cnt = f ? q4[i] : cnt;
        cum += (found || f) ? 0u : q4[i];
        found = found || f;
      }
      // exactly one lane holds the bin: above < remaining <= above + own
      const uint64_t hit = __ballot(above < remaining && remaining <= above + own);
      const int hl = hit ? __builtin_ctzll(hit) : 0;
      const uint32_t bin = static_cast<uint32_t>(
          __builtin_amdgcn_readlane(static_cast<int>(32 * lane + 4 * gv + b), hl));
      remaining -= static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cum), hl));
      const uint32_t in_bin =
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cnt), hl));
      prefix |= bin << shift;
      mask |= dmask << shift;
      n_eq = in_bin;  // the count of keys equal to T once shift reaches 0
      if (NW == 1) wave_lds_sync();  // the table is read before it is cleared again
      if (shift > 0 && in_bin <= 64u) {
        // list the bin's keys: exactly in_bin keys match (the bin's count),
        // so every wave's list stays below 64 entries
        uint32_t base = 0u;
#pragma unroll
        for (int v0 = 0; v0 < kSteps; v0 += 3) {
          if (base >= in_bin) continue;  // uniform: the list is complete
          place_group<kSteps>(
              v0, base, 64u + lane,
              [&](int j) {
                const uint32_t k = key[j];
                // only steps reaching past the prefix hold key 0 (uniform test)
                return (col0 + 256 * (j >> 2) + 256 <= vis || k != 0u) && (k & mask) == prefix;
              },
              [&](int j) { return key[j]; }, cand);
        }
        if (NW > 1 && lane == 0) xch[2][wr] = base;
        row_sync();
        // one list entry per lane: the waves' lists in order
        bool in_list;
        uint32_t xk = 0u;
        if (NW == 1) {
          in_list = static_cast<uint32_t>(lane) < in_bin;
          if (in_list) xk = cand[lane];
        } else {
          uint32_t lo = 0u;
          int sw = -1;
          uint32_t si = 0u;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t c = xch[2][w];
            if (static_cast<uint32_t>(lane) >= lo && static_cast<uint32_t>(lane) < lo + c) {
              sw = w;
              si = static_cast<uint32_t>(lane) - lo;
            }
            lo += c;
          }
          in_list = sw >= 0;
          if (in_list) xk = cand_all[sw][si];
        }
        bool alive = in_list;
        for (int bb = shift - 1; bb >= 0; --bb) {
          const bool one = alive && ((xk >> bb) & 1u);
          const uint32_t c1 = static_cast<uint32_t>(__popcll(__ballot(one)));
          if (c1 >= remaining) {
            prefix |= 1u << bb;
            alive = one;
          } else {
            remaining -= c1;
            alive = alive && !one;
          }
        }
        n_eq = static_cast<uint32_t>(__popcll(__ballot(alive)));
        shift = 0;
      }
      ++pass;
    }
    const uint32_t T = prefix, need_eq = remaining;

    // ---- ordered emission into the row's LDS slots (over the histogram)
    const bool all_eq = n_eq == need_eq;  // every key equal to T is chosen
    uint32_t base = 0u, eq_base = 0u;     // chosen (> T, == T) in earlier columns
    if (NW > 1) {
      // this wave's counts; earlier waves' totals give its starting point
      // (keys >= T) | (keys > T) << 16, one count for both emission paths (a
      // count per path keeps far more registers live)
      uint32_t c = 0u;
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        c += static_cast<uint32_t>(key[j] >= T) | (static_cast<uint32_t>(key[j] > T) << 16);
      uint32_t tot;
      wave_excl_scan(c, &tot);
      // recompute the tests below rather than keep 64 lane masks
#pragma unroll
      for (int j = 0; j < KPL; ++j) asm volatile("" : "+v"(key[j]));
      if (lane == 0) xch[3][wr] = tot;
      __syncthreads();  // also: every wave is done with the histogram
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t t = w < wr ? xch[3][w] : 0u;
        const uint32_t ge = t & 0xffffu, gt = t >> 16;
        if (all_eq) base += ge;
        else { base += gt; eq_base += ge - gt; }
      }
    }
    const uint32_t spare = static_cast<uint32_t>(cap + 64 * wr + lane);
    auto col = [&](int j) {
      return static_cast<uint16_t>(col0 + 256 * (j >> 2) + 4 * lane + (j & 3));
    };
    if (all_eq) {
      // the choice is key >= T (T > 0, so cleared keys are never chosen);
      // exactly `need` keys qualify
#pragma unroll
      for (int v0 = 0; v0 < kSteps; v0 += 3) {
        if (base >= static_cast<uint32_t>(need)) continue;  // uniform: all placed
        place_group<kSteps>(v0, base, spare, [&](int j) { return key[j] >= T; }, col, ob);
      }
    } else {
      // some keys equal to T are left out: keys > T, and the first need_eq
      // keys == T in column order
      const uint32_t n_gt = static_cast<uint32_t>(need) - need_eq;
#pragma unroll
      for (int v = 0; v < kSteps; ++v) {
        if (base >= n_gt && eq_base >= need_eq) continue;  // uniform: all placed
        uint32_t c = 0u;  // (keys > T) | (keys == T) << 16 of this lane's step
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c += static_cast<uint32_t>(key[4 * v + i] > T) |
               (static_cast<uint32_t>(key[4 * v + i] == T) << 16);
        uint32_t tot;
        const uint32_t ex = wave_excl_scan(c, &tot);
        uint32_t g = base + (ex & 0xffffu), e = eq_base + (ex >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t k = key[4 * v + i];
          const bool gt = k > T, eq = k == T;
          const bool ch = gt || (eq && e < need_eq);
          ob[ch ? g + (e < need_eq ? e : need_eq) : spare] = col(4 * v + i);
          g += gt;
          e += eq;
        }
        base += tot & 0xffffu;
        eq_base += tot >> 16;
      }
    }
    row_sync();
    if constexpr (PASS != kRegRows) {
      write_out(need, [&](int j) { return static_cast<int>(ob[j]); });
    } else if ((topk & 3) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      for (int j = 4 * tid_r; j < topk; j += 4 * nthr) {
        uint2 w = make_uint2(0u, 0u);
        if (j < need) w = *reinterpret_cast<const uint2*>(&ob[j]);  // inside the row's slots
        int4 o;
        o.x = j < need ? static_cast<int>(w.x & 0xffffu) : -1;
        o.y = j + 1 < need ? static_cast<int>(w.x >> 16) : -1;
        o.z = j + 2 < need ? static_cast<int>(w.y & 0xffffu) : -1;
        o.w = j + 3 < need ? static_cast<int>(w.y >> 16) : -1;
        *reinterpret_cast<int4*>(dst + j) = o;
      }
    } else {
      for (int j = tid_r; j < topk; j += nthr) {
        int o = -1;
        if (j < need) o = ob[j];
        dst[j] = o;
      }
    }
  } else {
    // every visible column is chosen
    if constexpr (PASS != kRegRows) write_out(need, [&](int j) { return j; });
    else for (int j = tid_r; j < topk; j += nthr) dst[j] = j < need ? j : -1;
  }
}

// Longest row the register-resident kernels take (8 waves of 4,096 columns).
constexpr int64_t kRegMaxVis = kRegChunkCols;

// One pass of the register kernel over items of at most max_cols columns
// (kRegChunk: chunks of kRegChunkCols); a.cap and a.words are set here.
template <int PASS>
hipError_t launch_reg(RegArgs a, int64_t max_cols, hipStream_t s) {
  const int64_t items = PASS == kRegChunk ? a.rows * a.cpr : a.rows;
  a.cap = static_cast<int>(max_cols < a.topk ? max_cols : a.topk);  // chosen slots per item
  // Few items of 2,049 - 16,384 columns take twice the waves, 2,048 columns
  // each: a row on few waves is latency-bound (one row of 4,096 columns
  // takes 8 us on two waves, 10 us on one; of 8,192, 8.5 us on four, 11.6
  // us on two).  Many items fill the chip anyway, and the extra waves'
  // exchanges only add work (at 1,024 rows of 16,384 columns eight waves
  // each take 32 us, four 29 us).
  const bool wide = PASS != kRegChunk && max_cols > 32 * 64 && max_cols <= 4 * 64 * 64 &&
                    items <= (max_cols > 2 * 64 * 64 ? 512 : 1024);
  const bool two_short = wide && max_cols <= 64 * 64;
  if (PASS != kRegChunk && max_cols <= 64 * 64 && !two_short) {
    // one wave per item, kShortWaves items per workgroup; per wave the
    // histogram, later the chosen columns + 64 spare slots (16-bit)
    if (!dispatch_fits((items + kShortWaves - 1) / kShortWaves, 64 * kShortWaves))
      return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((items + kShortWaves - 1) / kShortWaves));
    const dim3 block(64 * kShortWaves);
    int words = (a.cap + 64 + 1) / 2;
    if (words < kBins) words = kBins;
    a.words = (words + 3) & ~3;
    const size_t lds = static_cast<size_t>(kShortWaves) * a.words * sizeof(uint32_t);
    constexpr int P1 = PASS == kRegChunk ? kRegRows : PASS;  // (never a chunk pass here)
    if (max_cols <= 1024)
      hipLaunchKernelGGL((topk_reg_kernel<16, 1, P1>), grid, block, lds, s, a);
    else if (max_cols <= 2048)
      hipLaunchKernelGGL((topk_reg_kernel<32, 1, P1>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((topk_reg_kernel<64, 1, P1>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  // one item per workgroup of NW waves; two histograms per item, later the
  // chosen columns + 64 spare slots per wave (cap + 64 NW <= 4,608 16-bit
  // slots, inside the 2 x kBins words)
  a.words = 2 * kBins;
  const size_t lds = static_cast<size_t>(a.words) * sizeof(uint32_t);
  if (!dispatch_fits(items, 512)) return hipErrorInvalidValue;  // at most 8 waves each
  const dim3 grid(static_cast<unsigned>(items));
  constexpr int P2 = PASS == kRegChunk ? kRegRows : PASS;  // chunk items take 8 waves
  if (PASS == kRegChunk || max_cols > 4 * 64 * 64)
    hipLaunchKernelGGL((topk_reg_kernel<64, 8, PASS>), grid, dim3(512), lds, s, a);
  else if (max_cols > 2 * 64 * 64 && wide)
    hipLaunchKernelGGL((topk_reg_kernel<32, 8, P2>), grid, dim3(512), lds, s, a);
  else if (max_cols > 2 * 64 * 64)
    hipLaunchKernelGGL((topk_reg_kernel<64, 4, P2>), grid, dim3(256), lds, s, a);
  else if (max_cols > 64 * 64 && wide)
    hipLaunchKernelGGL((topk_reg_kernel<32, 4, P2>), grid, dim3(256), lds, s, a);
  else if (max_cols > 64 * 64)
    hipLaunchKernelGGL((topk_reg_kernel<64, 2, P2>), grid, dim3(128), lds, s, a);
  else
    hipLaunchKernelGGL((topk_reg_kernel<32, 2, P2>), grid, dim3(128), lds, s, a);
  return hipGetLastError();
}

RegArgs reg_args(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0, int32_t topk,
                 int32_t* out_idx) {
  RegArgs a{};
  a.scores = scores;
  a.rows = rows;
  a.stride = stride;
  a.q_pos0 = q_pos0;
  a.topk = topk;
  a.out_idx = out_idx;
  return a;
}

// Whether the two register passes (chunks, then merge) serve these rows:
// row starts 16-byte aligned, k a multiple of 4 (the merge reads candidates
// four at a time), every row showing at least k columns (the padding is
// never chosen), at most 32,768 candidates per row, and, in place, room for
// the last chunk's 2 k candidate floats inside the row.
bool reg_split_ok(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                  int32_t topk, bool in_place) {
  if (rows <= 0 || (stride & 3) != 0 || (reinterpret_cast<uintptr_t>(scores) & 15) != 0 ||
      (topk & 3) != 0)
    return false;
  const int64_t max_vis = (q_pos0 + rows) / 4;
  const int64_t cpr = (max_vis + kRegChunkCols - 1) / kRegChunkCols;
  if (cpr < 2 || cpr * topk > kRegMaxVis || (q_pos0 + 1) / 4 < topk) return false;
  return !in_place || (cpr - 1) * kRegChunkCols + 2 * static_cast<int64_t>(topk) <= stride;
}

// The two register passes; candidates in cand_score / cand_col (rows * cpr *
// topk each), or in place in the score rows when cand_score is null.
hipError_t launch_reg_split(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                            int32_t topk, int32_t* out_idx, float* cand_score, int32_t* cand_col,
                            hipStream_t s) {
  const int64_t max_vis = (q_pos0 + rows) / 4;
  const int cpr = static_cast<int>((max_vis + kRegChunkCols - 1) / kRegChunkCols);
  RegArgs a1 = reg_args(scores, rows, stride, q_pos0, topk, nullptr);
  a1.cpr = cpr;
  a1.cand_score = cand_score;
  a1.cand_col = cand_col;
  hipError_t e = launch_reg<kRegChunk>(a1, kRegChunkCols, s);
  if (e != hipSuccess) return e;
  const int n2 = cpr * topk;
  const bool in_place = cand_score == nullptr;
  RegArgs a2 = reg_args(in_place ? scores : cand_score, rows, in_place ? stride : n2, q_pos0,
                        topk, out_idx);
  a2.n2 = n2;
  a2.cstride = in_place ? kRegChunkCols : topk;
  a2.col_base = in_place ? reinterpret_cast<const int32_t*>(scores) + topk : cand_col;
  a2.col_stride = in_place ? stride : n2;
  a2.kmagic = static_cast<uint32_t>((uint64_t(1) << 32) / static_cast<uint64_t>(topk) + 1);
  return launch_reg<kRegMerge>(a2, n2, s);
}

template <int CPT, int PER>
hipError_t launch_cpt(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                      int32_t topk, int32_t* out_idx, int64_t fixed_n, const int32_t* remap,
                      hipStream_t s) {
  const bool dma = (stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  const int64_t max_vis = fixed_n >= 0 ? fixed_n : (q_pos0 + rows) / 4;
  const int64_t chunk = static_cast<int64_t>(PER) * kThreads;
  const int chunks = static_cast<int>((max_vis + chunk - 1) / chunk);
  const int64_t G = rows < 256 ? rows : 256;  // one persistent workgroup per CU
  const int cpr = chunks > 0 ? chunks : 1;
  if (remap) {  // merge pass: rows of candidate lists (no DMA: any stride)
    hipLaunchKernelGGL((topk_kernel<CPT, PER, false, kMerge>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk, cpr, out_idx,
                       fixed_n, remap, nullptr);
  } else if (dma) {
    hipLaunchKernelGGL((topk_kernel<CPT, PER, true, kRows>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk, cpr, out_idx,
                       int64_t(-1), nullptr, nullptr);
  } else {
    hipLaunchKernelGGL((topk_kernel<CPT, PER, false, kRows>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk, cpr, out_idx,
                       int64_t(-1), nullptr, nullptr);
  }
  return hipGetLastError();
}

// Per-row top-k with the variant that fits the longest row: a single chunk,
// or a tournament over chunks with the running top-k in LDS.
hipError_t launch_rows(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                       int32_t topk, int32_t* out_idx, int64_t fixed_n, const int32_t* remap,
                       hipStream_t s) {
  const int64_t max_vis = fixed_n >= 0 ? fixed_n : (q_pos0 + rows) / 4;
  if (max_vis <= kSplitChunk)
    return launch_cpt<0, 32>(scores, rows, stride, q_pos0, topk, out_idx, fixed_n, remap, s);
  if (topk <= 2048)
    return launch_cpt<2, 32>(scores, rows, stride, q_pos0, topk, out_idx, fixed_n, remap, s);
  return launch_cpt<4, 24>(scores, rows, stride, q_pos0, topk, out_idx, fixed_n, remap, s);
}

}  // namespace

hipError_t dsv4_launch_topk(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                            int32_t topk, int32_t* out_idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const bool aligned = (stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  const int64_t max_vis = (q_pos0 + rows) / 4;
  if (aligned && max_vis <= kRegMaxVis)
    return launch_reg<kRegRows>(reg_args(scores, rows, stride, q_pos0, topk, out_idx), max_vis, s);
  return launch_rows(scores, rows, stride, q_pos0, topk, out_idx, -1, nullptr, s);
}

int64_t dsv4_topk_split_chunks(int64_t rows, int64_t q_pos0) {
  const int64_t max_vis = (q_pos0 + rows) / 4;
  return (max_vis + kSplitChunk - 1) / kSplitChunk;
}

hipError_t dsv4_launch_topk_split(const float* scores, int64_t rows, int64_t stride,
                                  int64_t q_pos0, int32_t topk, int32_t* out_idx,
                                  int32_t* cand_idx, float* cand_score, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t cpr = dsv4_topk_split_chunks(rows, q_pos0);
  if (cpr < 1 || cpr * topk > (int64_t(1) << 30)) return hipErrorInvalidValue;
  static_assert(kSplitChunk == kRegChunkCols, "both two-pass top-k use the same chunks");
  if (reg_split_ok(scores, rows, stride, q_pos0, topk, false))
    return launch_reg_split(scores, rows, stride, q_pos0, topk, out_idx, cand_score, cand_idx, s);
  // pass 1: every (row, chunk) item on its own, as many workgroups as items
  // (at most one per CU, persistent)
  const int64_t items = rows * cpr;
  const int64_t G = items < 256 ? items : 256;
  const bool dma = (stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (dma)
    hipLaunchKernelGGL((topk_kernel<0, 32, true, kSplit>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk,
                       static_cast<int>(cpr), cand_idx, int64_t(-1), nullptr, cand_score);
  else
    hipLaunchKernelGGL((topk_kernel<0, 32, false, kSplit>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk,
                       static_cast<int>(cpr), cand_idx, int64_t(-1), nullptr, cand_score);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass 2: top-k of each row's cpr * topk candidates, mapped back to columns
  const int64_t n2 = cpr * topk;
  return launch_rows(cand_score, rows, n2, q_pos0, topk, out_idx, n2, cand_idx, s);
}

bool dsv4_topk_inplace_applies(const float* scores, int64_t rows, int64_t stride,
                               int64_t q_pos0, int32_t topk) {
  return reg_split_ok(scores, rows, stride, q_pos0, topk, true);
}

hipError_t dsv4_launch_topk_inplace(float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                                    int32_t topk, int32_t* out_idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!reg_split_ok(scores, rows, stride, q_pos0, topk, true)) return hipErrorInvalidValue;
  return launch_reg_split(scores, rows, stride, q_pos0, topk, out_idx, nullptr, nullptr, s);
}
