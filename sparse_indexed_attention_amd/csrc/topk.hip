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
// HBM-bound: every visible score is read once.  Design:
//   * Persistent workgroups (one per CU, 16 waves) walk a list of work items,
//     an item being a row or, for rows longer than one chunk, a chunk of a
//     row.  The next item is copied from HBM into an LDS row buffer with
//     global_load_lds_dwordx4 while the current item is processed, so HBM
//     reads overlap all the compute below.  Thread t holds columns
//     [PER*t, PER*t + PER) of the item in registers as order-preserving 32-bit
//     keys.
//   * MSB-first radix select with 11-bit digits starting at the highest bit
//     in which the item's max and min keys differ (all keys share the bits
//     above it); one LDS histogram (2,048 bins) per pass gives the exact
//     threshold key T and the number of T-valued keys still needed.
//   * Ordered emission: each thread counts its keys > T and == T, one block
//     scan turns the counts into offsets, and each chosen key lands at
//     (#greater before it) + min(#equal before it, needed equal): ascending
//     output, ties to the lower column.
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

template <typename F>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, F op) {
  for (int off = 32; off > 0; off >>= 1)
    v = op(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}

// Exclusive scan over the workgroup in thread order; `scr` holds kWaves
// entries.  *total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scr,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), off));
    if (lane >= off) incl += y;
  }
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

// Work item `it` of workgroup g: rows g, g + G, ...; chunks of a row in order.
template <int kChunk>
__device__ __forceinline__ bool item_of(int64_t it, int64_t rows, int64_t q_pos0, int64_t g,
                                        int64_t G, int chunks_per_row, Item* o) {
  const int64_t r_local = it / chunks_per_row;
  const int ch = static_cast<int>(it - r_local * chunks_per_row);
  const int64_t row = g + r_local * G;
  if (row >= rows) return false;
  const int64_t vis = visible_rows(q_pos0 + row);
  const int64_t base = static_cast<int64_t>(ch) * kChunk;
  o->row = row;
  o->base = base;
  int64_t n = vis - base;
  if (n > kChunk) n = kChunk;
  if (n < 0) n = 0;
  o->n = static_cast<int>(n);
  o->first = ch == 0;
  o->last = (ch == chunks_per_row - 1) || (base + kChunk >= vis);
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

// Copy the whole 16-byte chunks of item columns [0, n) to LDS `buf` in the
// chunk_slot order (the tail of fewer than 4 columns is read from global
// memory later).  Wave w issues the 1 KiB blocks w, w + 16, ...; lane L of
// block i writes slot 64i + L and fetches the chunk that maps there; a lane
// whose chunk lies past the last whole chunk re-reads the block's first chunk
// (always valid) and its bytes are never used.
__device__ __forceinline__ void issue_item(const float* src, int n, float* buf) {
  const int n4 = n & ~3;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = wave; i * 256 < n4; i += kWaves) {
    const int a = ((lane >> 3) & 7) ^ (i & 1);
    const int lp = 8 * a + ((lane & 7) ^ a);
    const int e = i * 256 + 4 * lp;
    global_to_lds16(src + (e + 4 <= n4 ? e : i * 256), buf + i * 256);
  }
}

// PER: columns per thread (chunk = PER * 1,024 columns).  DMA: rows start on
// 16-byte boundaries, so items are copied with LDS DMA ahead of their use;
// otherwise each item is loaded synchronously.
template <int CPT, int PER, bool DMA>
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ scores, int64_t rows, int64_t stride, int64_t q_pos0,
            int topk, int chunks_per_row, int32_t* __restrict__ out_idx) {
  constexpr int KMAX = CPT > 0 ? CPT * kThreads : 1;
  constexpr int kPer = PER;
  constexpr int kChunk = PER * kThreads;
  __shared__ __attribute__((aligned(16))) float rowbuf[kChunk];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scr[4][kWaves];
  __shared__ uint32_t s_red[2][kWaves];
  __shared__ uint32_t s_bin, s_cum;
  __shared__ uint32_t ckey[KMAX];
  __shared__ int32_t cidx[KMAX];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t g = blockIdx.x, G = gridDim.x;

  uint32_t key[kPer];
  Item cur, nx;
  int64_t it = 0;
  if (!item_of<kChunk>(it, rows, q_pos0, g, G, chunks_per_row, &cur)) return;
  if (DMA) issue_item(scores + cur.row * stride + cur.base, cur.n, rowbuf);
  int c = 0;  // carry entries of the current row

  while (true) {
    if (!DMA) {
      const float* src = scores + cur.row * stride + cur.base;
      for (int e = tid; e < cur.n; e += kThreads) rowbuf[e] = src[e];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of the item landed
    __syncthreads();                       // ... and every other wave's
    {
      // keys; 0 marks a column past the item's end (no float maps to key 0)
      const float* src = scores + cur.row * stride + cur.base;
      const int n4 = DMA ? (cur.n & ~3) : cur.n;
      const int e0 = tid * kPer;
      if (e0 + kPer <= n4) {
#pragma unroll
        for (int v = 0; v < kPer / 4; ++v) {
          const int slot = DMA ? chunk_slot((e0 >> 2) + v) : (e0 >> 2) + v;
          const float4 x = *reinterpret_cast<const float4*>(&rowbuf[4 * slot]);
          key[4 * v] = float_key(x.x);
          key[4 * v + 1] = float_key(x.y);
          key[4 * v + 2] = float_key(x.z);
          key[4 * v + 3] = float_key(x.w);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int e = e0 + j;
          const int at = DMA ? 4 * chunk_slot(e >> 2) + (e & 3) : e;
          const float f = (e < n4) ? rowbuf[at] : ((e < cur.n) ? src[e] : 0.f);
          key[j] = (e < cur.n) ? float_key(f) : 0u;
        }
      }
    }
    const bool have_next = item_of<kChunk>(it + 1, rows, q_pos0, g, G, chunks_per_row, &nx);
    __syncthreads();  // every thread has its keys: the row buffer takes the next item
    if (DMA && have_next) issue_item(scores + nx.row * stride + nx.base, nx.n, rowbuf);
    if (cur.first) c = 0;
    // chunk slots past a shorter row's end carry no work (uniform branch)
    if (!cur.first && cur.n == 0) {
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

    if (need < E) {
      uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        kmax = max(kmax, key[j]);
        kmin = min(kmin, key[j] ? key[j] : 0xffffffffu);
      }
#pragma unroll
      for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
        if (j < cv) { kmax = max(kmax, ck[j]); kmin = min(kmin, ck[j]); }
      kmax = wave_reduce(kmax, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
      kmin = wave_reduce(kmin, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
      if (lane == 0) { s_red[0][wave] = kmax; s_red[1][wave] = kmin; }
      __syncthreads();
      uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) { mx = max(mx, s_red[0][w]); mn = min(mn, s_red[1][w]); }

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
      while (shift > 0) {
        const int dbits = shift < 11 ? shift : 11;
        shift -= dbits;
        const uint32_t dmask = (1u << dbits) - 1u;
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
#pragma unroll
        for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j)
          if (j < cv && (ck[j] & mask) == prefix) atomicAdd(&hist[(ck[j] >> shift) & dmask], 1u);
        __syncthreads();
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
          uint32_t incl = own;
          for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(incl), off));
            if (lane + off < 64) incl += y;
          }
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
          }
        }
        __syncthreads();
        remaining -= s_cum;
        prefix |= s_bin << shift;
        mask |= dmask << shift;
      }
      T = prefix;
      need_eq = remaining;
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
    const uint32_t k_gt = __popc(gtm), k_eq = __popc(eqm);
    uint32_t tot_cgt = 0, tot_ceq = 0, tot_kgt, tot_keq;
    uint32_t cgt_b = 0, ceq_b = 0;
    if (CPT > 0) {
      cgt_b = block_exclusive_scan(c_gt, scr[0], &tot_cgt);
      ceq_b = block_exclusive_scan(c_eq, scr[1], &tot_ceq);
    }
    const uint32_t kgt_b = block_exclusive_scan(k_gt, scr[2], &tot_kgt) + tot_cgt;
    const uint32_t keq_b = block_exclusive_scan(k_eq, scr[3], &tot_keq) + tot_ceq;
    int32_t* dst = out_idx + cur.row * static_cast<int64_t>(topk);
    const bool to_out = (CPT == 0) || cur.last;
    if (CPT > 0) {
      // carry entries (at most CPT per thread)
      uint32_t gtb = cgt_b, eqb = ceq_b;
#pragma unroll
      for (int j = 0; j < (CPT > 0 ? CPT : 0); ++j) {
        if (j < cv) {
          const bool gt = ck[j] > T, eq = ck[j] == T;
          if (gt || (eq && eqb < need_eq)) {
            const uint32_t pos = gtb + (eqb < need_eq ? eqb : need_eq);
            if (to_out) dst[pos] = ci[j];
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
          dst[kgt_b + __popc(gtm & low) + (eqb < need_eq ? eqb : need_eq)] = col0 + j;
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
    if (cur.last) {
      const int64_t vis = visible_rows(q_pos0 + cur.row);
      const int64_t k_total = vis < topk ? vis : topk;
      for (int64_t j = k_total + tid; j < topk; j += kThreads) dst[j] = -1;
    }
    __syncthreads();  // LDS tables / carry reused by the next item
    if (!have_next) break;
    cur = nx;
    ++it;
  }
}

template <int CPT, int PER>
hipError_t launch_cpt(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                      int32_t topk, int32_t* out_idx, hipStream_t s) {
  const bool dma = (stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  const int64_t max_vis = (q_pos0 + rows) / 4;
  const int64_t chunk = static_cast<int64_t>(PER) * kThreads;
  const int chunks = static_cast<int>((max_vis + chunk - 1) / chunk);
  const int64_t G = rows < 256 ? rows : 256;  // one persistent workgroup per CU
  const int cpr = chunks > 0 ? chunks : 1;
  if (dma)
    hipLaunchKernelGGL((topk_kernel<CPT, PER, true>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk, cpr, out_idx);
  else
    hipLaunchKernelGGL((topk_kernel<CPT, PER, false>), dim3(static_cast<unsigned>(G)),
                       dim3(kThreads), 0, s, scores, rows, stride, q_pos0, topk, cpr, out_idx);
  return hipGetLastError();
}

}  // namespace

hipError_t dsv4_launch_topk(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                            int32_t topk, int32_t* out_idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t max_vis = (q_pos0 + rows) / 4;
  if (max_vis <= 32 * kThreads) return launch_cpt<0, 32>(scores, rows, stride, q_pos0, topk, out_idx, s);
  if (topk <= 2048) return launch_cpt<2, 32>(scores, rows, stride, q_pos0, topk, out_idx, s);
  return launch_cpt<4, 24>(scores, rows, stride, q_pos0, topk, out_idx, s);
}
