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
// One workgroup (16 waves) per row.  The row's scores are read from HBM once,
// turned into order-preserving 32-bit keys and held in LDS; everything else
// runs out of LDS:
//   1. max / min key of the row (during the load);
//   2. MSB-first radix select, 8-bit digits, starting at the highest bit in
//      which max and min differ (all keys share the bits above it), with an
//      LDS histogram per pass -> exact threshold key T and the number of keys
//      equal to T that are still needed;
//   3. ordered emission: each wave owns a contiguous segment; a first sweep
//      counts keys > T and == T per wave, the per-wave counts are scanned, and
//      a second sweep places every chosen column at
//      (#greater before it) + min(#equal before it, needed equal) using wave
//      ballots, so the output is ascending and ties go to the lower column.
// Rows longer than the LDS chunk (1M-token contexts) are processed as a
// tournament: the running top-k (keys and columns, at most k entries, in
// ascending column order) is kept in LDS and merged with each next chunk; the
// top-k of (carry ++ chunk) under the same total order is the top-k of
// everything seen so far.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

template <int CH, int KMAX, bool MULTI>
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ scores, int64_t stride, int64_t q_pos0, int topk,
            int32_t* __restrict__ out_idx, int vec4) {
  __shared__ uint32_t keys[CH];
  __shared__ uint32_t ckey[MULTI ? 2 : 1][MULTI ? KMAX : 1];
  __shared__ int32_t cidx[MULTI ? 2 : 1][MULTI ? KMAX : 1];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wcnt[kWaves][2];
  __shared__ uint32_t s_max, s_min, s_bin, s_cum;

  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t vis = visible_rows(q_pos0 + row);
  const float* src = scores + row * stride;
  int32_t* dst = out_idx + row * (int64_t)topk;
  const int64_t k_total = vis < topk ? vis : topk;

  int c = 0;    // carry entries (MULTI only)
  int cur = 0;  // carry buffer holding them
  for (int64_t base = 0; base < vis; base += CH) {
    const int n = static_cast<int>((vis - base) < CH ? (vis - base) : CH);
    const bool last = base + n >= vis;
    const int E = c + n;
    const int need = E < topk ? E : topk;

    // ---- load chunk as keys, track max/min
    if (tid == 0) { s_max = 0u; s_min = 0xffffffffu; }
    __syncthreads();
    uint32_t kmax = 0u, kmin = 0xffffffffu;
    const float* cs = src + base;
    int done = 0;
    if (vec4) {
      const int n4 = n >> 2;
      for (int i = tid; i < n4; i += kThreads) {
        const float4 v = reinterpret_cast<const float4*>(cs)[i];
        const uint32_t a = float_key(v.x), b = float_key(v.y), cc = float_key(v.z), d = float_key(v.w);
        *reinterpret_cast<u32x4_t*>(&keys[4 * i]) = u32x4_t{a, b, cc, d};
        kmax = max(max(kmax, max(a, b)), max(cc, d));
        kmin = min(min(kmin, min(a, b)), min(cc, d));
      }
      done = n4 << 2;
    }
    for (int i = done + tid; i < n; i += kThreads) {
      const uint32_t a = float_key(cs[i]);
      keys[i] = a;
      kmax = max(kmax, a);
      kmin = min(kmin, a);
    }
    if (MULTI) {
      for (int i = tid; i < c; i += kThreads) {
        const uint32_t a = ckey[cur][i];
        kmax = max(kmax, a);
        kmin = min(kmin, a);
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), off)));
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), off)));
    }
    if (lane == 0) {
      atomicMax(&s_max, kmax);
      atomicMin(&s_min, kmin);
    }
    __syncthreads();

    auto key_at = [&](int e) -> uint32_t {
      if (MULTI) return e < c ? ckey[cur][e] : keys[e - c];
      return keys[e];
    };
    auto idx_at = [&](int e) -> int32_t {
      if (MULTI) return e < c ? cidx[cur][e] : static_cast<int32_t>(base + (e - c));
      return static_cast<int32_t>(base + e);
    };

    // ---- threshold key T and number of T-keys still needed
    uint32_t T = 0u;
    uint32_t need_eq = 0u;
    if (need < E) {
      const uint32_t mx = s_max, mn = s_min;
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
        const int dbits = shift < 8 ? shift : 8;
        shift -= dbits;
        const uint32_t dmask = (1u << dbits) - 1u;
        for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) {
          const uint32_t k = key_at(e);
          if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
          // lane l owns bins 4l..4l+3; inclusive suffix sums over lanes
          const u32x4_t h = *reinterpret_cast<const u32x4_t*>(&hist[4 * lane]);
          const uint32_t own = h[0] + h[1] + h[2] + h[3];
          uint32_t incl = own;
          for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(incl), off));
            if (lane + off < 64) incl += y;
          }
          const uint32_t above = incl - own;
          const bool hit = above < remaining && remaining <= incl;
          if (hit) {
            uint32_t cum = above;
            int b = 4 * lane + 3;
            for (; b > 4 * lane; --b) {
              if (cum + h[b - 4 * lane] >= remaining) break;
              cum += h[b - 4 * lane];
            }
            s_bin = static_cast<uint32_t>(b);
            s_cum = cum;
          }
        }
        __syncthreads();
        remaining -= s_cum;
        prefix |= s_bin << shift;
        mask |= dmask << shift;
        __syncthreads();  // s_bin / s_cum / hist reused by the next pass
      }
      T = prefix;
      need_eq = remaining;
    }

    // ---- ordered emission
    const int seg = ((E + kWaves - 1) / kWaves + 63) & ~63;
    const int e_begin = wave * seg;
    const int e_end = min(E, e_begin + seg);
    uint32_t n_gt = 0, n_eq = 0;
    for (int e0 = e_begin; e0 < e_end; e0 += 64) {
      const int e = e0 + lane;
      const bool v = e < e_end;
      const uint32_t k = v ? key_at(e) : 0u;
      n_gt += __popcll(__ballot(v && k > T));
      n_eq += __popcll(__ballot(v && k == T));
    }
    if (lane == 0) { wcnt[wave][0] = n_gt; wcnt[wave][1] = n_eq; }
    __syncthreads();
    uint32_t gt_off = 0, eq_off = 0;
    for (int w2 = 0; w2 < wave; ++w2) { gt_off += wcnt[w2][0]; eq_off += wcnt[w2][1]; }
    const int nb = cur ^ 1;
    for (int e0 = e_begin; e0 < e_end; e0 += 64) {
      const int e = e0 + lane;
      const bool v = e < e_end;
      const uint32_t k = v ? key_at(e) : 0u;
      const bool gt = v && k > T;
      const bool eq = v && k == T;
      const uint64_t gm = __ballot(gt);
      const uint64_t em = __ballot(eq);
      const uint32_t gtb = gt_off + lanes_below(gm);
      const uint32_t eqb = eq_off + lanes_below(em);
      if (gt || (eq && eqb < need_eq)) {
        const uint32_t pos = gtb + (eqb < need_eq ? eqb : need_eq);
        const int32_t id = idx_at(e);
        if (!MULTI || last) {
          dst[pos] = id;
        } else {
          ckey[nb][pos] = k;
          cidx[nb][pos] = id;
        }
      }
      gt_off += __popcll(gm);
      eq_off += __popcll(em);
    }
    __syncthreads();  // carry / keys / wcnt reuse by the next chunk
    c = need;
    cur = nb;
  }
  for (int64_t j = k_total + tid; j < topk; j += kThreads) dst[j] = -1;
}

// Largest row held in LDS in one piece: 36,864 keys (144 KiB).
constexpr int kChunkSingle = 36864;
// Tournament chunk sizes leave room for two carry buffers of k entries.
constexpr int kChunkMulti2k = 28672;  // k <= 2048: 112 KiB + 32 KiB
constexpr int kChunkMulti4k = 20480;  // k <= 4096: 80 KiB + 64 KiB

}  // namespace

hipError_t dsv4_launch_topk(const float* scores, int64_t rows, int64_t stride, int64_t q_pos0,
                            int32_t topk, int32_t* out_idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t max_vis = (q_pos0 + rows) / 4;
  const int vec4 = ((stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0;
  const dim3 grid(static_cast<unsigned>(rows)), block(kThreads);
  if (max_vis <= kChunkSingle) {
    hipLaunchKernelGGL((topk_kernel<kChunkSingle, 1, false>), grid, block, 0, s, scores, stride,
                       q_pos0, topk, out_idx, vec4);
  } else if (topk <= 2048) {
    hipLaunchKernelGGL((topk_kernel<kChunkMulti2k, 2048, true>), grid, block, 0, s, scores,
                       stride, q_pos0, topk, out_idx, vec4);
  } else {
    hipLaunchKernelGGL((topk_kernel<kChunkMulti4k, 4096, true>), grid, block, 0, s, scores,
                       stride, q_pos0, topk, out_idx, vec4);
  }
  return hipGetLastError();
}
