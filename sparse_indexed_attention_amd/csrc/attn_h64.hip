// Fused windowed + pooled sparse prefill attention at the hot shape, H = 64
// heads, D = 512 dims, bf16 MFMA on gfx950.
//
// [P2 "perf(deepseek_v4): faster exact DeepSeek-V4 prefill", commit 1: one
// attention over the sliding raw-token window plus the pooled rows, B=1,
// H=64, D=512, bf16, masks rebuilt from offsets; P3 "[Discussion] Tile
// indexed-attention scoring ...", Possible design step 4.]
//
// Same definition, arguments and key walk as sparse_attn_kernel (one
// workgroup per query, 32-key tiles gathered straight into LDS, key slots
// masked from positions), with a work split chosen for this shape.  With 8
// waves:
//   * QK^T: wave w = hq + 4 kh computes S^T (16 keys x 16 heads) for key half
//     kh and head tile hq over all 512 dims -- its Q block (16 heads x 512
//     dims, 64 VGPRs) stays in registers, so the scores need no exchange
//     between waves; the wave then owns that (head tile, key half) for the
//     online softmax and writes P (bf16) to an LDS tile [head][key];
//   * P.V: wave w accumulates O for all 64 heads x dims 64w .. 64w+63
//     (64 VGPRs): every transposed V read (ds_read_b64_tr_b16, half the bytes
//     per clock of ds_read_b128) feeds four MFMAs (64 heads);
//   * per 32-key tile, each CU reads 128 KiB of K, 32 KiB of V and 32 KiB of
//     P from LDS.
// Softmax: online, fp32, exp2 with the scale folded in, against a per-head
// reference max that moves lazily.  Each owner computes P against the
// current reference and flags its heads whose tile max passes it by more
// than 2^8; the flags cross the next barrier, and only on a flagged tile
// (the first tile of every query, and rare jumps) do the owners move the
// reference, rewrite that tile's P and publish the rescale factors, which
// costs one more barrier.  Otherwise p <= 2^8.
// Pipeline, one barrier per tile over four LDS stages: P, the tile maxima
// and the flags are double-buffered by tile parity, so after the barrier of
// tile t a wave runs QK(t), P.V(t-1) and softmax(t) with no barrier between
// them, while the gathers of tiles t+1 and t+2 are in flight.  QK comes
// first so that P.V's MFMAs, not a stall, separate its last MFMA from the
// softmax's first read of its result.
#include <type_traits>

#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kD = 512;
constexpr int kH = 64;
constexpr int kKeys = 32;
constexpr int kStages = 4;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int kTileElems = kKeys * kD;
constexpr int kPStride = 40;          // bf16 per P row: 32 keys + 8 pad (80 B: conflict-free b128)
constexpr float kSlack = 8.f;         // lazy max slack, log2 units
constexpr int kInstsPerWave = kKeys / kNW;  // gather instructions per wave per tile (one row each)

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// 16-byte chunk c of tile row r sits at slot c ^ swz(r): r's low 4 bits
// rotated right by one, a bijection that keeps both the K fragment reads
// (16 rows, one chunk) and the transposed V reads conflict-free.
__device__ __forceinline__ int swz(int r) { return ((r & 1) << 3) | ((r >> 1) & 7); }

// max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows).
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__global__ void __launch_bounds__(kNT)
attn_h64_kernel(const uint16_t* __restrict__ q, int64_t q_pos0, float scale_log2,
                const uint16_t* __restrict__ raw, int64_t raw_pos0, int window,
                const uint16_t* __restrict__ pooled, int ratio,
                const int32_t* __restrict__ sel, int topk, uint16_t* __restrict__ out,
                int nsplit, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kStages][kTileElems];
  // P of even and of odd tiles: two arrays, so the compiler knows that the
  // P.V reads of one never alias the softmax's stores to the other
  __shared__ __attribute__((aligned(16))) uint16_t pbuf0[kH * kPStride];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf1[kH * kPStride];
  __shared__ float s_mx[2][2][kH];   // by tile parity, per key half: the tile max (log2 units)
  __shared__ __attribute__((aligned(16))) float s_alpha[kH];  // rescale factors of a flagged tile
  __shared__ float s_l[2][kH];       // per key half: the owner's row sum
  __shared__ int s_flag[2][kNW];     // by tile parity
  __shared__ int s_lastw[kNW];  // per wave: its last visible selection slot
  extern __shared__ int s_sel[];     // the query's selection row (topk ints)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = lane >> 4;
  const int l16 = lane & 15;
  // QK / softmax role
  const int hq = wave & 3;         // head tile: heads 16 hq .. 16 hq + 15
  const int kh = wave >> 2;        // key half of the tile: keys 16 kh .. 16 kh + 15
  const int own_head = 16 * hq + l16;
  // P.V role: dims 64 wave .. 64 wave + 63 of all heads

  int64_t t;
  {
    const int64_t nq = gridDim.x, full = nq / 8, rem = nq % 8;
    const int64_t x = blockIdx.x % 8, r = blockIdx.x / 8;
    t = x * full + (x < rem ? x : rem) + r;
  }
  const int split = blockIdx.y;
  const int64_t p = q_pos0 + t;
  const int64_t lo = (p - window + 1) > 0 ? (p - window + 1) : 0;
  const int n_win = static_cast<int>(p - lo + 1);
  const int64_t vis = visible_rows(p, ratio);
  const uint16_t* self_row = raw + (p - raw_pos0) * kD;

  // ---- Q block: B operand of S^T = K.Q^T.  Lane group kb holds dims
  // 128 kb .. 128 kb + 127 over the 16 steps (the contraction order is the
  // same permutation for K below).
  bf16x8_t qf[16];
  {
    const uint16_t* qp = q + ((t * kH + own_head) * (int64_t)kD + 128 * kb);
#pragma unroll
    for (int j = 0; j < 16; ++j) qf[j] = *reinterpret_cast<const bf16x8_t*>(qp + 8 * j);
  }

  int n_slots;
  if (sel) {
    // the selection row straight into LDS, 64 slots per wave instruction,
    // in flight with the Q loads
    const int32_t* sp = sel + t * topk;
    for (int c = wave; c * 64 < topk; c += kNW) {
      const int j = c * 64 + lane;
      if (j < topk) global_to_lds4(sp + j, &s_sel[c * 64]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // trailing slots that name no visible row are dropped: the last
    // visible slot of this wave's share, then the largest over the waves
    int last = -1;
    for (int i = 0; i * kNT < topk; ++i) {
      const int j = i * kNT + tid;
      bool v = false;
      if (j < topk) {
        const int32_t s = s_sel[j];
        v = s >= 0 && s < vis;
      }
      const uint64_t b = __ballot(v);
      if (b) last = i * kNT + wave * 64 + 63 - __builtin_clzll(b);
    }
    s_lastw[wave] = last;  // wave-uniform
    __syncthreads();
    last = s_lastw[0];
#pragma unroll
    for (int w = 1; w < kNW; ++w) last = max(last, s_lastw[w]);
    n_slots = last + 1;
  } else {
    n_slots = static_cast<int>(vis);
  }
  const int n_keys = n_win + n_slots;
  const int n_tiles_all = (n_keys + kKeys - 1) / kKeys;
  const int tile_lo = static_cast<int>((static_cast<int64_t>(split) * n_tiles_all) / nsplit);
  const int n_tiles =
      static_cast<int>((static_cast<int64_t>(split + 1) * n_tiles_all) / nsplit) - tile_lo;

  auto key_row = [&](int j) -> const uint16_t* {
    if (j < n_win) return raw + (lo + j - raw_pos0) * kD;
    if (j < n_keys) {
      const int sl = j - n_win;
      const int64_t s = sel ? static_cast<int64_t>(s_sel[sl]) : sl;
      if (s >= 0 && s < vis) return pooled + s * kD;
    }
    return nullptr;
  };
  // Row lookup of two tiles at once: lane k < 32 finds key slot k of
  // `tile`, lane 32 + k slot k of tile + 1; the ballot's low and high words
  // are the two tiles' validity masks (bit k: slot k has a row).
  struct Look {
    uint32_t lo, hi;
    uint64_t valid;
  };
  auto lookup = [&](int tile) -> Look {
    const uint16_t* rk = key_row(tile * kKeys + lane);
    Look lk;
    lk.valid = __ballot(rk != nullptr);
    const uint64_t ra = reinterpret_cast<uint64_t>(rk ? rk : self_row);
    lk.lo = static_cast<uint32_t>(ra);
    lk.hi = static_cast<uint32_t>(ra >> 32);
    return lk;
  };
  // one whole 1 KiB row per wave instruction: rows wave, wave+8, +16, +24
  // of the lookup's tile `half` (0: its first tile, 1: the second)
  auto issue = [&](const Look& lk, int buf, int half, int u0, int u1) {
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int i = wave + kNW * u + kKeys * half;
      const uint64_t base =
          (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lk.hi), i))) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lk.lo), i));
      const int r = i & (kKeys - 1);
      const uint32_t off = static_cast<uint32_t>((lane ^ swz(r)) * 16);
      global_to_lds16_s(reinterpret_cast<const void*>(base), off, &tiles[buf][r * kD]);
    }
  };

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the selection are in

  f32x4_t o[4][4];  // [head tile][dim tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int n = 0; n < 4; ++n) o[a][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // owner: reference max of head own_head
  float l_part = 0.f;       // owner: row sum of its key half
  float sv[4];              // owner: the last tile's masked logits (log2 units)
  float psum = 0.f;         // owner: the last tile's row sum, not yet added
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = -INFINITY;

  // A-fragment rows: S^T row m of key half kh is tile key 16 kh + 4 (m % 4)
  // + m / 4, so the owner's four values (rows 4 kb + i) are keys
  // 16 kh + 4 i + kb: in P's column order (below) one 8-byte run.
  const int qk_row = 16 * kh + 4 * (l16 & 3) + (l16 >> 2);
  const int qk_swz = swz(qk_row);
  // P.V B-operand rows (transposed reads): keys 4 (l16 / 4) + kb and + 16
  const int trow0 = 4 * (l16 >> 2) + kb;
  const int trow1 = 16 + trow0;
  const int sw0 = swz(trow0), sw1 = swz(trow1);
  const int dsub = 4 * (l16 & 3);
  // P is stored [head][column], column 8 b + e holding key 4 e + b: the
  // k-element e of lane group b in the P.V A operand (whose B operand, read
  // transposed, holds keys 4 e + b), so each A fragment is one 16-byte read.

  // The swizzle terms pass through an empty asm at each use, so the compiler
  // forms the few swizzled LDS addresses of a tile when it needs them rather
  // than keeping some thirty of them live across the loop.
  auto opaque = [](int x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  auto qk = [&](auto stage) -> f32x4_t {
    const uint16_t* rb = tiles[decltype(stage)::value] + qk_row * kD;
    const int q_swz = opaque(qk_swz);
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int chunk = 16 * kb + j;
      const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(rb + ((chunk ^ q_swz) * 8));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, qf[j], acc, 0, 0, 0);
    }
    return acc;
  };

  auto pv = [&](auto stage, auto par) {
    const uint16_t* tb = tiles[decltype(stage)::value];
    const uint16_t* pb = decltype(par)::value ? pbuf1 : pbuf0;
    const int s0w = opaque(sw0), s1w = opaque(sw1);
    bf16x8_t pa[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      pa[a] = *reinterpret_cast<const bf16x8_t*>(&pb[(16 * a + l16) * kPStride + 8 * kb]);
    i16x4_t fv[2][2];
    auto ld = [&](int n, int bi) {
      const int d = 64 * wave + 16 * n + dsub;
      const int ch = d >> 3, off = d & 7;
      fv[bi][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tb + trow0 * kD + ((ch ^ s0w) * 8) + off));
      fv[bi][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tb + trow1 * kD + ((ch ^ s1w) * 8) + off));
    };
    ld(0, 0);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int bi = n & 1;
      if (n + 1 < 4) ld(n + 1, bi ^ 1);
      bf16x8_t b;
      *reinterpret_cast<i16x4_t*>(&b) = fv[bi][0];
      *(reinterpret_cast<i16x4_t*>(&b) + 1) = fv[bi][1];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        o[a][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[a], b, o[a][n], 0, 0, 0);
    }
  };

  // P values of the owner's four keys against reference m (m = -inf: 0)
  auto write_p = [&](float m, auto par) {
    const float mu = (m == -INFINITY) ? 0.f : m;
    float pr[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
      s += pr[i];
    }
    uint2 w;
    w.x = pack_bf16x2(pr[0], pr[1]);
    w.y = pack_bf16x2(pr[2], pr[3]);
    uint16_t* pw = decltype(par)::value ? pbuf1 : pbuf0;
    *reinterpret_cast<uint2*>(&pw[own_head * kPStride + 8 * kb + 4 * kh]) = w;
    psum = rows_sum(s);
  };

  if (n_tiles > 0) {
    Look lk = lookup(tile_lo);  // tiles 0 and 1
    issue(lk, 0, 0, 0, kInstsPerWave);
    uint32_t vm_cur = static_cast<uint32_t>(lk.valid), vm_next = 0u;
    if (n_tiles > 1) {
      issue(lk, 1, 1, 0, kInstsPerWave);
      vm_next = static_cast<uint32_t>(lk.valid >> 32);
    }
    if (n_tiles > 2) lk = lookup(tile_lo + 2);  // tiles 2 and 3
    // Iteration `it` (unrolled over the four stages, so every LDS address is
    // a lane base plus an immediate; `st` is it % kStages, and the parity
    // it % 2 of P, the tile maxima and the flags follows):
    //   wait for tile it's rows; the barrier (tile it, P(it-1), the maxima
    //   and flags of it-1; stage it-2 and the parity-it buffers are free);
    //   gather tile it+2; QK(it); settle the flags of it-1 (owners move
    //   references, rewrite P(it-1), publish factors; one more barrier,
    //   rare); then P.V(it-1) and softmax(it) -> P(it), which need no
    //   barrier between them.
    // `kind` 0 is the first tile (no P.V, no flags), 1 a middle tile
    // (1 <= it < n_tiles), 2 the final pass (it = n_tiles: P.V only); the
    // middle tiles carry no tile-count tests around QK, P.V and softmax, so
    // those are one basic block the compiler can interleave.
    auto step = [&](auto st, auto kind_c, int it) {
      constexpr int S = decltype(st)::value;
      constexpr int kind = decltype(kind_c)::value;
      constexpr bool has_qk = kind != 2, has_pv = kind != 0;
      constexpr int SP = (S + kStages - 1) % kStages;  // tile it-1
      constexpr int SN = (S + 2) % kStages;            // tile it+2
      constexpr int PAR = S & 1, PARP = PAR ^ 1;      // parity of tile it, of it-1
      if constexpr (has_qk) {
        // this wave's rows of tile `it` landed (tile it+1 may still fly)
        if (it + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0F70 | kInstsPerWave);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      __syncthreads();
      uint32_t vm_after = 0u;
      if (it + 2 < n_tiles) {
        // tile it+2 is the lookup's first tile when it is even, else its second
        issue(lk, SN, S & 1, 0, kInstsPerWave);
        vm_after = static_cast<uint32_t>(lk.valid >> (32 * (S & 1)));
        if ((S & 1) && it + 3 < n_tiles) lk = lookup(tile_lo + it + 3);
      }
      // QK(it) first: its MFMAs are done by the time the softmax reads them,
      // P.V(it-1) issuing in between
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (has_qk) sc = qk(std::integral_constant<int, S>{});
      if constexpr (has_pv) {
        // ---- flags of tile it-1: move the references where a tile max
        // passed them by more than the slack (uniform decision)
        int any = 0;
#pragma unroll
        for (int w = 0; w < kNW; ++w) any |= s_flag[PARP][w];
        if (__builtin_expect(any, 0)) {
          const float tmax = fmaxf(s_mx[PARP][0][own_head], s_mx[PARP][1][own_head]);
          const bool bump = tmax > m_ref + kSlack;
          const float m_new = bump ? tmax : m_ref;
          const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
          if (kh == 0 && kb == 0) s_alpha[own_head] = alpha;
          // heads without a bump rewrite the same P
          if (__ballot(bump)) write_p(m_new, std::integral_constant<int, PARP>{});
          psum = l_part * alpha + psum;
          l_part = 0.f;
          m_ref = m_new;
          __syncthreads();  // P(it-1) as settled, the factors
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4_t al = *reinterpret_cast<const f32x4_t*>(&s_alpha[16 * a + 4 * kb]);
#pragma unroll
            for (int n = 0; n < 4; ++n) o[a][n] *= al;
          }
        }
        l_part += psum;
        pv(std::integral_constant<int, SP>{}, std::integral_constant<int, PARP>{});
      }
      if constexpr (has_qk) {
        // ---- the softmax of the owned (head tile, key half):
        // rows 4 kb + i are keys 16 kh + 4 i + kb
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kh + 4 * i + kb;
          sv[i] = ((vm_cur >> key) & 1u) ? sc[i] * scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[i]);
        }
        mx = rows_max(mx);
        s_mx[PAR][kh][own_head] = mx;  // the four lanes of a head store the same value
        const bool flag = __ballot(mx > m_ref + kSlack) != 0;
        s_flag[PAR][wave] = flag ? 1 : 0;  // wave-uniform
        write_p(m_ref, std::integral_constant<int, PAR>{});
      }
      vm_cur = vm_next;
      vm_next = vm_after;
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    step(S0{}, K0{}, 0);
    int it = 1;
    for (; it + kStages <= n_tiles; it += kStages) {
      step(S1{}, K1{}, it);
      step(S2{}, K1{}, it + 1);
      step(S3{}, K1{}, it + 2);
      step(S0{}, K1{}, it + 3);
    }
    // it % 4 == 1 here, and at most three middle tiles are left
    if (it < n_tiles) step(S1{}, K1{}, it++);
    if (it < n_tiles) step(S2{}, K1{}, it++);
    if (it < n_tiles) step(S3{}, K1{}, it++);
    switch (it & 3) {  // it == n_tiles: the last tile's P.V
      case 0: step(S0{}, K2{}, it); break;
      case 1: step(S1{}, K2{}, it); break;
      case 2: step(S2{}, K2{}, it); break;
      default: step(S3{}, K2{}, it); break;
    }
  }

  // ---- row sums of the two key halves, then O normalised (or the split's
  // partial state)
  if (kb == 0) s_l[kh][own_head] = l_part;
  __syncthreads();  // also: every wave is done with the tile stages
  if (nsplit > 1) {
    float* po = part_o + ((t * nsplit + split) * kH) * static_cast<int64_t>(kD);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 16 * a + 4 * kb + i;
#pragma unroll
        for (int n = 0; n < 4; ++n) po[hh * static_cast<int64_t>(kD) + 64 * wave + 16 * n + l16] = o[a][n][i];
      }
    if (kh == 0 && kb == 0) {
      part_ml[((t * nsplit + split) * kH + own_head) * 2] = m_ref;
      part_ml[((t * nsplit + split) * kH + own_head) * 2 + 1] = s_l[0][own_head] + s_l[1][own_head];
    }
    return;
  }
  uint16_t* stage = &tiles[0][0] + wave * (kH * 64);  // this wave's 64 heads x 64 dims
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * a + 4 * kb + i;
      const float l = s_l[0][hh] + s_l[1][hh];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) stage[hh * 64 + 16 * n + l16] = bf16_rne(o[a][n][i] * inv);
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  // 64 heads x 8 chunks of 16 B per wave
#pragma unroll
  for (int c0 = 0; c0 < 8; ++c0) {
    const int c = c0 * 64 + lane;
    const int hh = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4_t*>(out + (t * kH + hh) * (int64_t)kD + 64 * wave + 8 * ch) =
        *reinterpret_cast<const u32x4_t*>(stage + hh * 64 + 8 * ch);
  }
}

}  // namespace

// Whether the kernel's LDS (static arrays + the selection row, topk ints)
// fits a workgroup's 160 KiB: up to k = 5,160 selected slots.
bool dsv4_attn_h64_fits(int32_t topk) {
  constexpr size_t kStatic = sizeof(uint16_t) * kStages * kTileElems   // tiles
                             + sizeof(uint16_t) * 2 * kH * kPStride   // pbuf0, pbuf1
                             + sizeof(float) * (4 * kH + kH + 2 * kH) // s_mx, s_alpha, s_l
                             + sizeof(int) * (3 * kNW);               // s_flag, s_lastw
  return kStatic + sizeof(int) * static_cast<size_t>(topk) <= 160 * 1024;
}

// Launch of the H = 64, D = 512 kernel (arguments as dsv4_launch_sparse_attn).
hipError_t dsv4_launch_sparse_attn_h64(const void* q, int64_t T, int64_t q_pos0, float scale_log2,
                                       const void* raw_kv, int64_t raw_pos0, int32_t window,
                                       const void* pooled, int32_t ratio, const int32_t* sel_idx,
                                       int32_t topk, void* out, int32_t nsplit, float* part_o,
                                       float* part_ml, hipStream_t s) {
  if (!dispatch_fits(T, kNT)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(nsplit));
  const size_t dyn = static_cast<size_t>(sel_idx ? topk : 0) * sizeof(int);
  hipLaunchKernelGGL(attn_h64_kernel, grid, dim3(kNT), dyn, s, static_cast<const uint16_t*>(q),
                     q_pos0, scale_log2, static_cast<const uint16_t*>(raw_kv), raw_pos0, window,
                     static_cast<const uint16_t*>(pooled), ratio, sel_idx, topk,
                     static_cast<uint16_t*>(out), nsplit, part_o, part_ml);
  return hipGetLastError();
}
