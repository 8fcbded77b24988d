// Fused windowed + pooled sparse prefill attention, bf16 MFMA on gfx950.
//
// [P2 "perf(deepseek_v4): faster exact DeepSeek-V4 prefill", commit 1: one
// attention over the sliding raw-token window plus the pooled rows (small-pool
// or indexer top-k), B=1, H=64, D=512, bf16, causality / window / pooled
// visibility rebuilt from offsets; P3 "[Discussion] Tile indexed-attention
// scoring ...", Possible design step 4: the selected rows feed the indexed
// mixed attention.]
//
// Per query p and head h, keys = raw rows p-window+1 .. p (clipped at 0) plus
// the pooled rows listed in the query's selection with 0 <= s < (p+1)/r
// (all of them when no selection is given); values are the keys (one KV row
// shared by all heads); out = softmax(scale * q.K) . K.  The pool's ratio r
// is 4 on the indexer path and 128 in the CompressedAttention mode; r = 0
// (no pool) is the window-only LocalAttention mode [P2 commit 1: the same
// kernel serves LocalAttention, CompressedAttention and
// SparseCompressedAttention].
//
// Mapping onto CDNA4:
//   * one workgroup per query; a wave owns 16 heads and one half of the head
//     dimension (8 waves at H = 64, D = 512), so its Q block (B operand) and
//     its O block (16 heads x D/2, fp32) stay in registers with room left for
//     two waves per SIMD, which hide each other's LDS latency;
//   * keys are gathered 32 at a time straight into LDS with
//     global_load_lds_dwordx4 (each wave instruction moves 64 x 16 B, one whole
//     1 KiB row at D = 512), three LDS stages deep: the gathers of tiles i+1
//     and i+2 are in flight while tile i is computed, and no VGPRs hold
//     in-flight data;
//   * 16-byte chunk c of row r sits at slot c ^ swz(r), swz rotating r's low
//     4 bits right by one, which keeps both LDS read patterns below free of
//     bank conflicts; each DMA instruction's row address is wave-uniform
//     (one lane looks it up per key), so it goes out in the saddr form;
//   * QK^T is computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_16x16x32_bf16, each wave over its half of the dims; the two
//     halves' partial tiles are summed through LDS (a + b == b + a, so both
//     waves hold bit-identical scores).  In S^T each lane holds 8 keys of one
//     head, exactly the A-operand layout PV needs (key order inside the
//     contraction is permuted the same way for P and V), so probabilities
//     never leave the lane;
//   * PV reads its B operand (4 keys x 16 dims per 16-lane block) from the same
//     row-major tile with ds_read_b64_tr_b16, which transposes in the LDS read
//     path; no second, transposed copy of the tile is written;
//   * online softmax in fp32 (exp2, scale folded in) against a lazily moved
//     reference max: O is rescaled only on tiles where some head's max passes
//     the reference by more than 2^8, keeping p <= 256 (exact math, rounding
//     of p to bf16 is scale-free);
//   * O is normalised, rounded to bf16 and staged through LDS once at the end
//     for 16-byte coalesced stores.
// Masked key slots (empty, invisible or past the end) are loaded from the
// query's own raw row so the tile never holds non-finite data, and their
// logits are set to -inf.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kKeys = 32;   // keys per LDS tile
constexpr int kStages = 3;  // LDS tile stages: two tiles in flight while one is computed

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;


// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// row-swap permutes: permlane16_swap of a value with itself pairs rows 0/1 and
// 2/3, permlane32_swap pairs the two halves; every lane ends with the result.
__device__ __forceinline__ float xor16_32_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xor16_32_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int NHG, int DSPLIT>
__global__ void __launch_bounds__(NHG * DSPLIT * 64)
sparse_attn_kernel(const uint16_t* __restrict__ q, int64_t q_pos0, int H, float scale_log2,
                   const uint16_t* __restrict__ raw, int64_t raw_pos0, int window,
                   const uint16_t* __restrict__ pooled, int ratio,
                   const int32_t* __restrict__ sel, int topk, uint16_t* __restrict__ out,
                   int nsplit, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int NW = NHG * DSPLIT;
  constexpr int NT = NW * 64;
  constexpr int DH = D / DSPLIT;          // dims per wave
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
  // LDS slot of 16-byte chunk c of tile row r is c ^ swz(r).  For 16+ chunks
  // per row swz rotates the row's low 4 bits right by one: still a bijection,
  // so the QK fragment reads (16 rows, one chunk) stay conflict-free, and the
  // PV tr16 reads of a 32-lane pass (rows 4m+kb for kb pairs {0,1} / {2,3}, two
  // adjacent chunks) now cover all 16 bank groups instead of 8 twice.
  auto swz = [](int r) -> int {
    if constexpr (SWZ == 15) return ((r & 1) << 3) | ((r >> 1) & 7);
    else return r & SWZ;
  };
  constexpr int RPI = 64 / CPR;           // rows per 64-lane load instruction
  constexpr int INSTS = kKeys / RPI;      // load instructions per tile
  constexpr int KSTEP = DH / 32;          // QK^T contraction steps per wave
  constexpr int NTILE = DH / 16;          // PV output column tiles per wave
  constexpr int TILE_ELEMS = kKeys * D;
  static_assert(RPI >= 1 && kKeys % RPI == 0 && KSTEP >= 1, "tile shape");
  // load instructions every wave issues per tile (waves may issue one more)
  constexpr int kNewer = INSTS / NW < 15 ? INSTS / NW : 15;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kStages][TILE_ELEMS];
  // partial S^T tiles of the two dim halves, double-buffered by tile parity
  __shared__ __attribute__((aligned(16))) float xs[DSPLIT > 1 ? 2 : 1][DSPLIT > 1 ? NW : 1][DSPLIT > 1 ? 64 * 8 : 1];
  __shared__ int s_last;
  extern __shared__ int s_sel[];  // the query's selection row (topk ints, dynamic)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: SGPR addressing
  const int hg = wave % NHG;   // head group
  const int dh = wave / NHG;   // dim half
  const int kb = lane >> 4;    // 16-lane group
  const int l16 = lane & 15;

  // XCD-contiguous queries: workgroup b runs on XCD b % 8, which takes the
  // (b % 8)-th eighth of the queries, so neighbours (whose selections and
  // windows overlap) share that XCD's L2.  A bijection for any gridDim.x.
  int64_t t;
  {
    const int64_t nq = gridDim.x, full = nq / 8, rem = nq % 8;
    const int64_t x = blockIdx.x % 8, r = blockIdx.x / 8;
    t = x * full + (x < rem ? x : rem) + r;
  }
  const int split = blockIdx.y;  // key split (nsplit > 1: partial results)
  const int64_t p = q_pos0 + t;
  const int64_t lo = (p - window + 1) > 0 ? (p - window + 1) : 0;
  const int n_win = static_cast<int>(p - lo + 1);
  const int64_t vis = visible_rows(p, ratio);
  const uint16_t* self_row = raw + (p - raw_pos0) * D;  // always valid

  // ---- Q block (B operand of S^T = K.Q^T): lane group kb holds dims
  // dh*DH + kb*DH/4 .. + DH/4 over the KSTEP steps.  Loaded first, so its
  // latency overlaps the selection row's.
  const int head = hg * 16 + l16;
  const bool hv = head < H;
  bf16x8_t qf[KSTEP];
  {
    const uint16_t* qp = q + ((t * H + head) * (int64_t)D + dh * DH + kb * (DH / 4));
#pragma unroll
    for (int j = 0; j < KSTEP; ++j)
      qf[j] = hv ? *reinterpret_cast<const bf16x8_t*>(qp + j * 8) : bf16x8_t{};
  }

  // ---- selection row into LDS; number of pooled slots to walk
  int n_slots;
  if (sel) {
    if (tid == 0) s_last = -1;
    __syncthreads();
    int last = -1;
    const int32_t* sp = sel + t * topk;
    for (int j = tid; j < topk; j += NT) {
      const int32_t s = sp[j];
      s_sel[j] = s;
      if (s >= 0 && s < vis) last = j;
    }
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
    if (lane == 0) atomicMax(&s_last, last);
    __syncthreads();
    n_slots = s_last + 1;
  } else {
    n_slots = static_cast<int>(vis);
  }
  const int n_keys = n_win + n_slots;
  const int n_tiles_all = (n_keys + kKeys - 1) / kKeys;
  // This workgroup's tiles: all of them, or split `split` of nsplit balanced
  // ranges (a range may be empty when there are fewer tiles than splits).
  const int tile_lo = static_cast<int>((static_cast<int64_t>(split) * n_tiles_all) / nsplit);
  const int n_tiles =
      static_cast<int>((static_cast<int64_t>(split + 1) * n_tiles_all) / nsplit) - tile_lo;

  auto key_row = [&](int j) -> const uint16_t* {  // row of key slot j, or nullptr
    if (j < n_win) return raw + (lo + j - raw_pos0) * D;
    if (j < n_keys) {
      const int sl = j - n_win;
      const int64_t s = sel ? static_cast<int64_t>(s_sel[sl]) : sl;
      if (s >= 0 && s < vis) return pooled + s * D;
    }
    return nullptr;
  };

  // Gather of a tile, in two parts so the row lookups can run an iteration
  // ahead of the DMA issue.  lookup(tile): lane k (< 32) finds key slot k's
  // row (the selection row in LDS, then the address); the ballot of found
  // rows is the tile's validity mask (bit k: key slot k has a row).
  struct Look {
    uint32_t lo, hi;  // lane k's row address (RPI == 1)
    uint32_t valid;
    int tile;
  };
  auto lookup = [&](int tile) -> Look {
    const uint16_t* rk = lane < kKeys ? key_row(tile * kKeys + lane) : nullptr;
    Look lk;
    lk.valid = static_cast<uint32_t>(__ballot(rk != nullptr));
    const uint64_t ra = reinterpret_cast<uint64_t>(rk ? rk : self_row);
    lk.lo = static_cast<uint32_t>(ra);
    lk.hi = static_cast<uint32_t>(ra >> 32);
    lk.tile = tile;
    return lk;
  };
  // issue(lk, buf): instruction i moves rows i*RPI .. i*RPI+RPI-1 into stage
  // `buf`.  With one row per instruction its address is wave-uniform: read
  // from the owning lane, sent in the saddr form with per-lane chunk offsets.
  auto issue = [&](const Look& lk, int buf) {
    if constexpr (RPI == 1) {
      for (int i = wave; i < INSTS; i += NW) {
        const uint64_t base =
            (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lk.hi), i))) << 32) |
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lk.lo), i));
        const uint32_t off = static_cast<uint32_t>(((lane % CPR) ^ swz(i)) * 16);
        global_to_lds16_s(reinterpret_cast<const void*>(base), off, &tiles[buf][i * D]);
      }
    } else {
      for (int i = wave; i < INSTS; i += NW) {
        const int row = i * RPI + lane / CPR;
        const int slot = lane % CPR;
        const uint16_t* rp = key_row(lk.tile * kKeys + row);
        if (!rp) rp = self_row;
        global_to_lds16(rp + (slot ^ swz(row)) * 8, &tiles[buf][i * RPI * D]);
      }
    }
  };

  // Drain the compiler's own loads (Q, selection) before the first LDS DMA is issued, so
  // the only vector-memory operations in flight inside the loop are the tile
  // gathers the loop accounts for.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  f32x4_t o[NTILE];
#pragma unroll
  for (int n = 0; n < NTILE; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // per head (this lane's head l16): reference max, log2 units
  float l_run = 0.f;
  constexpr float kSlack = 8.f;

  // key order inside a tile: M tile mt, row m -> key mt*16 + 4*(m%4) + m/4
  // (so the 4 keys one tr16 read covers are rows kb, kb+4, kb+8, kb+12)
  const int qk_row0 = 4 * (l16 & 3) + (l16 >> 2);
  const int qk_row1 = 16 + qk_row0;
  const int trow0 = 4 * (l16 >> 2) + kb;  // PV keys, mt = 0: 4*q + kb
  const int trow1 = 16 + trow0;           // mt = 1
  const int dsub = 4 * (l16 & 3);

  // ---- partial S^T (32 keys x 16 heads) of tile `tile` over this wave's
  // dims.  Fragment reads go out in batches; scheduling barriers keep batch
  // b+1's reads issued ahead of batch b's MFMAs.
  auto qk = [&](int tile, f32x4_t& sacc0, f32x4_t& sacc1) {
    const uint16_t* tb = tiles[tile % kStages];
    sacc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sacc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int QB = KSTEP < 4 ? KSTEP : 4;  // k-steps per batch
    const uint16_t* rb0 = tb + qk_row0 * D;
    const uint16_t* rb1 = tb + qk_row1 * D;
    bf16x8_t fa[2][2][QB];  // [buffer][m tile][step]
    auto load_batch = [&](int j0, int bi) {
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int chunk = dh * (DH / 8) + kb * KSTEP + j0 + u;
        fa[bi][0][u] = *reinterpret_cast<const bf16x8_t*>(rb0 + ((chunk ^ swz(qk_row0)) * 8));
        fa[bi][1][u] = *reinterpret_cast<const bf16x8_t*>(rb1 + ((chunk ^ swz(qk_row1)) * 8));
      }
    };
    load_batch(0, 0);
#pragma unroll
    for (int j0 = 0; j0 < KSTEP; j0 += QB) {
      const int bi = (j0 / QB) & 1;
      if (j0 + QB < KSTEP) load_batch(j0 + QB, bi ^ 1);
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[bi][0][u], qf[j0 + u], sacc0, 0, 0, 0);
        sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[bi][1][u], qf[j0 + u], sacc1, 0, 0, 0);
      }
    }
  };
  // two planes of 64 x 16 B: each 16-lane phase covers all 64 banks once
  auto put_partial = [&](int tile, const f32x4_t& sacc0, const f32x4_t& sacc1) {
    if constexpr (DSPLIT > 1) {
      *reinterpret_cast<f32x4_t*>(&xs[tile & 1][wave][lane * 4]) = sacc0;
      *reinterpret_cast<f32x4_t*>(&xs[tile & 1][wave][256 + lane * 4]) = sacc1;
    }
  };
  auto add_partner = [&](int tile, f32x4_t& sacc0, f32x4_t& sacc1) {
    if constexpr (DSPLIT > 1) {
      // same heads, other dims (a + b == b + a: both waves hold identical scores)
      const int partner = (wave + NHG) % NW;
      sacc0 += *reinterpret_cast<const f32x4_t*>(&xs[tile & 1][partner][lane * 4]);
      sacc1 += *reinterpret_cast<const f32x4_t*>(&xs[tile & 1][partner][256 + lane * 4]);
    }
  };
  // ---- O += P . V over this wave's dims; P = A operand (head l16, keys
  // mt*16 + 4*i + kb); V via tr16: lane j of a 16-lane block addresses key
  // q = j/4 of the 4 and dims 4*(j%4) .. +3 of the 16-dim column tile
  auto pv = [&](int tile, const bf16x8_t& pa) {
    const uint16_t* tb = tiles[tile % kStages];
    constexpr int PB = NTILE < 4 ? NTILE : 4;  // column tiles per batch
    const uint16_t* r0 = tb + trow0 * D;
    const uint16_t* r1 = tb + trow1 * D;
    const int sw0 = swz(trow0), sw1 = swz(trow1);
    i16x4_t fv[2][2][PB];  // [buffer][key group][column tile]
    auto load_batch = [&](int n0, int bi) {
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int d = dh * DH + (n0 + u) * 16 + dsub;
        const int ch = d >> 3;
        const int off = d & 7;
        fv[bi][0][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(r0 + ((ch ^ sw0) * 8) + off));
        fv[bi][1][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(r1 + ((ch ^ sw1) * 8) + off));
      }
    };
    load_batch(0, 0);
#pragma unroll
    for (int n0 = 0; n0 < NTILE; n0 += PB) {
      const int bi = (n0 / PB) & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (n0 + PB < NTILE) load_batch(n0 + PB, bi ^ 1);
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        bf16x8_t b;
        *reinterpret_cast<i16x4_t*>(&b) = fv[bi][0][u];
        *(reinterpret_cast<i16x4_t*>(&b) + 1) = fv[bi][1][u];
        o[n0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[n0 + u], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Software pipeline, one workgroup barrier per tile.  Iteration `tile`
  // finishes that tile (its partner partial, softmax, P.V) and computes the
  // next tile's partial S^T: half the head groups before their softmax, so
  // the MFMAs of QK(tile+1) run beside its VALU work, the other half after
  // their P.V.  Stage use at iteration `tile`: tile (P.V), tile+1
  // (QK), tile+2 (gather in flight, into the stage tile-1 released).
  // Validity masks of the tiles in flight: current, next, and the one after.
  // An empty split (fewer tiles than splits) skips the pipeline and leaves
  // the empty softmax state (o = 0, m = -inf, l = 0).
  if (n_tiles > 0) {
    // Tile indices below are local to the split (stages and parities); the
    // lookups take the split's global tile index tile_lo + local.
    Look lk = lookup(tile_lo);
    issue(lk, 0);
    uint32_t vm_cur = lk.valid;
    uint32_t vm_next = 0u;
    if (n_tiles > 1) {
      lk = lookup(tile_lo + 1);
      issue(lk, 1);
      vm_next = lk.valid;
    }
    if (n_tiles > 2) lk = lookup(tile_lo + 2);  // the next tile to issue, looked up ahead
    f32x4_t s_own0, s_own1;  // this wave's partial S^T of the current tile
    if (n_tiles > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | kNewer);  // tile 0 landed; tile 1 may fly
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();  // publishes tile 0
    qk(0, s_own0, s_own1);
    put_partial(0, s_own0, s_own1);
    for (int tile = 0; tile < n_tiles; ++tile) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's gather of tile+1 (issued last) landed
      // publishes the partials of `tile` and the rows of tile+1; every wave
      // is done with tile-1, whose stage takes tile+2
      __syncthreads();
      uint32_t vm_after = 0u;
      if (tile + 2 < n_tiles) {
        issue(lk, (tile + 2) % kStages);
        vm_after = lk.valid;
        if (tile + 3 < n_tiles) lk = lookup(tile_lo + tile + 3);  // latency hides under this tile
      }
      const uint32_t vmask = vm_cur;
      vm_cur = vm_next;
      vm_next = vm_after;

      f32x4_t sacc0 = s_own0, sacc1 = s_own1;
      add_partner(tile, sacc0, sacc1);
      // The next tile's partial S^T.  Head groups 0-1 compute it here, so its
      // MFMAs overlap their softmax; the other half after their P.V, so the
      // eight waves' fragment reads of tile+1 do not all follow the barrier
      // at once (same results either way: the partials are published by the
      // next iteration's barrier).
      const bool qk_first = hg < (NHG + 1) / 2;
      if (qk_first && tile + 1 < n_tiles) qk(tile + 1, s_own0, s_own1);

      // lane holds, for head l16, keys mt*16 + 4*i + kb (output rows 4*kb + i)
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0 = 4 * i + kb, k1 = 16 + 4 * i + kb;
        sv[i] = ((vmask >> k0) & 1u) ? sacc0[i] * scale_log2 : -INFINITY;
        sv[4 + i] = ((vmask >> k1) & 1u) ? sacc1[i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(sv[i], sv[4 + i]));
      }
      mx = xor16_32_max(mx);
      // Lazy rescale: exponentials are taken against a reference max m_ref that
      // only moves when the running max passes it by more than kSlack (log2
      // units); p <= 2^kSlack stays far from fp32 / bf16 overflow.
      const bool bump = mx > m_ref + kSlack;
      const float m_new = bump ? mx : m_ref;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      float psum = 0.f;
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);  // v_exp_f32 (tiny results flush to 0)
        psum += pr[i];
      }
      psum = xor16_32_sum(psum);
      bf16x8_t pa;
      {
        uint32_t pk[4];
        pk[0] = pack_bf16x2(pr[0], pr[1]);
        pk[1] = pack_bf16x2(pr[2], pr[3]);
        pk[2] = pack_bf16x2(pr[4], pr[5]);
        pk[3] = pack_bf16x2(pr[6], pr[7]);
        pa = *reinterpret_cast<const bf16x8_t*>(pk);
      }
      if (qk_first && tile + 1 < n_tiles) put_partial(tile + 1, s_own0, s_own1);
      if (__ballot(bump)) {
        const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
        l_run *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kb + i);
#pragma unroll
        for (int n = 0; n < NTILE; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[n][i] *= al[i];
      }
      m_ref = m_new;
      l_run += psum;
      pv(tile, pa);
      if (!qk_first && tile + 1 < n_tiles) {
        qk(tile + 1, s_own0, s_own1);
        put_partial(tile + 1, s_own0, s_own1);
      }
    }
  }
  if (nsplit > 1) {
    // ---- partial state of this split: O unnormalised (fp32, relative to
    // m_ref), and m_ref (log2 units) and l per head
    float* po = part_o + ((t * nsplit + split) * H) * static_cast<int64_t>(D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = hg * 16 + 4 * kb + i;
      if (hh < H) {
#pragma unroll
        for (int n = 0; n < NTILE; ++n) po[hh * static_cast<int64_t>(D) + dh * DH + n * 16 + l16] = o[n][i];
      }
    }
    if (dh == 0 && kb == 0 && hv) {
      part_ml[((t * nsplit + split) * H + head) * 2] = m_ref;
      part_ml[((t * nsplit + split) * H + head) * 2 + 1] = l_run;
    }
    return;
  }
  __syncthreads();  // every wave is done with the tile stages

  // ---- normalise, round, stage through LDS, store 16-byte chunks
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = __shfl(inv, 4 * kb + i);
  static_assert(NW * 16 * DH <= kStages * TILE_ELEMS, "output staging fits the tile stages");
  uint16_t* stage = &tiles[0][0] + wave * 16 * DH;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < NTILE; ++n)
      stage[(4 * kb + i) * DH + n * 16 + l16] = bf16_rne(o[n][i] * iv[i]);
  constexpr int CPH = DH / 8;  // 16-byte chunks per head row of this wave
  for (int c = lane; c < 16 * CPH; c += 64) {
    const int hr = c / CPH;
    const int hh = hg * 16 + hr;
    if (hh < H) {
      *reinterpret_cast<u32x4_t*>(out + (t * H + hh) * (int64_t)D + dh * DH + (c % CPH) * 8) =
          *reinterpret_cast<const u32x4_t*>(stage + hr * DH + (c % CPH) * 8);
    }
  }
}

template <int D, int NHG>
hipError_t launch_hg(const dim3& grid, size_t dyn, hipStream_t s, const uint16_t* q, int64_t q_pos0,
                     int H, float sl2, const uint16_t* raw, int64_t raw_pos0, int window,
                     const uint16_t* pooled, int ratio, const int32_t* sel, int topk,
                     uint16_t* out, int nsplit, float* part_o, float* part_ml) {
  constexpr int DSPLIT = D >= 64 ? 2 : 1;
  hipLaunchKernelGGL((sparse_attn_kernel<D, NHG, DSPLIT>), grid, dim3(NHG * DSPLIT * 64), dyn, s,
                     q, q_pos0, H, sl2, raw, raw_pos0, window, pooled, ratio, sel, topk, out,
                     nsplit, part_o, part_ml);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const void* q, int64_t T, int64_t q_pos0, int H, float sl2, const void* raw,
                    int64_t raw_pos0, int window, const void* pooled, int ratio,
                    const int32_t* sel, int topk, void* out, int nsplit, float* part_o,
                    float* part_ml, hipStream_t s) {
  if (!dispatch_fits(T, 512)) return hipErrorInvalidValue;  // at most 512 work-items each
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(nsplit));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* rr = static_cast<const uint16_t*>(raw);
  const auto* pp = static_cast<const uint16_t*>(pooled);
  auto* oo = static_cast<uint16_t*>(out);
  const size_t dyn = static_cast<size_t>(sel ? topk : 0) * sizeof(int);
  switch ((H + 15) / 16) {
    case 1: return launch_hg<D, 1>(grid, dyn, s, qq, q_pos0, H, sl2, rr, raw_pos0, window, pp, ratio, sel, topk, oo, nsplit, part_o, part_ml);
    case 2: return launch_hg<D, 2>(grid, dyn, s, qq, q_pos0, H, sl2, rr, raw_pos0, window, pp, ratio, sel, topk, oo, nsplit, part_o, part_ml);
    case 3: return launch_hg<D, 3>(grid, dyn, s, qq, q_pos0, H, sl2, rr, raw_pos0, window, pp, ratio, sel, topk, oo, nsplit, part_o, part_ml);
    default: return launch_hg<D, 4>(grid, dyn, s, qq, q_pos0, H, sl2, rr, raw_pos0, window, pp, ratio, sel, topk, oo, nsplit, part_o, part_ml);
  }
}

// Merge of the key splits of one query's attention.  Split s left, per head,
// its reference max m_s (log2 units), its sum l_s of 2^(logit - m_s), and O_s
// = sum of 2^(logit - m_s) * value (fp32, unnormalised; zero for an empty
// split).  With M the largest m_s over non-empty splits (l_s > 0) and
// w_s = 2^(m_s - M) (0 for empty splits):
//   out = sum_s w_s O_s / sum_s w_s l_s, rounded to bf16 (ties to even).
// One workgroup per (query, head).  Wave 0 reduces the nsplit (m, l) pairs
// (one lane each); then thread i accumulates 4 dims over every G-th split
// (G = 256 / (D/4) thread groups), and the G partial sums are added in group
// order.  All sums have a fixed order: the result is deterministic.
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    int nsplit, int H, int D, uint16_t* __restrict__ out) {
  __shared__ float s_w[kMaxAttnSplits];
  __shared__ float s_inv;
  __shared__ f32x4_t s_acc[256];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  if (tid < 64) {
    float m = -INFINITY, l = 0.f;
    if (tid < nsplit) {
      const float* ml = part_ml + ((t * nsplit + tid) * H + h) * 2;
      m = ml[0];
      l = ml[1];
    }
    const bool live = l > 0.f;
    float M = live ? m : -INFINITY;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = live ? exp2f(m - M) : 0.f;
    float L = w * l;
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (tid < nsplit) s_w[tid] = w;
    if (tid == 0) s_inv = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  const int nd4 = D / 4;                 // 8 .. 128
  const int G = 256 / nd4;               // thread groups over the splits
  const int d4 = tid % nd4, g = tid / nd4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = part_o + (t * nsplit * H + h) * static_cast<int64_t>(D) + 4 * d4;
  const int64_t sstride = static_cast<int64_t>(H) * D;
#pragma unroll 4
  for (int sp = g; sp < nsplit; sp += G) {
    const float w = s_w[sp];
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(po + sp * sstride);
    acc += w * v;
  }
  s_acc[tid] = acc;
  __syncthreads();
  if (tid < nd4) {
    f32x4_t sum = s_acc[tid];
    for (int gg = 1; gg < G; ++gg) sum += s_acc[gg * nd4 + tid];
    const float inv = s_inv;
    uint16_t* op = out + (t * H + h) * static_cast<int64_t>(D) + 4 * tid;
#pragma unroll
    for (int j = 0; j < 4; ++j) op[j] = bf16_rne(sum[j] * inv);
  }
}

}  // namespace

hipError_t dsv4_launch_attn_combine(const float* part_o, const float* part_ml, int64_t T,
                                    int32_t nsplit, int32_t n_heads, int32_t head_dim, void* out,
                                    hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (nsplit > kMaxAttnSplits || head_dim % 4 != 0 || head_dim > 1024 || !dispatch_fits(T, 256))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>(T), static_cast<unsigned>(n_heads)),
                     dim3(256), 0, s, part_o, part_ml, nsplit, n_heads, head_dim,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t dsv4_launch_sparse_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                                   int32_t head_dim, float scale, const void* raw_kv,
                                   int64_t raw_pos0, int32_t window, const void* pooled,
                                   int32_t ratio, const int32_t* sel_idx, int32_t topk,
                                   void* out, int32_t nsplit, float* part_o, float* part_ml,
                                   hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (nsplit < 1) return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  if (head_dim == 512 && n_heads == 64 && dsv4_attn_h64_fits(sel_idx ? topk : 0))
    return dsv4_launch_sparse_attn_h64(q, T, q_pos0, sl2, raw_kv, raw_pos0, window, pooled, ratio,
                                       sel_idx, topk, out, nsplit, part_o, part_ml, s);
  switch (head_dim) {
    case 32: return launch_d<32>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, ratio, sel_idx, topk, out, nsplit, part_o, part_ml, s);
    case 64: return launch_d<64>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, ratio, sel_idx, topk, out, nsplit, part_o, part_ml, s);
    case 128: return launch_d<128>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, ratio, sel_idx, topk, out, nsplit, part_o, part_ml, s);
    case 256: return launch_d<256>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, ratio, sel_idx, topk, out, nsplit, part_o, part_ml, s);
    case 512: return launch_d<512>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, ratio, sel_idx, topk, out, nsplit, part_o, part_ml, s);
    default: return hipErrorInvalidValue;
  }
}
