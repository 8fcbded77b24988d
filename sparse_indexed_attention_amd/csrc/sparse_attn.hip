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
// the pooled rows listed in the query's selection with 0 <= s < (p+1)/4
// (all of them when no selection is given); values are the keys (one KV row
// shared by all heads); out = softmax(scale * q.K) . K.
//
// Mapping onto CDNA4:
//   * one workgroup per query, one wave per 16 heads (4 waves at H = 64);
//   * keys are gathered 32 at a time (each row contiguous, 16-byte loads,
//     one 1 KiB row per 64 lanes) into LDS twice: row-major for the QK^T
//     operand and transposed (dims x keys) for the PV operand;
//   * QK^T is computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_16x16x32_bf16: the wave's Q block is the B operand and
//     stays in VGPRs; in the result each lane holds 8 keys of one head, which
//     is exactly the A-operand layout PV needs (the key order inside the
//     contraction is permuted the same way for P and V), so probabilities
//     never leave the lane;
//   * online softmax in fp32 (exp2 with the scale folded in), running max
//     and sum per head reduced across the four 16-lane groups;
//   * O (16 heads x D per wave) accumulates in fp32 registers; the final
//     1/sum scaling and bf16 rounding happen once at the end.
#include "dsv4_device.h"

using namespace dsv4;

namespace {

constexpr int kKeys = 32;  // keys per LDS tile

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
sparse_attn_kernel(const uint16_t* __restrict__ q, int64_t q_pos0, int H, float scale_log2,
                   const uint16_t* __restrict__ raw, int64_t raw_pos0, int window,
                   const uint16_t* __restrict__ pooled, const int32_t* __restrict__ sel,
                   int topk, uint16_t* __restrict__ out) {
  constexpr int NT = NW * 64;
  constexpr int KP = D + 8;        // row-major key tile pitch (uint16)
  constexpr int VP = kKeys + 8;    // transposed tile pitch (uint16)
  constexpr int KSTEP = D / 32;    // QK^T contraction steps
  constexpr int NTILE = D / 16;    // PV output column tiles
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kKeys * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vtile[D * VP];
  __shared__ int s_valid[kKeys];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = lane >> 4;   // 16-lane group
  const int l16 = lane & 15;

  const int64_t t = blockIdx.x;
  const int64_t p = q_pos0 + t;
  const int64_t lo = (p - window + 1) > 0 ? (p - window + 1) : 0;
  const int n_win = static_cast<int>(p - lo + 1);
  const int64_t vis = visible_rows(p);

  // ---- number of pooled slots to walk
  int n_slots;
  if (sel) {
    if (tid == 0) s_last = -1;
    __syncthreads();
    int last = -1;
    const int32_t* sp = sel + t * topk;
    for (int j = tid; j < topk; j += NT) {
      const int32_t s = sp[j];
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
  const int n_tiles = (n_keys + kKeys - 1) / kKeys;

  // ---- this wave's Q block (B operand of S^T = K.Q^T)
  const int head = wave * 16 + l16;
  const bool hv = head < H;
  bf16x8_t qf[KSTEP];
  {
    const uint16_t* qp = q + ((t * H + head) * (int64_t)D + kb * (D / 4));
#pragma unroll
    for (int j = 0; j < KSTEP; ++j)
      qf[j] = hv ? *reinterpret_cast<const bf16x8_t*>(qp + j * 8) : bf16x8_t{};
  }

  f32x4_t o[NTILE];
#pragma unroll
  for (int n = 0; n < NTILE; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // per head (this lane's head l16)
  float l_run = 0.f;

  for (int tile = 0; tile < n_tiles; ++tile) {
    __syncthreads();  // previous tile fully consumed
    // ---- gather 32 keys into LDS (row-major and transposed)
    for (int ci = tid; ci < kKeys * CPR; ci += NT) {
      const int kk = ci / CPR;
      const int c8 = ci - kk * CPR;
      const int j = tile * kKeys + kk;
      const uint16_t* rp = nullptr;
      if (j < n_win) {
        rp = raw + (lo + j - raw_pos0) * D;
      } else if (j < n_keys) {
        const int slot = j - n_win;
        int64_t s = sel ? static_cast<int64_t>(sel[t * topk + slot]) : slot;
        if (s >= 0 && s < vis) rp = pooled + s * D;
      }
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (rp) v = *reinterpret_cast<const u32x4_t*>(rp + c8 * 8);
      if (c8 == 0) s_valid[kk] = rp != nullptr;
      *reinterpret_cast<u32x4_t*>(&ktile[kk * KP + c8 * 8]) = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vtile[(c8 * 8 + 2 * e) * VP + kk] = static_cast<uint16_t>(v[e] & 0xffffu);
        vtile[(c8 * 8 + 2 * e + 1) * VP + kk] = static_cast<uint16_t>(v[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T (32 keys x 16 heads) = K . Q^T
    f32x4_t sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kp = &ktile[(mt * 16 + l16) * KP + kb * (D / 4)];
#pragma unroll
      for (int j = 0; j < KSTEP; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + j * 8);
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j], sacc[mt], 0, 0, 0);
      }
    }
    // lane holds keys mt*16 + 4*kb + i (i < 4) for head l16
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = mt * 16 + 4 * kb + i;
        const float x = s_valid[kk] ? sacc[mt][i] * scale_log2 : -INFINITY;
        sv[mt * 4 + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = exp2f(sv[i] - m_use);
      psum += pr[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- rescale O rows (heads 4*kb + i) by their head's alpha
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kb + i);
#pragma unroll
    for (int n = 0; n < NTILE; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= al[i];

    // ---- P (A operand: head l16, keys {4kb+i, 16+4kb+i}) . V
    bf16x8_t pa;
    {
      uint32_t pk[4];
      pk[0] = pack_bf16x2(pr[0], pr[1]);
      pk[1] = pack_bf16x2(pr[2], pr[3]);
      pk[2] = pack_bf16x2(pr[4], pr[5]);
      pk[3] = pack_bf16x2(pr[6], pr[7]);
      pa = *reinterpret_cast<const bf16x8_t*>(pk);
    }
#pragma unroll
    for (int n = 0; n < NTILE; ++n) {
      const uint16_t* vp = &vtile[(n * 16 + l16) * VP];
      uint32_t bk[4];
      const uint2 lo4 = *reinterpret_cast<const uint2*>(vp + 4 * kb);
      const uint2 hi4 = *reinterpret_cast<const uint2*>(vp + 16 + 4 * kb);
      bk[0] = lo4.x; bk[1] = lo4.y; bk[2] = hi4.x; bk[3] = hi4.y;
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(bk);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[n], 0, 0, 0);
    }
  }

  // ---- normalise and store: lane holds heads 4*kb + i, dim n*16 + l16
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = __shfl(inv, 4 * kb + i);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = wave * 16 + 4 * kb + i;
    if (hh < H) {
      uint16_t* op = out + (t * H + hh) * (int64_t)D;
#pragma unroll
      for (int n = 0; n < NTILE; ++n) op[n * 16 + l16] = f32_to_bf16_bits(o[n][i] * iv[i]);
    }
  }
}

template <int D>
hipError_t launch_d(const void* q, int64_t T, int64_t q_pos0, int H, float scale_log2,
                    const void* raw, int64_t raw_pos0, int window, const void* pooled,
                    const int32_t* sel, int topk, void* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(T));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* rr = static_cast<const uint16_t*>(raw);
  const auto* pp = static_cast<const uint16_t*>(pooled);
  auto* oo = static_cast<uint16_t*>(out);
  const int nw = (H + 15) / 16;
  switch (nw) {
    case 1: hipLaunchKernelGGL((sparse_attn_kernel<D, 1>), grid, dim3(64), 0, s, qq, q_pos0, H, scale_log2, rr, raw_pos0, window, pp, sel, topk, oo); break;
    case 2: hipLaunchKernelGGL((sparse_attn_kernel<D, 2>), grid, dim3(128), 0, s, qq, q_pos0, H, scale_log2, rr, raw_pos0, window, pp, sel, topk, oo); break;
    case 3: hipLaunchKernelGGL((sparse_attn_kernel<D, 3>), grid, dim3(192), 0, s, qq, q_pos0, H, scale_log2, rr, raw_pos0, window, pp, sel, topk, oo); break;
    default: hipLaunchKernelGGL((sparse_attn_kernel<D, 4>), grid, dim3(256), 0, s, qq, q_pos0, H, scale_log2, rr, raw_pos0, window, pp, sel, topk, oo); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t dsv4_launch_sparse_attn(const void* q, int64_t T, int64_t q_pos0, int32_t n_heads,
                                   int32_t head_dim, float scale, const void* raw_kv,
                                   int64_t raw_pos0, int32_t window, const void* pooled,
                                   const int32_t* sel_idx, int32_t topk, void* out,
                                   hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  switch (head_dim) {
    case 32: return launch_d<32>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, sel_idx, topk, out, s);
    case 64: return launch_d<64>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, sel_idx, topk, out, s);
    case 128: return launch_d<128>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, sel_idx, topk, out, s);
    case 256: return launch_d<256>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, sel_idx, topk, out, s);
    case 512: return launch_d<512>(q, T, q_pos0, n_heads, sl2, raw_kv, raw_pos0, window, pooled, sel_idx, topk, out, s);
    default: return hipErrorInvalidValue;
  }
}
