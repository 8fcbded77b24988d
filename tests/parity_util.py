"""Shared helpers of the GPU parity tests: building the chunk state on the
device through the C ABI and on the host through the oracle from the same
seeded inputs, and the comparison rules.

Comparison rules (written here once, used by every test):
  * pooled rows, remainders, selected indices: bit-exact;
  * scores: |gpu - ref| <= 1e-3 * |ref| + 1e-6 * max_s |ref[t, s]| and -inf
    exactly where the oracle masks;
  * selections against the fp64 oracle: equal, except that where the k-th and
    (k+1)-th oracle scores of a row are within 1e-3 relative, rows whose
    oracle score lies inside that band may differ (any choice among them is
    a correct top-k up to rounding); the GPU's choice must still be a valid
    top-k of its own fp32 scores (checked bit-exactly by running the oracle's
    top-k on those fp32 scores);
  * attention output: max |gpu - ref| <= 2e-2 against fp64.
"""
from __future__ import annotations

import numpy as np
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

SCORE_RTOL = 1e-3
SCORE_ATOL_ROWSCALE = 1e-6
TIE_BAND = 1e-3
ATTN_ATOL = 2e-2


def bf16_t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


class ChunkState:
    """Device caches (through dsv4_compress) and oracle caches for one chunk of a workload."""

    def __init__(self, wl: SI.Workload, seed: int = 0, with_attn_q: bool = True,
                 prefix_rem: int = 0):
        self.wl = wl
        inp = SI.make_inputs(wl, seed, with_attn_q=with_attn_q)
        if not wl.bf16:  # float32 case fed to bf16 kernels: round the inputs once, both sides
            for k in list(inp):
                if isinstance(inp[k], np.ndarray) and k != "w":
                    inp[k] = SI.as_bf16_values(inp[k])
                    inp[k + "_t"] = bf16_t(inp[k])
        self.inp = inp
        T = wl.chunk
        n_prefix = wl.prefix_tokens // 4
        cap = wl.capacity_rows
        self.icache = dsv4.PoolCache(cap, wl.idx_dim)
        self.acache = dsv4.PoolCache(cap, wl.head_dim)
        self.ostate_i = O.PoolingCacheState(wl.idx_dim, cap)
        self.ostate_a = O.PoolingCacheState(wl.head_dim, cap)
        if n_prefix:
            self.icache.rows[:n_prefix].copy_(inp["prefix_idx_rows_t"])
            self.acache.rows[:n_prefix].copy_(inp["prefix_attn_rows_t"])
            self.icache.set_state(n_prefix, 0)
            self.acache.set_state(n_prefix, 0)
            self.ostate_i.rows[:n_prefix] = inp["prefix_idx_rows"]
            self.ostate_a.rows[:n_prefix] = inp["prefix_attn_rows"]
            self.ostate_i.n_rows = self.ostate_a.n_rows = n_prefix
        self.q_pos0 = wl.q_pos0
        self.raw_pos0 = inp["raw_pos0"]
        chunk_raw = inp["raw_kv"][wl.q_pos0 - self.raw_pos0:]
        chunk_raw_t = inp["raw_kv_t"][wl.q_pos0 - self.raw_pos0:]
        assert chunk_raw.shape[0] == T
        # ---- compress the chunk (device through the ABI, host through the oracle)
        dsv4.dsv4_compress(self.icache, inp["idx_keys_t"].cuda())
        dsv4.dsv4_compress(self.acache, chunk_raw_t.cuda())
        O.compress(self.ostate_i, inp["idx_keys"])
        O.compress(self.ostate_a, chunk_raw)
        self.S = self.icache.n_rows
        assert self.S == self.ostate_i.n_rows == wl.n_rows_after
        # ---- device inputs
        self.q_idx = inp["q_idx_t"].cuda()
        self.w = inp["w_t"].cuda()
        self.raw_kv = inp["raw_kv_t"].cuda()
        self.q_attn = inp["q_attn_t"].cuda() if with_attn_q else None

    def oracle_keys(self):
        return self.ostate_i.rows[:self.S]

    def oracle_pooled(self):
        return self.ostate_a.rows[:self.S]


def assert_scores_close(gpu, ref, rows=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    mref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), mref), "mask (-inf) positions differ"
    fin = ~mref
    rowmax = np.max(np.where(fin, np.abs(ref), 0.0), axis=1, keepdims=True)
    bound = SCORE_RTOL * np.abs(ref) + SCORE_ATOL_ROWSCALE * rowmax
    err = np.abs(np.where(fin, gpu, 0.0) - np.where(fin, ref, 0.0))
    bad = fin & ~(err <= bound)
    assert not bad.any(), (f"{bad.sum()} scores out of tolerance; worst rel "
                           f"{np.max(np.where(fin, err / (np.abs(ref) + 1e-30), 0)):.3g}")


def assert_selection_matches(gpu_idx, ref_scores, q_pos0, topk):
    """Row-wise: GPU selection vs the fp64 oracle selection with the near-tie band."""
    gpu_idx = np.asarray(gpu_idx)
    ref_sel = O.topk_select(ref_scores, q_pos0, topk)
    n_band_rows = 0
    for t in range(gpu_idx.shape[0]):
        if np.array_equal(gpu_idx[t], ref_sel[t]):
            continue
        vis = O.visible_rows(q_pos0 + t)
        k_eff = min(topk, vis)
        r = np.asarray(ref_scores[t, :vis], dtype=np.float64)
        srt = np.sort(r)[::-1]
        assert k_eff < vis, f"row {t}: everything visible must be selected"
        rk, rk1 = srt[k_eff - 1], srt[k_eff]
        scale = max(abs(rk), 1e-30)
        assert rk - rk1 < TIE_BAND * scale, f"row {t}: selections differ outside a near tie"
        band = TIE_BAND * scale + SCORE_ATOL_ROWSCALE * np.max(np.abs(r))
        g = set(int(s) for s in gpu_idx[t] if s >= 0)
        o = set(int(s) for s in ref_sel[t] if s >= 0)
        assert len(g) == k_eff and all(0 <= s < vis for s in g)
        for s in g.symmetric_difference(o):
            assert abs(r[s] - rk) <= band, f"row {t}: index {s} far from the threshold"
        n_band_rows += 1
    return n_band_rows
