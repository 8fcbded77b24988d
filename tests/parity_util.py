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


# ---------------------------------------------------------------- row samples

def spread_rows(T: int, n: int, tile: int = 0, seed: int = 0, shares: int = 8):
    """About ``n`` rows of a T-row chunk, spread over ``shares`` equal
    contiguous shares (the attention kernel deals queries to the eight XCDs
    in contiguous eighths, so every share is a different XCD's work): each
    share's first and last row and seeded random rows inside it, plus the
    first and last row of every ``tile``-row query tile and both rows around
    every share's middle 4-token boundary."""
    rows = set()
    rng = np.random.default_rng(seed)
    bounds = [T * i // shares for i in range(shares + 1)]
    per = max(2, n // shares)
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            continue
        rows.update({a, b - 1})
        m = (a + b) // 2 // 4 * 4
        rows.update({m - 1, m})
        rows.update(int(r) for r in rng.integers(a, b, size=max(0, per - 4)))
    if tile:
        for t0 in range(0, T, tile):
            rows.update({t0, min(T, t0 + tile) - 1})
    return sorted(r for r in rows if 0 <= r < T)


# ---------------------------------------------------------------- needle attention
# With N(0,1) queries over ~2,000 keys the softmax is nearly flat, and leaving
# out a whole 32-key group of keys moves the output by less than the 2e-2 bar.
# Needle queries make every 32-key group decisive: each query's key list
# (window rows oldest first, then the selection's slots in order -- the order
# the attention walks its keys) is cut into groups of 32, one key of each
# group is a needle for one head (groups dealt to heads round-robin), and that
# head's query is a sum of its needles scaled so that each needle's logit is
# about ln(number of keys): each needle then carries a large share of its
# head's softmax.  A pooled needle is first projected off the span of the
# query's window rows (unless it lies mostly inside it: a pooled row of the
# window's own tokens), so the window keys (larger than pooled rows) get no
# large logits from it.  A skipped, repeated or wrongly gathered group moves
# its head's output far beyond that head's bar (``check_needle_rows``).

NEEDLE_GROUP = 32


def attention_keys(t, q_pos0, window, raw, raw_pos0, pooled, sel, ratio=4):
    """(key rows of query t in walk order, float64 [n, D]; window key count)."""
    p = q_pos0 + t
    lo = max(0, p - window + 1)
    keys = [np.asarray(raw[j - raw_pos0], dtype=np.float64) for j in range(lo, p + 1)]
    n_win = len(keys)
    if pooled is not None:
        vis = O.visible_rows(p, ratio)
        slots = range(vis) if sel is None else [int(s) for s in sel[t] if 0 <= int(s) < vis]
        keys += [np.asarray(pooled[s], dtype=np.float64) for s in slots]
    return np.stack(keys, axis=0), n_win


def needle_queries(T, q_pos0, H, window, raw, raw_pos0, pooled, sel, scale, seed=0,
                   ratio=4, noise=0.1, rows=None):
    """bf16-exact attention queries [T, H, D] with one needle per 32-key group
    (for the queries in ``rows``, default all; the others are plain noise).

    ``sel`` rows must hold their valid slots first (trailing -1 only), so the
    slot order equals the key order.  A pooled row whose tokens all lie in
    the query's window is a mean of window keys: it can never outweigh them,
    and leaving it out barely moves the output, so a needle is drawn among
    the other keys of its group (``without_window_rows`` removes such rows
    from a selection)."""
    rng = np.random.default_rng(seed)
    D = np.asarray(raw).shape[1]
    q = rng.standard_normal((T, H, D), dtype=np.float32) * np.float32(noise)
    for t in (range(T) if rows is None else rows):
        K, n_win = attention_keys(t, q_pos0, window, raw, raw_pos0, pooled, sel, ratio)
        U = np.linalg.qr(K[:n_win].T)[0]                 # [D, n_win] orthonormal
        perp = K[n_win:] - (K[n_win:] @ U) @ U.T          # pooled keys off the window span
        ok = np.ones(K.shape[0], dtype=bool)
        ok[n_win:] = np.einsum("ij,ij->i", perp, perp) >= 0.25 * np.einsum("ij,ij->i", K[n_win:], K[n_win:])
        n = K.shape[0]
        target = np.log(n)
        for g in range((n + NEEDLE_GROUP - 1) // NEEDLE_GROUP):
            g0, g1 = g * NEEDLE_GROUP, min(n, (g + 1) * NEEDLE_GROUP)
            cand = np.nonzero(ok[g0:g1])[0]
            j = g0 + int(rng.choice(cand) if cand.size else rng.integers(0, g1 - g0))
            k = K[j]
            d = k if (j < n_win or not ok[j]) else perp[j - n_win]
            q[t, g % H] += target / (scale * float(d @ k)) * d
    return SI.as_bf16_values(q.astype(np.float32))


def without_window_rows(sel, q_pos0, window, ratio=4):
    """Selection with the pooled rows whose tokens all lie inside the query's
    window removed (valid slots compacted to the front, -1 after)."""
    sel = np.asarray(sel)
    out = np.full_like(sel, -1)
    for t in range(sel.shape[0]):
        p = q_pos0 + t
        lo = max(0, p - window + 1)
        vis = O.visible_rows(p, ratio)
        keep = [int(s) for s in sel[t] if 0 <= int(s) < vis and ratio * int(s) < lo]
        out[t, :len(keep)] = keep
    return out


def group_power(q_row, K, scale):
    """Per head h: the smallest change of that head's output (max |.| over
    dims) when one of the 32-key groups dealt to h (groups g with g % H == h)
    is left out or counted twice; inf for a head with no group."""
    q_row = np.asarray(q_row, dtype=np.float64)
    H = q_row.shape[0]
    logits = scale * (q_row @ K.T)                       # [H, n]
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    num = e @ K                                          # [H, D]
    den = e.sum(axis=1, keepdims=True)
    out = num / den
    power = np.full(H, np.inf)
    n = K.shape[0]
    for g, g0 in enumerate(range(0, n, NEEDLE_GROUP)):
        h = g % H
        eg = e[h, g0:g0 + NEEDLE_GROUP]
        ng = eg @ K[g0:g0 + NEEDLE_GROUP]
        dg = eg.sum()
        dup = np.abs((num[h] + ng) / (den[h, 0] + dg) - out[h]).max()
        drop = np.abs((num[h] - ng) / (den[h, 0] - dg) - out[h]).max() if den[h, 0] > dg * (1 + 1e-12) else np.inf
        power[h] = min(power[h], drop, dup)
    return power


def _bf16_ulp(x):
    x = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def check_needle_rows(g_out, rows, q, q_pos0, window, raw, raw_pos0, pooled, sel, scale,
                      ratio=4, atol=None):
    """GPU output rows vs the fp64 oracle, head by head, at a bar of
    min(2e-2, a quarter of the smallest change one of the head's groups
    makes when left out or counted twice): a single skipped, repeated or
    wrongly gathered 32-key group fails its head.  Each bar must stay at
    least one bf16 ulp of the head's largest output (twice the rounding of
    the bf16 output), so that output rounding alone cannot fail it (the
    case's own power, checked on the oracle)."""
    atol = ATTN_ATOL if atol is None else atol
    worst = 0.0
    for i, t in enumerate(rows):
        ref = O.sparse_prefill_attention(q[t:t + 1], q_pos0 + t, raw, raw_pos0, window, pooled,
                                         None if sel is None else sel[t:t + 1], scale,
                                         ratio=ratio)[0]
        K, _ = attention_keys(t, q_pos0, window, raw, raw_pos0, pooled, sel, ratio)
        bar = np.minimum(atol, group_power(q[t], K, scale) / 4)   # [H]
        floor = _bf16_ulp(np.abs(ref).max(axis=1))
        assert np.all(bar >= floor), (t, np.argmin(bar - floor), bar.min())
        err = np.abs(np.asarray(g_out[i], dtype=np.float64) - ref).max(axis=1)   # [H]
        bad = np.nonzero(err > bar)[0]
        assert bad.size == 0, (t, [(int(h), float(err[h]), float(bar[h])) for h in bad[:4]])
        worst = max(worst, float(err.max()))
    return worst
