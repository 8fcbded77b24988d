"""Parity at the full workload sizes, in the launch configuration the bench
times, on rows the oracle can compute one by one.

Sampled rows: the first and last rows of every query tile, rows on both sides
of a 4-token boundary, and seeded random rows.  Pooled rows of the chunk and
the all-pooled selections are checked in full.
"""
import math

import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import ATTN_ATOL, ChunkState, assert_scores_close, assert_selection_matches

pytestmark = pytest.mark.gpu


def sample_rows(T, tile, n_random, seed=0):
    rows = set()
    for t0 in range(0, T, tile):
        rows.update({t0, min(T, t0 + tile) - 1})
    rows.update({1, 2, 3, 4, T // 2 - 1, T // 2})
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, T, size=n_random))
    return sorted(r for r in rows if 0 <= r < T)


def run_chunk(cs: ChunkState, tile: int):
    wl = cs.wl
    T, S = wl.chunk, cs.S
    tile_rows = T if tile == 0 else tile
    stride = dsv4.dsv4_score_stride(S)
    scratch = torch.empty((tile_rows, stride), device="cuda")
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    ap = dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx, cs.w, T, cs.q_pos0,
                                  wl.idx_heads, wl.topk, idx, scratch, tile)
    out = torch.empty((T, wl.heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, wl.window,
                                  cs.acache, idx, out)
    torch.cuda.synchronize()
    return ap, scratch, idx, out


def check_chunk(cs: ChunkState, tile: int, n_random: int, n_attn: int):
    wl = cs.wl
    T, S = wl.chunk, cs.S
    ap, scratch, idx, out = run_chunk(cs, tile)
    assert not ap
    # pooled rows appended by this chunk: bit-exact
    n_new = T // 4
    np.testing.assert_array_equal(cs.icache.rows[S - n_new:S].float().cpu().numpy(),
                                  cs.oracle_keys()[S - n_new:S])
    np.testing.assert_array_equal(cs.acache.rows[S - n_new:S].float().cpu().numpy(),
                                  cs.oracle_pooled()[S - n_new:S])
    tile_rows = T if tile == 0 else tile
    last_t0 = (T - 1) // tile_rows * tile_rows
    rows = sample_rows(T, tile_rows, n_random)
    keys = cs.oracle_keys()
    gidx = idx.cpu().numpy()
    # the last tile's scores, recomputed (the score kernel is deterministic):
    # over rows longer than 32,768 columns the select keeps its chunk
    # candidates in the scratch's score rows
    last = torch.empty((T - last_t0, dsv4.dsv4_score_stride(S)), device="cuda")
    dsv4.dsv4_indexer_scores(cs.icache, cs.q_idx[last_t0:].contiguous(),
                             cs.w[last_t0:].contiguous(), cs.q_pos0 + last_t0, last)
    torch.cuda.synchronize()
    g_scr = last.cpu().numpy()
    for t in rows:
        ref = O.indexer_scores(cs.inp["q_idx"][t:t + 1], cs.inp["w"][t:t + 1], keys,
                               cs.q_pos0 + t, S)
        assert_selection_matches(gidx[t:t + 1], ref, cs.q_pos0 + t, wl.topk)
        if t >= last_t0:
            g = g_scr[t - last_t0:t - last_t0 + 1, :S]
            assert_scores_close(g, ref)
            # the GPU's choice is the exact top-k of its own fp32 scores
            np.testing.assert_array_equal(gidx[t:t + 1],
                                          O.topk_select(g.astype(np.float64), cs.q_pos0 + t, wl.topk))
    # attention on a subset of the sampled rows, fed the GPU's own selection
    pooled = cs.oracle_pooled()
    g_out = out[rows[:n_attn]].float().cpu().numpy()
    for i, t in enumerate(rows[:n_attn]):
        ref = O.sparse_prefill_attention(cs.inp["q_attn"][t:t + 1], cs.q_pos0 + t,
                                         cs.inp["raw_kv"], cs.raw_pos0, wl.window, pooled,
                                         gidx[t:t + 1], 1 / math.sqrt(wl.head_dim))
        err = np.abs(g_out[i] - ref[0]).max()
        assert err <= ATTN_ATOL, (t, err)


def test_ctx4k_chunk2048():
    check_chunk(ChunkState(SI.CTX_4K), tile=0, n_random=24, n_attn=12)


def test_ctx128k_chunk2048():
    check_chunk(ChunkState(SI.CTX_128K), tile=0, n_random=12, n_attn=8)


def test_ctx1m_chunk4096_tile1024():
    check_chunk(ChunkState(SI.CTX_1M), tile=SI.CTX_1M.tile_rows, n_random=4, n_attn=6)


def test_ctx16k_eight_chunks_skip_then_full():
    """Eight 2,048-token chunks from an empty cache with k = 2,048: the first
    four take the all-pooled path (S = 512 .. 2,048 <= k, selections checked in
    full), the last four the full path (sampled rows)."""
    wl = SI.CTX_16K
    T, k = wl.chunk, wl.topk
    seed = 0
    icache = dsv4.PoolCache(wl.capacity_rows, wl.idx_dim)
    acache = dsv4.PoolCache(wl.capacity_rows, wl.head_dim)
    ost = O.PoolingCacheState(wl.idx_dim, wl.capacity_rows)
    total = 8 * T
    keys_all = SI.as_bf16_values(SI.normal(seed, "idx_keys_stream", (total, wl.idx_dim)))
    kv_all = SI.as_bf16_values(SI.normal(seed, "kv_stream", (total, wl.head_dim)))
    keys_dev = torch.from_numpy(keys_all).to(torch.bfloat16).cuda()
    kv_dev = torch.from_numpy(kv_all).to(torch.bfloat16).cuda()
    for c in range(8):
        q_pos0 = c * T
        dsv4.dsv4_compress(icache, keys_dev[q_pos0:q_pos0 + T])
        dsv4.dsv4_compress(acache, kv_dev[q_pos0:q_pos0 + T])
        O.compress(ost, keys_all[q_pos0:q_pos0 + T])
        S = icache.n_rows
        assert S == acache.n_rows == (c + 1) * T // 4
        q = SI.as_bf16_values(SI.normal(seed, f"q_idx_chunk{c}", (T, wl.idx_heads, wl.idx_dim)))
        w = SI.uniform(seed, f"w_chunk{c}", (T, wl.idx_heads))
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        scratch = torch.empty((T, dsv4.dsv4_score_stride(S)), device="cuda")
        ap = dsv4.dsv4_indexer_select(icache, acache.n_rows,
                                      torch.from_numpy(q).to(torch.bfloat16).cuda(),
                                      torch.from_numpy(w).cuda(), T, q_pos0, wl.idx_heads, k,
                                      idx, scratch)
        torch.cuda.synchronize()
        gidx = idx.cpu().numpy()
        if c < 4:
            assert ap, f"chunk {c + 1} should take the all-pooled path"
            np.testing.assert_array_equal(gidx, O.all_pooled_selection(T, q_pos0, k))
        else:
            assert not ap
            for t in sample_rows(T, T, 6, seed=c):
                ref = O.indexer_scores(q[t:t + 1], w[t:t + 1], ost.rows[:S], q_pos0 + t, S)
                assert_selection_matches(gidx[t:t + 1], ref, q_pos0 + t, k)
    np.testing.assert_array_equal(icache.rows[:icache.n_rows].float().cpu().numpy(),
                                  ost.rows[:ost.n_rows])


# ---------------------------------------------------------------- sibling modes and narrow steps
# The same launch configurations bench.py times: the 2,048-row chunk at 128K
# context in the window-only and ratio-128 modes, and T = 1-4 query rows at
# the end of a context.

def test_ctx128k_chunk2048_local_and_ratio128_modes():
    wl = SI.CTX_128K
    cs = ChunkState(wl)
    T, H, D, W = wl.chunk, wl.heads, wl.head_dim, wl.window
    scale = 1 / math.sqrt(D)
    rows = sample_rows(T, T, 6, seed=3)
    # window only
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, None, None, out)
    torch.cuda.synchronize()
    g = out[rows].float().cpu().numpy()
    for i, t in enumerate(rows):
        ref = O.sparse_prefill_attention(cs.inp["q_attn"][t:t + 1], cs.q_pos0 + t, cs.inp["raw_kv"],
                                         cs.raw_pos0, W, None, None, scale)
        assert np.abs(g[i] - ref[0]).max() <= ATTN_ATOL, ("local", t)
    # ratio-128 pool: prefix rows, then the chunk through the compressor
    prefix_t, prefix = SI.prefix_rows_ratio(wl, 0, 128)
    n128 = prefix.shape[0]
    c128 = dsv4.PoolCache(n128 + T // 128 + 1, D, ratio=128)
    c128.rows[:n128].copy_(prefix_t)
    c128.set_state(n128, 0)
    chunk = cs.inp["raw_kv"][cs.q_pos0 - cs.raw_pos0:]
    dsv4.dsv4_compress(c128, cs.raw_kv[cs.q_pos0 - cs.raw_pos0:])
    st = O.PoolingCacheState(D, n128 + T // 128 + 1, ratio=128)
    st.rows[:n128] = prefix
    st.n_rows = n128
    O.compress(st, chunk)
    S = c128.n_rows
    assert S == st.n_rows == (cs.q_pos0 + T) // 128
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, c128, None, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c128.rows[n128:S].float().cpu().numpy(), st.rows[n128:S])
    g = out[rows].float().cpu().numpy()
    for i, t in enumerate(rows):
        ref = O.sparse_prefill_attention(cs.inp["q_attn"][t:t + 1], cs.q_pos0 + t, cs.inp["raw_kv"],
                                         cs.raw_pos0, W, st.rows[:S], None, scale, ratio=128)
        assert np.abs(g[i] - ref[0]).max() <= ATTN_ATOL, ("ratio128", t)


@pytest.mark.parametrize("wl,T", [(SI.CTX_128K, 4), (SI.CTX_1M, 2)], ids=["ctx128k-T4", "ctx1m-T2"])
def test_narrow_steps_at_end_of_context(wl, T):
    """T query rows at the last positions the caches cover, as bench.py's
    narrow section runs them: indexer select with the scratch
    dsv4_indexer_scratch_bytes sizes (the chunk-parallel top-k at 1M), then
    the key-split attention with its planned split count.  Every row is
    checked."""
    cs = ChunkState(wl)
    S = cs.S
    H, D, W, k = wl.heads, wl.head_dim, wl.window, wl.topk
    q0 = 4 * S - T
    scratch = torch.empty(dsv4.dsv4_indexer_scratch_bytes(T, S) // 4, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    assert not dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx[:T], cs.w[:T], T, q0,
                                        wl.idx_heads, k, idx, scratch, 0)
    ns, nb = dsv4.dsv4_sparse_attn_narrow_plan(T, H, D, W, k)
    assert ns > 1
    ws = torch.empty(nb // 4, device="cuda")
    raw_lo = q0 - W + 1
    raw = cs.raw_kv[raw_lo - cs.raw_pos0:q0 + T - cs.raw_pos0]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_attn_narrow(cs.q_attn[:T], q0, raw, raw_lo, W, cs.acache, idx, out, ns, ws)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    ref = O.indexer_scores(cs.inp["q_idx"][:T], cs.inp["w"][:T], cs.oracle_keys(), q0, S)
    assert_selection_matches(gidx, ref, q0, k)
    raw_np = cs.inp["raw_kv"][raw_lo - cs.raw_pos0:q0 + T - cs.raw_pos0]
    ref_o = O.sparse_prefill_attention(cs.inp["q_attn"][:T], q0, raw_np, raw_lo, W,
                                       cs.oracle_pooled(), gidx, 1 / math.sqrt(D))
    err = np.abs(out.float().cpu().numpy() - ref_o).max()
    assert err <= ATTN_ATOL, err
