"""Parity at the full workload sizes, in the launch configuration the bench
times.

Rows checked against the oracle:
  * 4K and 16K: every query row of the chunk (scores, selection, attention);
  * 128K: 256 rows, 1M: 64 rows, spread over the eight contiguous shares the
    attention kernel deals to the eight XCDs, with the first and last row of
    every indexer tile and rows on both sides of 4-token boundaries.
Pooled rows of the chunk and the all-pooled selections are checked in full.

Attention is checked twice per workload: with the workload's N(0,1) queries
on the GPU's own selection (max |err| <= 2e-2 against fp64), and with needle
queries on that selection less its pooled rows made only of window tokens,
under which every 32-key group of keys carries a large share of one head's
softmax, so that one skipped, repeated or wrongly gathered group fails
(``parity_util.check_needle_rows``).
"""
import math

import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import (ATTN_ATOL, ChunkState, assert_scores_close, assert_selection_matches,
                         bf16_t, check_needle_rows, needle_queries, spread_rows,
                         without_window_rows)

pytestmark = pytest.mark.gpu


def select(cs: ChunkState, tile: int):
    wl = cs.wl
    T, S = wl.chunk, cs.S
    tile_rows = T if tile == 0 else tile
    scratch = torch.empty((tile_rows, dsv4.dsv4_score_stride(S)), device="cuda")
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    ap = dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx, cs.w, T, cs.q_pos0,
                                  wl.idx_heads, wl.topk, idx, scratch, tile)
    torch.cuda.synchronize()
    del scratch
    return ap, idx


def gpu_scores(icache, q, w, q_pos0, S, rows, tile_rows):
    """fp32 GPU scores [len(rows), S] of the given chunk rows, each computed
    by dsv4_indexer_scores over the query tile that holds it (scores are
    bitwise independent of the launch shape)."""
    T = q.shape[0]
    buf = torch.empty((tile_rows, dsv4.dsv4_score_stride(S)), device="cuda")
    got = {}
    for t0 in range(0, T, tile_rows):
        t1 = min(T, t0 + tile_rows)
        rr = [r for r in rows if t0 <= r < t1]
        if not rr:
            continue
        dsv4.dsv4_indexer_scores(icache, q[t0:t1].contiguous(), w[t0:t1].contiguous(),
                                 q_pos0 + t0, buf[:t1 - t0])
        pick = torch.tensor([r - t0 for r in rr], device="cuda")
        g = buf.index_select(0, pick)[:, :S].cpu().numpy()
        for i, r in enumerate(rr):
            got[r] = g[i]
    del buf
    return np.stack([got[r] for r in rows])


def check_scores_and_selection(q, w, keys, q_pos0, S, topk, rows, g_scores, gidx):
    """Oracle scores of ``rows``; GPU scores within tolerance; the GPU's
    selection equal to the oracle's up to near ties, and bit-equal to the
    exact top-k of the GPU's own fp32 scores."""
    contiguous = rows == list(range(rows[0], rows[0] + len(rows)))
    if contiguous:
        ref = O.indexer_scores(q[rows[0]:rows[-1] + 1], w[rows[0]:rows[-1] + 1], keys,
                               q_pos0 + rows[0], S)
    for i, t in enumerate(rows):
        r = ref[i:i + 1] if contiguous else O.indexer_scores(q[t:t + 1], w[t:t + 1], keys,
                                                               q_pos0 + t, S)
        assert_scores_close(g_scores[i:i + 1], r)
        assert_selection_matches(gidx[t:t + 1], r, q_pos0 + t, topk)
        np.testing.assert_array_equal(
            gidx[t:t + 1], O.topk_select(g_scores[i:i + 1].astype(np.float64), q_pos0 + t, topk))


def attention(q_np, q_pos0, raw_t, raw_pos0, window, cache, idx, H, D):
    T = q_np.shape[0]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(bf16_t(q_np.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                  raw_t, raw_pos0, window, cache, idx, out)
    torch.cuda.synchronize()
    return out


def check_random_q_attention(g_out, rows, q, q_pos0, raw, raw_pos0, window, pooled, gidx, D):
    for i, t in enumerate(rows):
        ref = O.sparse_prefill_attention(q[t:t + 1], q_pos0 + t, raw, raw_pos0, window, pooled,
                                         gidx[t:t + 1], 1 / math.sqrt(D))
        err = np.abs(g_out[i] - ref[0]).max()
        assert err <= ATTN_ATOL, (t, err)


def check_chunk(cs: ChunkState, tile: int, rows, attn_rows, needle_rows):
    wl = cs.wl
    T, S, H, D, W = wl.chunk, cs.S, wl.heads, wl.head_dim, wl.window
    ap, idx = select(cs, tile)
    assert not ap
    # pooled rows appended by this chunk: bit-exact
    n_new = T // 4
    np.testing.assert_array_equal(cs.icache.rows[S - n_new:S].float().cpu().numpy(),
                                  cs.oracle_keys()[S - n_new:S])
    np.testing.assert_array_equal(cs.acache.rows[S - n_new:S].float().cpu().numpy(),
                                  cs.oracle_pooled()[S - n_new:S])
    tile_rows = T if tile == 0 else tile
    gidx = idx.cpu().numpy()
    g_scores = gpu_scores(cs.icache, cs.q_idx, cs.w, cs.q_pos0, S, rows, tile_rows)
    check_scores_and_selection(cs.inp["q_idx"], cs.inp["w"], cs.oracle_keys(), cs.q_pos0, S,
                               wl.topk, rows, g_scores, gidx)
    # attention with the workload's queries, fed the GPU's own selection
    pooled = cs.oracle_pooled()
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, cs.acache,
                                  idx, out)
    torch.cuda.synchronize()
    g = out[attn_rows].float().cpu().numpy()
    check_random_q_attention(g, attn_rows, cs.inp["q_attn"], cs.q_pos0, cs.inp["raw_kv"],
                             cs.raw_pos0, W, pooled, gidx, D)
    # needle queries on the same selection (less the pooled rows made of
    # window tokens): every 32-key group decisive
    scale = 1 / math.sqrt(D)
    nsel = without_window_rows(gidx, cs.q_pos0, W)
    qn = needle_queries(T, cs.q_pos0, H, W, cs.inp["raw_kv"], cs.raw_pos0, pooled, nsel, scale,
                        seed=1, rows=needle_rows)
    g = attention(qn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, cs.acache,
                  torch.from_numpy(nsel).cuda(), H, D)
    check_needle_rows(g[needle_rows].float().cpu().numpy(), needle_rows, qn, cs.q_pos0, W,
                      cs.inp["raw_kv"], cs.raw_pos0, pooled, nsel, scale)


def test_ctx4k_chunk2048_every_row():
    wl = SI.CTX_4K
    every = list(range(wl.chunk))
    check_chunk(ChunkState(wl), tile=0, rows=every, attn_rows=every,
                needle_rows=spread_rows(wl.chunk, 256, seed=4))


def test_ctx128k_chunk2048():
    wl = SI.CTX_128K
    rows = spread_rows(wl.chunk, 256, seed=128)
    check_chunk(ChunkState(wl), tile=0, rows=rows, attn_rows=rows,
                needle_rows=spread_rows(wl.chunk, 128, seed=129))


def test_ctx1m_chunk4096_tile1024():
    wl = SI.CTX_1M
    rows = spread_rows(wl.chunk, 64, tile=wl.tile_rows, seed=1024)
    assert len(rows) >= 64
    check_chunk(ChunkState(wl), tile=wl.tile_rows, rows=rows, attn_rows=rows, needle_rows=rows)


def test_ctx16k_eight_chunks_skip_then_full():
    """Eight 2,048-token chunks from an empty cache with k = 2,048: the first
    four take the all-pooled path (S = 512 .. 2,048 <= k, selections checked in
    full), the last four the full path: scores and selections of every row,
    attention of every row of the last chunk and of 128 spread rows of the
    others, with N(0,1) and with needle queries."""
    wl = SI.CTX_16K
    T, k, H, D, W = wl.chunk, wl.topk, wl.heads, wl.head_dim, wl.window
    scale = 1 / math.sqrt(D)
    seed = 0
    icache = dsv4.PoolCache(wl.capacity_rows, wl.idx_dim)
    acache = dsv4.PoolCache(wl.capacity_rows, wl.head_dim)
    ost = O.PoolingCacheState(wl.idx_dim, wl.capacity_rows)
    osa = O.PoolingCacheState(wl.head_dim, wl.capacity_rows)
    total = 8 * T
    keys_all = SI.as_bf16_values(SI.normal(seed, "idx_keys_stream", (total, wl.idx_dim)))
    kv_all = SI.as_bf16_values(SI.normal(seed, "kv_stream", (total, wl.head_dim)))
    keys_dev = torch.from_numpy(keys_all).to(torch.bfloat16).cuda()
    kv_dev = torch.from_numpy(kv_all).to(torch.bfloat16).cuda()
    every = list(range(T))
    for c in range(8):
        q_pos0 = c * T
        dsv4.dsv4_compress(icache, keys_dev[q_pos0:q_pos0 + T])
        dsv4.dsv4_compress(acache, kv_dev[q_pos0:q_pos0 + T])
        O.compress(ost, keys_all[q_pos0:q_pos0 + T])
        O.compress(osa, kv_all[q_pos0:q_pos0 + T])
        S = icache.n_rows
        assert S == acache.n_rows == (c + 1) * T // 4
        q = SI.as_bf16_values(SI.normal(seed, f"q_idx_chunk{c}", (T, wl.idx_heads, wl.idx_dim)))
        w = SI.uniform(seed, f"w_chunk{c}", (T, wl.idx_heads))
        q_d, w_d = torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(w).cuda()
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        scratch = torch.empty((T, dsv4.dsv4_score_stride(S)), device="cuda")
        ap = dsv4.dsv4_indexer_select(icache, acache.n_rows, q_d, w_d, T, q_pos0, wl.idx_heads,
                                      k, idx, scratch)
        torch.cuda.synchronize()
        gidx = idx.cpu().numpy()
        if c < 4:
            assert ap, f"chunk {c + 1} should take the all-pooled path"
            np.testing.assert_array_equal(gidx, O.all_pooled_selection(T, q_pos0, k))
            continue
        assert not ap
        # rows <= 32,768 columns: the select leaves the scores in its scratch
        g_scores = scratch[:, :S].cpu().numpy()
        check_scores_and_selection(q, w, ost.rows[:S], q_pos0, S, k, every, g_scores, gidx)
        # attention: the window reaches back into the previous chunk
        raw_pos0 = max(0, q_pos0 - W + 1)
        raw_np = kv_all[raw_pos0:q_pos0 + T]
        raw_t = kv_dev[raw_pos0:q_pos0 + T]
        pooled = osa.rows[:S]
        arows = every if c == 7 else spread_rows(T, 128, seed=c)
        qa = SI.as_bf16_values(SI.normal(seed, f"q_attn_chunk{c}", (T, H, D)))
        g = attention(qa, q_pos0, raw_t, raw_pos0, W, acache, idx, H, D)
        check_random_q_attention(g[arows].float().cpu().numpy(), arows, qa, q_pos0, raw_np,
                                 raw_pos0, W, pooled, gidx, D)
        nrows = spread_rows(T, 128, seed=100 + c)
        nsel = without_window_rows(gidx, q_pos0, W)
        qn = needle_queries(T, q_pos0, H, W, raw_np, raw_pos0, pooled, nsel, scale, seed=c,
                            rows=nrows)
        g = attention(qn, q_pos0, raw_t, raw_pos0, W, acache, torch.from_numpy(nsel).cuda(), H, D)
        check_needle_rows(g[nrows].float().cpu().numpy(), nrows, qn, q_pos0, W, raw_np,
                          raw_pos0, pooled, nsel, scale)
    np.testing.assert_array_equal(icache.rows[:icache.n_rows].float().cpu().numpy(),
                                  ost.rows[:ost.n_rows])
    np.testing.assert_array_equal(acache.rows[:acache.n_rows].float().cpu().numpy(),
                                  osa.rows[:osa.n_rows])


def test_ctx128k_needles_at_topk_4096():
    """The largest selection (k = 4,096, 132 key groups per query, so two or
    three needles per head) over the 128K attention cache, every query of
    the chunk in one launch, through both attention entry points."""
    wl = SI.CTX_128K
    cs = ChunkState(wl, with_attn_q=False)
    T, S, H, D, W, k = wl.chunk, cs.S, wl.heads, wl.head_dim, wl.window, 4096
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(4096)
    sel = np.empty((T, k), np.int32)
    for t in range(T):   # rows older than the window (see without_window_rows)
        old = (cs.q_pos0 + t - W + 1 + 3) // 4
        sel[t] = np.sort(rng.choice(old, size=k, replace=False))
    rows = spread_rows(T, 64, seed=40)
    pooled = cs.oracle_pooled()
    qn = needle_queries(T, cs.q_pos0, H, W, cs.inp["raw_kv"], cs.raw_pos0, pooled, sel, scale,
                        seed=41, rows=rows)
    seld = torch.from_numpy(sel).cuda()
    g = attention(qn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, cs.acache, seld, H, D)
    check_needle_rows(g[rows].float().cpu().numpy(), rows, qn, cs.q_pos0, W, cs.inp["raw_kv"],
                      cs.raw_pos0, pooled, sel, scale)
    # the key-split entry point on four of the queries, its planned split count
    sub = rows[len(rows) // 2:len(rows) // 2 + 4]
    q4 = bf16_t(qn[sub].reshape(4, H * D)).cuda().view(4, H, D)
    for j, t in enumerate(sub):
        ns, nb = dsv4.dsv4_sparse_attn_narrow_plan(1, H, D, W, k)
        assert ns > 1
        ws = torch.empty(nb // 4, device="cuda")
        out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
        p = cs.q_pos0 + t
        dsv4.dsv4_sparse_attn_narrow(q4[j:j + 1].contiguous(), p, cs.raw_kv, cs.raw_pos0, W,
                                     cs.acache, seld[t:t + 1].contiguous(), out, ns, ws)
        torch.cuda.synchronize()
        check_needle_rows(out.float().cpu().numpy(), [0], qn[t:t + 1], p, W, cs.inp["raw_kv"],
                          cs.raw_pos0, pooled, sel[t:t + 1], scale)


# ---------------------------------------------------------------- sibling modes and narrow steps
# The same launch configurations bench.py times: the 2,048-row chunk at 128K
# context in the window-only and ratio-128 modes, and T = 1-4 query rows at
# the end of a context.

def test_ctx128k_chunk2048_local_and_ratio128_modes():
    wl = SI.CTX_128K
    cs = ChunkState(wl)
    T, H, D, W = wl.chunk, wl.heads, wl.head_dim, wl.window
    scale = 1 / math.sqrt(D)
    rows = spread_rows(T, 64, seed=3)
    # window only: N(0,1) queries and needles (4 groups of 32 window keys)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, None, None, out)
    torch.cuda.synchronize()
    g = out[rows].float().cpu().numpy()
    for i, t in enumerate(rows):
        ref = O.sparse_prefill_attention(cs.inp["q_attn"][t:t + 1], cs.q_pos0 + t, cs.inp["raw_kv"],
                                         cs.raw_pos0, W, None, None, scale)
        assert np.abs(g[i] - ref[0]).max() <= ATTN_ATOL, ("local", t)
    qn = needle_queries(T, cs.q_pos0, H, W, cs.inp["raw_kv"], cs.raw_pos0, None, None, scale,
                        seed=5, rows=rows)
    g = attention(qn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, None, None, H, D)
    check_needle_rows(g[rows].float().cpu().numpy(), rows, qn, cs.q_pos0, W, cs.inp["raw_kv"],
                      cs.raw_pos0, None, None, scale)
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
    # needles over every visible ratio-128 row (about 1,150 keys, 36 groups)
    nrows = rows[::2]
    qn = needle_queries(T, cs.q_pos0, H, W, cs.inp["raw_kv"], cs.raw_pos0, st.rows[:S], None,
                        scale, seed=6, ratio=128, rows=nrows)
    g = attention(qn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, W, c128, None, H, D)
    check_needle_rows(g[nrows].float().cpu().numpy(), nrows, qn, cs.q_pos0, W, cs.inp["raw_kv"],
                      cs.raw_pos0, st.rows[:S], None, scale, ratio=128)


@pytest.mark.parametrize("wl,T", [(SI.CTX_128K, 4), (SI.CTX_1M, 2)], ids=["ctx128k-T4", "ctx1m-T2"])
def test_narrow_steps_at_end_of_context(wl, T):
    """T query rows at the last positions the caches cover, as bench.py's
    narrow section runs them: indexer select with the scratch
    dsv4_indexer_scratch_bytes sizes (the chunk-parallel top-k at 1M), then
    the key-split attention with its planned split count (34 splits of the
    2,176 keys), with N(0,1) and with needle queries.  Every row is
    checked."""
    cs = ChunkState(wl)
    S = cs.S
    H, D, W, k = wl.heads, wl.head_dim, wl.window, wl.topk
    scale = 1 / math.sqrt(D)
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
                                       cs.oracle_pooled(), gidx, scale)
    err = np.abs(out.float().cpu().numpy() - ref_o).max()
    assert err <= ATTN_ATOL, err
    nsel = without_window_rows(gidx, q0, W)
    qn = needle_queries(T, q0, H, W, raw_np, raw_lo, cs.oracle_pooled(), nsel, scale, seed=7)
    dsv4.dsv4_sparse_attn_narrow(bf16_t(qn.reshape(T, H * D)).cuda().view(T, H, D), q0, raw,
                                 raw_lo, W, cs.acache, torch.from_numpy(nsel).cuda(), out, ns, ws)
    torch.cuda.synchronize()
    check_needle_rows(out.float().cpu().numpy(), list(range(T)), qn, q0, W, raw_np, raw_lo,
                      cs.oracle_pooled(), nsel, scale)
