"""GPU parity of the HIP path (called through the C ABI) against the CPU oracle.

Sizes are chosen so the oracle finishes in seconds while still spanning
several kernel tiles and a ragged tail; the full-size workloads are checked on
sampled rows in test_gpu_fullsize.py.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import (ATTN_ATOL, ChunkState, assert_scores_close, assert_selection_matches,
                         bf16_t)

pytestmark = pytest.mark.gpu



# ====================================================================== compressor

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_compress_golden_10_tokens(dtype):
    """Page 1, Correctness: 10 tokens at ratio 4 -> 2 pooled rows + 2-token remainder."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((10, 64)).astype(np.float32)
    if dtype == torch.bfloat16:
        x = SI.as_bf16_values(x)
    cache = dsv4.PoolCache(8, 64, dtype=dtype)
    dsv4.dsv4_compress(cache, torch.from_numpy(x).to(dtype).cuda())
    st = O.PoolingCacheState(64, 8, out_bf16=(dtype == torch.bfloat16))
    O.compress(st, x)
    torch.cuda.synchronize()
    assert cache.n_rows == 2 and cache.n_rem == 2
    np.testing.assert_array_equal(cache.rows[:2].float().cpu().numpy(), st.rows[:2])
    np.testing.assert_array_equal(cache.rem[:2].float().cpu().numpy(), x[8:10])


@pytest.mark.parametrize("dim", [128, 512])
def test_compress_any_split_is_bit_exact(dim):
    rng = np.random.default_rng(dim)
    n = 203
    x = SI.as_bf16_values(rng.standard_normal((n, dim)).astype(np.float32) * 3)
    ref = O.PoolingCacheState(dim, 64)
    O.compress(ref, x)
    xd = bf16_t(x).cuda()
    splits = [[n], [1] * 9 + [n - 9], [3, 5, 7, 11, 13, 17, 19, 128], [2, 0, 2, 0, 199]]
    for _ in range(6):
        cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(1, 12)))
        splits.append(list(np.diff(np.concatenate([[0], cuts, [n]]))))
    for parts in splits:
        c = dsv4.PoolCache(64, dim)
        pos = 0
        for p in parts:
            dsv4.dsv4_compress(c, xd[pos:pos + p])
            pos += p
        torch.cuda.synchronize()
        assert (c.n_rows, c.n_rem) == (ref.n_rows, ref.n_rem) == (50, 3)
        np.testing.assert_array_equal(c.rows[:50].float().cpu().numpy(), ref.rows[:50])
        np.testing.assert_array_equal(c.rem[:3].float().cpu().numpy(), ref.rem)


def test_compress_capacity_error_leaves_device_and_host_state():
    c = dsv4.PoolCache(2, 32)
    x = bf16_t(np.ones((9, 32), np.float32)).cuda()
    dsv4.dsv4_compress(c, x[:6])
    torch.cuda.synchronize()
    snap = c.rows.clone(), c.rem.clone()
    with pytest.raises(dsv4.DSV4Error) as e:
        dsv4.dsv4_compress(c, x[:7])        # 2 + 7 = 9 -> 2 more rows > capacity
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert (c.n_rows, c.n_rem) == (1, 2)
    assert torch.equal(c.rows, snap[0]) and torch.equal(c.rem, snap[1])


# ====================================================================== path decision

def test_select_all_pooled_and_empty_paths():
    """Page 1, Summary/Correctness: all-pooled skip selects sequential indices
    without reading q or w; empty pools keep the full path (all slots empty)."""
    T, topk = 41, 16
    for S_tokens in (0, 3, 10, 64):
        c = dsv4.PoolCache(32, 128)
        if S_tokens:
            dsv4.dsv4_compress(c, bf16_t(np.ones((S_tokens, 128), np.float32)).cuda())
        S = c.n_rows
        q_pos0 = max(0, 4 * S + c.n_rem - T)
        T_eff = min(T, 4 * S + c.n_rem - q_pos0)
        out = torch.full((T_eff, topk), 123, dtype=torch.int32, device="cuda")
        ap = dsv4.dsv4_indexer_select(c, S, None, None, T_eff, q_pos0, 64, topk, out)
        torch.cuda.synchronize()
        want, want_ap = O.indexer_select(None, None, None, S, T_eff, q_pos0, topk, S)
        assert ap == want_ap == (S > 0)
        np.testing.assert_array_equal(out.cpu().numpy(), want)


def test_select_row_guard():
    c = dsv4.PoolCache(32, 128)
    dsv4.dsv4_compress(c, bf16_t(np.ones((40, 128), np.float32)).cuda())
    out = torch.zeros((8, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(dsv4.DSV4Error) as e:
        dsv4.dsv4_indexer_select(c, 9, None, None, 8, 32, 64, 8, out)
    assert e.value.code == -4


# ====================================================================== scores

def _score_case(T, S_tokens, q_pos0_back, heads, dim, seed):
    rng = np.random.default_rng(seed)
    c = dsv4.PoolCache(S_tokens // 4 + 1, dim)
    raw = SI.as_bf16_values(rng.standard_normal((S_tokens, dim)).astype(np.float32))
    dsv4.dsv4_compress(c, bf16_t(raw).cuda())
    st = O.PoolingCacheState(dim, S_tokens // 4 + 1)
    O.compress(st, raw)
    S = c.n_rows
    q_pos0 = S_tokens - q_pos0_back
    q = SI.as_bf16_values(rng.standard_normal((T, heads, dim)).astype(np.float32))
    w = (rng.random((T, heads)).astype(np.float32) * 1.5 - 0.25).astype(np.float32)
    return c, st, S, q_pos0, q, w


@pytest.mark.parametrize("T,S_tokens,back,heads,dim", [
    (64, 64, 64, 4, 32),        # tiny case shape: 4 heads x 32, 16 pooled rows
    (203, 2811, 203, 64, 128),  # ragged rows and columns, masked tail
    (77, 1500, 300, 40, 64),    # two partly filled head tiles
    (16, 9000, 16, 33, 128),
    # many query blocks, few key tiles: one XCD column group with two splits, then
    # one split; longer key ranges: two and four column groups
    (2048, 2600, 2048, 16, 64),
    (4096, 5000, 4096, 8, 32),
    (2048, 9000, 2048, 4, 32),
    (1024, 16400, 1024, 4, 32),
])
def test_scores_match_oracle_and_fold_equals_second_pass(T, S_tokens, back, heads, dim):
    _check_scores(T, S_tokens, back, heads, dim, seed=T + S_tokens)


@pytest.mark.parametrize("case", range(16))
def test_scores_random_shapes_match_oracle(case):
    """Seeded random shapes over every kernel variant (head counts 1-64 in one
    or two 32-head tiles, dims 32/64/128), 1 to 2,048 query rows and up to
    3,000 pooled rows, so that the launch takes one to eight XCD column groups,
    one or many splits per group, and splits that start past the last key."""
    rng = np.random.default_rng(5000 + case)
    heads = int(rng.choice([1, 4, 16, 33, 40, 64]))
    dim = int(rng.choice([32, 64, 128]))
    while True:
        T = int(np.exp(rng.uniform(0.0, np.log(2048.0))))  # log-uniform, 1 .. 2,047
        S_tokens = int(rng.integers(max(T, 16), 12001))
        if T * (S_tokens // 4) * heads * dim <= 2.5e9:  # oracle time
            break
    back = int(rng.integers(T, min(S_tokens, T + 3000) + 1))
    _check_scores(T, S_tokens, back, heads, dim, seed=6000 + case)


def test_scores_bitwise_independent_of_launch_shape():
    """A row's scores are the same bits whichever call computes them: a 2,048-row
    launch (few long splits), sub-ranges of 1, 64, 1,000 and 48 rows (more, shorter
    splits and other XCD column groups) and the rows one call at a time for a few."""
    T, S_tokens, heads, dim = 2048, 36000, 64, 128
    c, st, S, q_pos0, q, w = _score_case(T, S_tokens, T, heads, dim, seed=424242)
    stride = dsv4.dsv4_score_stride(S)
    qd, wd = bf16_t(q).cuda(), torch.from_numpy(w).cuda()
    full = torch.empty((T, stride), device="cuda")
    dsv4.dsv4_indexer_scores(c, qd, wd, q_pos0, full)
    ranges = [(0, 1), (0, 64), (100, 1100), (2000, 2048), (777, 778), (1999, 2000)]
    parts = []
    for a, b in ranges:
        out = torch.empty((b - a, stride), device="cuda")
        dsv4.dsv4_indexer_scores(c, qd[a:b].contiguous(), wd[a:b].contiguous(), q_pos0 + a, out)
        parts.append(out)
    torch.cuda.synchronize()
    f = full[:, :S].cpu().numpy().view(np.uint32)
    for (a, b), out in zip(ranges, parts):
        assert np.array_equal(out[:, :S].cpu().numpy().view(np.uint32), f[a:b]), (a, b)


def _check_scores(T, S_tokens, back, heads, dim, seed):
    c, st, S, q_pos0, q, w = _score_case(T, S_tokens, back, heads, dim, seed=seed)
    stride = dsv4.dsv4_score_stride(S)
    folded = torch.full((T, stride), 7.0, device="cuda")
    raw = torch.full((T, stride), 7.0, device="cuda")
    qd, wd = bf16_t(q).cuda(), torch.from_numpy(w).cuda()
    dsv4.dsv4_indexer_scores(c, qd, wd, q_pos0, folded, fold_mask=True)
    dsv4.dsv4_indexer_scores(c, qd, wd, q_pos0, raw, fold_mask=False)
    torch.cuda.synchronize()
    g_fold = folded.cpu().numpy()
    g_raw = raw.cpu().numpy()
    assert np.all(g_fold[:, S:] == 7.0) and np.all(g_raw[:, S:] == 7.0)  # nothing past S
    ref = O.indexer_scores(q, w, st.rows[:S], q_pos0, S, fold_mask=True)
    assert_scores_close(g_fold[:, :S], ref)
    assert_scores_close(g_raw[:, :S], O.indexer_scores(q, w, st.rows[:S], q_pos0, S, fold_mask=False))
    # page 2, commit 5 / review: second-pass mask with the same sentinel is bit-identical
    second = O.apply_pooled_mask(g_raw[:, :S].astype(np.float64), q_pos0).astype(np.float32)
    assert np.array_equal(second.view(np.uint32), g_fold[:, :S].view(np.uint32))


# ====================================================================== top-k

def _topk_gpu(scores_np, q_pos0, n_cols, topk, stride=None):
    rows, width = scores_np.shape
    stride = stride or width
    buf = np.zeros((rows, stride), np.float32)
    buf[:, :width] = scores_np
    d = torch.from_numpy(buf).cuda()
    out = torch.full((rows, topk), 99, dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select(d, q_pos0, n_cols, topk, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "signed_zero", "constant"])
@pytest.mark.parametrize("topk", [1, 7, 64, 512])
def test_topk_exact_on_given_scores(kind, topk):
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{topk}".encode()))
    rows, q_pos0 = 37, 1900
    n_cols = (q_pos0 + rows) // 4
    if kind == "normal":
        s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(-5, 6, size=(rows, n_cols)).astype(np.float32)
    elif kind == "zeros":
        s = np.where(rng.random((rows, n_cols)) < 0.9, 0.0, rng.random((rows, n_cols))).astype(np.float32)
    elif kind == "signed_zero":
        s = np.where(rng.random((rows, n_cols)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        s[:, ::97] = 1.0
    else:
        s = np.full((rows, n_cols), 2.5, np.float32)
    for t in range(rows):  # garbage beyond the visible prefix must be ignored
        s[t, O.visible_rows(q_pos0 + t):] = np.float32(1e30)
    got = _topk_gpu(s, q_pos0, n_cols, topk)
    want = O.topk_select(s.astype(np.float64), q_pos0, topk)
    np.testing.assert_array_equal(got, want)


def test_topk_unaligned_stride_and_short_rows():
    rng = np.random.default_rng(3)
    rows, q_pos0, topk = 50, 0, 8   # rows see 0..12 pooled rows: k > visible for most
    n_cols = 13
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    got = _topk_gpu(s, q_pos0, n_cols, topk, stride=13)   # stride not a multiple of 4
    np.testing.assert_array_equal(got, O.topk_select(s.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("topk", [2048, 4096])
def test_topk_multi_chunk_rows(topk):
    """Rows longer than one LDS chunk (tournament over chunks)."""
    rng = np.random.default_rng(topk)
    rows, q_pos0 = 6, 4 * 70000
    n_cols = (q_pos0 + rows) // 4
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    s[1] = rng.integers(0, 50, size=n_cols).astype(np.float32)   # heavy ties across chunks
    s[2, :] = 1.0
    s[3] = np.abs(s[3])
    s[3, ::5] = 0.0
    got = _topk_gpu(s, q_pos0, n_cols, topk)
    np.testing.assert_array_equal(got, O.topk_select(s.astype(np.float64), q_pos0, topk))


# ====================================================================== indexer select

def test_select_full_path_tiled_equals_untiled_and_oracle():
    c, st, S, q_pos0, q, w = _score_case(300, 6000, 300, 64, 128, seed=21)
    topk = 256
    qd, wd = bf16_t(q).cuda(), torch.from_numpy(w).cuda()
    results = {}
    for tile in (0, 1, 64, 100, 299, 512):
        rows = 300 if tile == 0 else min(tile, 300)
        scratch = torch.empty(dsv4.dsv4_indexer_scratch_bytes(rows, S) // 4, device="cuda")
        out = torch.full((300, topk), 5, dtype=torch.int32, device="cuda")
        ap = dsv4.dsv4_indexer_select(c, S, qd, wd, 300, q_pos0, 64, topk, out, scratch, tile)
        assert not ap
        torch.cuda.synchronize()
        results[tile] = out.cpu().numpy()
    for tile, r in results.items():
        assert np.array_equal(r, results[0]), f"tile {tile} differs from untiled"
    ref = O.indexer_scores(q, w, st.rows[:S], q_pos0, S)
    assert_selection_matches(results[0], ref, q_pos0, topk)


def test_select_gpu_choice_is_exact_topk_of_gpu_scores():
    c, st, S, q_pos0, q, w = _score_case(130, 4000, 130, 64, 128, seed=5)
    topk = 300
    qd, wd = bf16_t(q).cuda(), torch.from_numpy(w).cuda()
    stride = dsv4.dsv4_score_stride(S)
    scratch = torch.empty((130, stride), device="cuda")
    out = torch.empty((130, topk), dtype=torch.int32, device="cuda")
    dsv4.dsv4_indexer_select(c, S, qd, wd, 130, q_pos0, 64, topk, out, scratch)
    torch.cuda.synchronize()
    g_scores = scratch.cpu().numpy()[:, :S].astype(np.float64)
    np.testing.assert_array_equal(out.cpu().numpy(), O.topk_select(g_scores, q_pos0, topk))


# ====================================================================== attention

def _attn_case(T, q_pos0, H, D, W, topk, seed, sel_mode="random"):
    rng = np.random.default_rng(seed)
    S_tokens = q_pos0 + T
    S = S_tokens // 4
    pooled = SI.as_bf16_values(rng.standard_normal((S, D)).astype(np.float32) * 0.5)
    cache = dsv4.PoolCache(S + 3, D)
    cache.rows[:S].copy_(bf16_t(pooled))
    cache.set_state(S, S_tokens - 4 * S)
    raw_pos0 = max(0, q_pos0 - W + 1)
    raw = SI.as_bf16_values(rng.standard_normal((q_pos0 + T - raw_pos0, D)).astype(np.float32))
    q = SI.as_bf16_values(rng.standard_normal((T, H, D)).astype(np.float32))
    sel = None
    if sel_mode == "random":
        sel = np.full((T, topk), -1, np.int32)
        for t in range(T):
            v = O.visible_rows(q_pos0 + t)
            k = min(topk, v)
            sel[t, :k] = np.sort(rng.choice(v, size=k, replace=False)) if v else []
        # decoys the kernel must ignore: empty slots inside, rows beyond visibility
        sel[::3, 0] = -1
        if topk > 2:
            sel[1::4, topk - 1] = S - 1
    return cache, pooled, raw, raw_pos0, q, sel


@pytest.mark.parametrize("T,q_pos0,H,D,W,topk", [
    (64, 0, 4, 32, 16, 8),        # tiny case shape (16-token window, 16 pooled rows)
    (37, 900, 64, 512, 128, 64),  # full head shape, ragged tile tail
    (20, 3000, 64, 512, 128, 200),
    (45, 150, 24, 128, 40, 32),   # partial head tile
    (9, 60, 64, 256, 1, 16),      # window of one token
])
def test_attention_matches_oracle(T, q_pos0, H, D, W, topk):
    cache, pooled, raw, raw_pos0, q, sel = _attn_case(T, q_pos0, H, D, W, topk, seed=T * 7 + D)
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                  bf16_t(raw).cuda(), raw_pos0, W, cache,
                                  torch.from_numpy(sel).cuda(), out)
    torch.cuda.synchronize()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= ATTN_ATOL, err


def test_attention_null_selection_and_trimmed_raw_buffer_bitwise():
    T, q_pos0, H, D, W = 30, 500, 64, 512, 128
    cache, pooled, raw, raw_pos0, q, _ = _attn_case(T, q_pos0, H, D, W, 0, seed=4, sel_mode="none")
    S = cache.n_rows
    qd = bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D)
    seq = O.all_pooled_selection(T, q_pos0, S + 7)
    outs = []
    for sel in (None, torch.from_numpy(seq).cuda()):
        o = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
        dsv4.dsv4_sparse_prefill_attn(qd, q_pos0, bf16_t(raw).cuda(), raw_pos0, W, cache, sel, o)
        outs.append(o)
    # raw buffer with 50 older rows in front (a trimmed cache seen from further back)
    rng = np.random.default_rng(9)
    older = SI.as_bf16_values(rng.standard_normal((50, D)).astype(np.float32))
    o = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(qd, q_pos0, bf16_t(np.concatenate([older, raw])).cuda(),
                                  raw_pos0 - 50, W, cache, None, o)
    outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, None, 1 / math.sqrt(D))
    assert np.abs(outs[0].float().cpu().numpy() - ref).max() <= ATTN_ATOL


def test_attention_is_deterministic():
    T, q_pos0, H, D, W, topk = 16, 2000, 64, 512, 128, 128
    cache, pooled, raw, raw_pos0, q, sel = _attn_case(T, q_pos0, H, D, W, topk, seed=11)
    qd = bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D)
    outs = []
    for _ in range(3):
        o = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
        dsv4.dsv4_sparse_prefill_attn(qd, q_pos0, bf16_t(raw).cuda(), raw_pos0, W, cache,
                                      torch.from_numpy(sel).cuda(), o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


# ====================================================================== tiny workload end to end

def test_tiny_workload_end_to_end():
    """64-token prefill from an empty cache (4 indexer heads x 32, k 8,
    attention H 4, D 32, window 16), inputs rounded to bf16 on both sides."""
    wl = SI.TINY
    cs = ChunkState(wl)
    S = cs.S
    assert S == 16
    out = torch.empty((wl.chunk, wl.topk), dtype=torch.int32, device="cuda")
    scratch = torch.empty((wl.chunk, dsv4.dsv4_score_stride(S)), device="cuda")
    ap = dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx, cs.w, wl.chunk,
                                  cs.q_pos0, wl.idx_heads, wl.topk, out, scratch)
    attn = torch.empty((wl.chunk, wl.heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(cs.q_attn, cs.q_pos0, cs.raw_kv, cs.raw_pos0, wl.window,
                                  cs.acache, out, attn)
    torch.cuda.synchronize()
    assert not ap   # 16 pooled rows > k = 8: full path
    np.testing.assert_array_equal(cs.icache.rows[:S].float().cpu().numpy(), cs.oracle_keys())
    np.testing.assert_array_equal(cs.acache.rows[:S].float().cpu().numpy(), cs.oracle_pooled())
    ref_scores = O.indexer_scores(cs.inp["q_idx"], cs.inp["w"], cs.oracle_keys(), cs.q_pos0, S)
    assert_scores_close(scratch.cpu().numpy()[:, :S], ref_scores)
    gsel = out.cpu().numpy()
    assert_selection_matches(gsel, ref_scores, cs.q_pos0, wl.topk)
    ref = O.sparse_prefill_attention(cs.inp["q_attn"], cs.q_pos0, cs.inp["raw_kv"], cs.raw_pos0,
                                     wl.window, cs.oracle_pooled(), gsel,
                                     1 / math.sqrt(wl.head_dim))
    assert np.abs(attn.float().cpu().numpy() - ref).max() <= ATTN_ATOL


def test_topk_constant_rows_between_ordinary_rows():
    """A row whose visible scores are all equal (a zero query or zero head
    weights give such a row of zeros) followed, in the same persistent
    workgroup, by ordinary rows longer than 4,096 columns: every row must
    still be the oracle's selection (each workgroup takes rows g, g + 256, ...
    of a 2,048-row tile)."""
    rng = np.random.default_rng(44)
    rows, q_pos0, topk = 1024, 4 * 30000, 2048
    n_cols = (q_pos0 + rows) // 4
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    s[::3] = 0.0                       # every third row constant (ties everywhere)
    s[1::7] = np.float32(-2.5)
    got = _topk_gpu(s, q_pos0, n_cols, topk)
    np.testing.assert_array_equal(got, O.topk_select(s.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("levels", [40, 10, 3])
def test_topk_tie_heavy_long_rows(levels):
    """Single-chunk rows of 30,000 columns holding only `levels` distinct
    values: the threshold bin holds ~30,000/levels keys, so the finish takes
    the one-wave bit-by-bit path (40 levels) or further histogram passes
    (10, 3); several rows share each persistent workgroup."""
    rng = np.random.default_rng(levels)
    rows, q_pos0, topk = 600, 4 * 30000, 2048
    n_cols = (q_pos0 + rows) // 4
    s = rng.integers(0, levels, size=(rows, n_cols)).astype(np.float32) - levels / 2
    got = _topk_gpu(s, q_pos0, n_cols, topk)
    np.testing.assert_array_equal(got, O.topk_select(s.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("T,q_pos0,W,topk", [
    (70, 0, 128, 2048),   # the stream's first tokens: clipped window, 0-17 pooled rows
    (1, 5000, 128, 4096), # the largest k, more slots than visible rows (1,250)
    (5, 130, 128, 1),     # a single slot
    (3, 10, 1, 64),       # a one-token window, mostly empty selections
    (33, 127, 128, 64),   # the first query whose window is full, ragged tile tail
])
def test_attention_hot_shape_edges(T, q_pos0, W, topk):
    """The H = 64, D = 512 shape at its edges: positions from 0, windows cut
    at the stream start, k = 1 and k = DSV4_MAX_TOPK, selections mostly empty
    (every slot a query cannot see is -1 or a decoy row beyond visibility)."""
    H, D = 64, 512
    cache, pooled, raw, raw_pos0, q, sel = _attn_case(T, q_pos0, H, D, W, topk,
                                                      seed=9000 + T + q_pos0 + topk)
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                  bf16_t(raw).cuda(), raw_pos0, W, cache,
                                  torch.from_numpy(sel).cuda(), out)
    torch.cuda.synchronize()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= ATTN_ATOL, err


def test_attention_unsorted_and_duplicate_selections():
    """Selections the indexer never makes but the ABI accepts: slots in
    descending order and repeated rows.  Each listed slot is a key, as in the
    definition (a row listed twice is attended twice)."""
    T, q_pos0, H, D, W, topk = 12, 2000, 64, 512, 128, 96
    cache, pooled, raw, raw_pos0, q, sel = _attn_case(T, q_pos0, H, D, W, topk, seed=77)
    sel = sel[:, ::-1].copy()                 # descending, -1 slots first
    sel[:, 5] = sel[:, 6]                     # a repeated row in every query
    sel[3, :] = sel[3, 7]                     # one query: a single row, topk times
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                  bf16_t(raw).cuda(), raw_pos0, W, cache,
                                  torch.from_numpy(sel).cuda(), out)
    torch.cuda.synchronize()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    assert np.abs(out.float().cpu().numpy() - ref).max() <= ATTN_ATOL


@pytest.mark.parametrize("case", range(12))
def test_attention_random_shapes_match_oracle(case):
    """Seeded random attention shapes: heads (1-64, partial head tiles), head
    dims 32-512, windows 1-256, k 1-600, positions from the first tokens to a
    few thousand, selections with empty and invisible slots; the per-query
    kernel and the key-split path (random split count) against the oracle."""
    rng = np.random.default_rng(3000 + case)
    T = int(rng.integers(1, 24))
    H = int(rng.choice([1, 7, 16, 33, 64]))
    D = int(rng.choice([32, 64, 128, 256, 512]))
    W = int(rng.choice([1, 16, 128, 256]))
    topk = int(rng.choice([1, 8, 64, 600]))
    q_pos0 = int(rng.choice([0, 5, int(rng.integers(40, 600)), int(rng.integers(600, 5000))]))
    cache, pooled, raw, raw_pos0, q, sel = _attn_case(T, q_pos0, H, D, W, topk, seed=4000 + case)
    qd = bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D)
    rawd, seld = bf16_t(raw).cuda(), torch.from_numpy(sel).cuda()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(qd, q_pos0, rawd, raw_pos0, W, cache, seld, out)
    ns = int(rng.integers(1, 9))
    ws = torch.empty(T * ns * H * (D + 2), device="cuda")  # (m, l, O) of every split
    out2 = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_attn_narrow(qd, q_pos0, rawd, raw_pos0, W, cache, seld, out2, ns, ws)
    torch.cuda.synchronize()
    for o in (out, out2):
        err = np.abs(o.float().cpu().numpy() - ref).max()
        assert err <= ATTN_ATOL, (case, err)
