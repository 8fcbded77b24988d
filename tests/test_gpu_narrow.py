"""GPU parity of the narrow-query steps (T = 1-4: decode, draft verification,
q2-q4 prefill bands) against the CPU oracle, through the C ABI: the indexer
select at narrow T, and the key-split attention (each query's key tiles over
several workgroups, merged by a second kernel) in the three attention modes,
with planned and explicit split counts, including more splits than tiles.

Attention outputs: max |gpu - ref| <= 2e-2 against the fp64 oracle, the bar
of the prefill kernel.  Selections: exact (same rules as the prefill tests).
"""
import math

import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import ATTN_ATOL, bf16_t

pytestmark = pytest.mark.gpu


def _case(T, q_pos0, H, D, W, topk, seed, ratio=4, mode="sel"):
    rng = np.random.default_rng(seed)
    raw_pos0 = max(0, q_pos0 - W + 1)
    raw = SI.as_bf16_values(rng.standard_normal((q_pos0 + T - raw_pos0, D)).astype(np.float32))
    q = SI.as_bf16_values(rng.standard_normal((T, H, D)).astype(np.float32))
    cache = pooled = sel = None
    if mode != "local":
        S = (q_pos0 + T) // ratio
        pooled = SI.as_bf16_values(rng.standard_normal((S, D)).astype(np.float32) * 0.5)
        cache = dsv4.PoolCache(S + 1, D, ratio=ratio)
        cache.rows[:S].copy_(bf16_t(pooled))
        cache.set_state(S, (q_pos0 + T) - ratio * S)
    if mode == "sel":
        sel = np.full((T, topk), -1, np.int32)
        for t in range(T):
            v = O.visible_rows(q_pos0 + t, ratio)
            k = min(topk, v)
            sel[t, :k] = np.sort(rng.choice(v, size=k, replace=False))
        sel[:, 1] = -1          # an empty slot inside every row
    return q, raw, raw_pos0, cache, pooled, sel


def _narrow(q, q_pos0, raw, raw_pos0, W, cache, sel, n_splits):
    T, H, D = q.shape
    ws_bytes = T * n_splits * H * (D + 2) * 4
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda") if n_splits > 1 else None
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_attn_narrow(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                 bf16_t(raw).cuda(), raw_pos0, W, cache,
                                 None if sel is None else torch.from_numpy(sel).cuda(), out,
                                 n_splits, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("splits", ["plan", 1, 3, 64])
def test_narrow_indexed_attention_matches_oracle(T, splits):
    q_pos0, H, D, W, topk = 5000, 64, 512, 128, 512
    q, raw, raw_pos0, cache, pooled, sel = _case(T, q_pos0, H, D, W, topk, seed=T)
    ns = dsv4.dsv4_sparse_attn_narrow_plan(T, H, D, W, topk)[0] if splits == "plan" else splits
    got = _narrow(q, q_pos0, raw, raw_pos0, W, cache, sel, ns)
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    err = np.abs(got - ref).max()
    assert err <= ATTN_ATOL, (ns, err)


@pytest.mark.parametrize("T,splits", [(1, "plan"), (1, 3), (3, 8), (4, 64)])
def test_narrow_local_attention_matches_oracle(T, splits):
    # window 128 = 4 tiles: 8 and 64 splits leave most splits empty
    q_pos0, H, D, W = 700, 64, 512, 128
    q, raw, raw_pos0, _, _, _ = _case(T, q_pos0, H, D, W, 0, seed=10 + T, mode="local")
    ns = dsv4.dsv4_sparse_attn_narrow_plan(T, H, D, W, 0)[0] if splits == "plan" else splits
    got = _narrow(q, q_pos0, raw, raw_pos0, W, None, None, ns)
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, None, None, 1 / math.sqrt(D))
    assert np.abs(got - ref).max() <= ATTN_ATOL


@pytest.mark.parametrize("T", [1, 4])
def test_narrow_compressed_attention_matches_oracle(T):
    q_pos0, H, D, W = 128 * 300 + 7, 64, 512, 128
    q, raw, raw_pos0, cache, pooled, _ = _case(T, q_pos0, H, D, W, 0, seed=20 + T, ratio=128,
                                               mode="all")
    ns = dsv4.dsv4_sparse_attn_narrow_plan(T, H, D, W, cache.n_rows)[0]
    assert ns > 1
    got = _narrow(q, q_pos0, raw, raw_pos0, W, cache, None, ns)
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, None,
                                     1 / math.sqrt(D), ratio=128)
    assert np.abs(got - ref).max() <= ATTN_ATOL


def test_narrow_attention_small_heads_and_dims():
    # partial head tile and a head dim the prefill kernel splits once
    T, q_pos0, H, D, W, topk = 2, 900, 24, 128, 40, 64
    q, raw, raw_pos0, cache, pooled, sel = _case(T, q_pos0, H, D, W, topk, seed=31)
    got = _narrow(q, q_pos0, raw, raw_pos0, W, cache, sel, 5)
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    assert np.abs(got - ref).max() <= ATTN_ATOL


def test_narrow_attention_is_deterministic_and_checks_workspace():
    T, q_pos0, H, D, W, topk = 4, 3000, 64, 512, 128, 256
    q, raw, raw_pos0, cache, pooled, sel = _case(T, q_pos0, H, D, W, topk, seed=41)
    a = _narrow(q, q_pos0, raw, raw_pos0, W, cache, sel, 12)
    b = _narrow(q, q_pos0, raw, raw_pos0, W, cache, sel, 12)
    assert np.array_equal(a, b)
    small = torch.empty(10, dtype=torch.float32, device="cuda")
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsv4.DSV4Error) as e:
        dsv4.dsv4_sparse_attn_narrow(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                     bf16_t(raw).cuda(), raw_pos0, W, cache,
                                     torch.from_numpy(sel).cuda(), out, 12, small)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert not out.any()   # nothing was enqueued


# ====================================================================== chunk-parallel top-k

def _scores(kind, rows, q_pos0, seed):
    rng = np.random.default_rng(seed)
    n_cols = (q_pos0 + rows) // 4
    if kind == "normal":
        s = rng.standard_normal((rows, n_cols), dtype=np.float32)
    elif kind == "ties":
        s = rng.integers(0, 40, size=(rows, n_cols)).astype(np.float32)
    elif kind == "signed_zero":
        s = np.where(rng.random((rows, n_cols)) < 0.5, np.float32(-0.0), np.float32(0.0))
        s = s.astype(np.float32)
        s[:, ::1013] = 1.0
    else:
        s = np.full((rows, n_cols), -3.25, np.float32)
    for t in range(rows):  # beyond the visible prefix: never chosen
        s[t, O.visible_rows(q_pos0 + t):] = np.float32(1e30)
    return s


def _topk_both(s, q_pos0, topk):
    rows, n_cols = s.shape
    d = torch.from_numpy(s).cuda()
    nb = dsv4.dsv4_topk_split_workspace_bytes(rows, q_pos0, topk)
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda") if nb else None
    a = torch.full((rows, topk), 99, dtype=torch.int32, device="cuda")
    b = torch.full((rows, topk), 77, dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select_split(d, q_pos0, n_cols, topk, a, ws)
    dsv4.dsv4_topk_select(d, q_pos0, n_cols, topk, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy(), nb


@pytest.mark.parametrize("rows,q_pos0", [(1, (1 << 20) - 4), (3, 4 * 100000), (64, 4 * 70000)])
@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zero", "constant"])
@pytest.mark.parametrize("topk", [1, 2048, 4096])
def test_split_topk_equals_per_row_kernel(rows, q_pos0, kind, topk):
    s = _scores(kind, rows, q_pos0, seed=rows * 7 + topk)
    a, b, nb = _topk_both(s, q_pos0, topk)
    assert nb > 0  # the two-pass path ran
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("rows,q_pos0,topk", [(300, 4 * 70000, 2048), (130, 4 * 40000, 4096),
                                              (1024, (1 << 20) - 1024, 2048)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_split_topk_many_rows_equals_per_row_kernel(rows, q_pos0, topk, kind):
    """More than 64 rows take the two-pass top-k when k % 4 == 0 and a row has
    at most 32,768 chunk candidates (whole tiles at 1M context included); the
    result is the per-row kernel's, and sampled rows are the oracle's."""
    s = _scores(kind, rows, q_pos0, seed=rows + topk)
    a, b, nb = _topk_both(s, q_pos0, topk)
    assert nb > 0
    np.testing.assert_array_equal(a, b)
    rng = np.random.default_rng(rows)
    for t in rng.choice(rows, 6, replace=False):
        vis = O.visible_rows(q_pos0 + int(t))
        np.testing.assert_array_equal(a[t], O.topk_row(s[t].astype(np.float64), vis, topk))


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_split_topk_matches_oracle(kind):
    rows, q_pos0, topk = 2, 4 * 70000, 2048        # 3 chunks, the last one short
    s = _scores(kind, rows, q_pos0, seed=3)
    a, _, nb = _topk_both(s, q_pos0, topk)
    assert nb > 0
    np.testing.assert_array_equal(a, O.topk_select(s.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("T,S_tokens,topk", [(3, 140000, 512), (64, 4 * 70000, 2048),
                                            (200, 4 * 40000, 512),
                                            # the last chunk's 2k candidates do not fit
                                            # the row: workspace split or per-row kernel
                                            (3, 140000, 2048), (100, 140000, 2048)])
def test_select_long_rows_equals_per_row_kernel_and_oracle(T, S_tokens, topk):
    """Indexer select over rows longer than one 32,768-column chunk (2 or 3
    chunks): its top-k runs in two register passes whose chunk candidates are
    kept in the tile's own score rows.  It must equal the LDS-staged per-row
    kernel on the same GPU scores (computed separately and kept), with the
    scratch dsv4_indexer_scratch_bytes sizes and with only the score rows, and
    the oracle's selection from the oracle's scores."""
    from test_gpu_parity import _score_case
    from parity_util import assert_selection_matches
    c, st, S, q_pos0, q, w = _score_case(T, S_tokens, T, 64, 128, seed=T + 8)
    assert S > 32768
    qd, wd = bf16_t(q).cuda(), torch.from_numpy(w).cuda()
    stride = dsv4.dsv4_score_stride(S)
    sc = torch.empty((T, stride), device="cuda")
    dsv4.dsv4_indexer_scores(c, qd, wd, q_pos0, sc)
    per_row = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select(sc, q_pos0, S, topk, per_row)
    outs = []
    for nbytes in (dsv4.dsv4_indexer_scratch_bytes(T, S), T * stride * 4):
        scratch = torch.empty(nbytes // 4, device="cuda")
        out = torch.full((T, topk), 5, dtype=torch.int32, device="cuda")
        assert not dsv4.dsv4_indexer_select(c, S, qd, wd, T, q_pos0, 64, topk, out, scratch, 0)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], per_row) and torch.equal(outs[1], per_row)
    ref = O.indexer_scores(q, w, st.rows[:S], q_pos0, S)
    assert_selection_matches(outs[0].cpu().numpy(), ref, q_pos0, topk)
