"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a worked
example from the pages (tests/golden/), a closed form, a hand-computed value,
brute force written a different way on tiny inputs, or an independent library
routine (numpy.matmul, torch's bf16 conversion, torch's scaled_dot_product
attention).  They are chosen so that a dropped term, a wrong sign, an
off-by-one in visibility, a transposed operand or a wrong tie rule in the
oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsv4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_hand_values():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 1.0,                       # tie -> even (mantissa 0)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,       # tie -> even (mantissa 2)
        one + 2.0 ** -8 + 2.0 ** -20: one + 2.0 ** -7,  # just above the tie -> up
        -(one + 2.0 ** -8): -1.0,
        3.0: 3.0,
        0.0: 0.0,
    }
    x = np.array(list(cases.keys()), dtype=np.float32)
    want = np.array(list(cases.values()), dtype=np.float32)
    np.testing.assert_array_equal(O.round_to_bf16(x), want)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-30).astype(np.float32),
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x), want)


# ---------------------------------------------------------------- compressor

def test_golden_10_tokens_two_rows_two_remainder():
    g = golden("p1_correctness_10tok_ratio4.json")
    st = O.PoolingCacheState(dim=8, capacity=16)
    x = np.arange(g["n_tokens"] * 8, dtype=np.float32).reshape(g["n_tokens"], 8)
    appended = O.compress(st, x)
    assert appended == g["expected_pooled_rows"] == st.n_rows
    assert st.n_rem == g["expected_remainder_tokens"]
    np.testing.assert_array_equal(st.rem, x[8:10])  # the last two tokens wait


def test_pool_order_left_to_right_float32():
    # a + b with b = 2^-24 is an exact tie in float32 and rounds back to a;
    # adding c = 2^-24 afterwards again rounds away, so ((a+b)+c)+d = 1.
    # A pairwise sum (a+b)+(c+d) would give 1 + 2^-23 instead.
    tiny = 2.0 ** -24
    x = np.array([[1.0], [tiny], [tiny], [0.0]], dtype=np.float32)
    st = O.PoolingCacheState(dim=1, capacity=1, out_bf16=False)
    O.compress(st, x)
    assert st.rows[0, 0] == np.float32(0.25)


def test_pool_rounds_once_to_bf16():
    # mean = (1 + 2^-7 + 2^-8 ... ) chosen so the float32 mean is an exact bf16
    # tie: mean = 1 + 2^-8 -> bf16 1.0 (even), 1 + 3*2^-8 -> 1 + 2^-6.
    for mean, want in ((1 + 2.0 ** -8, 1.0), (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6)):
        x = np.full((4, 1), mean, dtype=np.float32)
        st = O.PoolingCacheState(dim=1, capacity=1, out_bf16=True)
        O.compress(st, x)
        assert st.rows[0, 0] == np.float32(want)


def test_pool_constant_and_ramp_closed_forms():
    st = O.PoolingCacheState(dim=3, capacity=32)
    O.compress(st, np.full((128, 3), -2.5, dtype=np.float32))
    assert st.n_rows == 32 and st.n_rem == 0
    assert np.all(st.rows[:32] == np.float32(-2.5))
    # x_p = p: row s = mean(4s..4s+3) = 4s + 1.5, exact in bf16 for s < 32
    st = O.PoolingCacheState(dim=2, capacity=32)
    x = np.repeat(np.arange(128, dtype=np.float32)[:, None], 2, axis=1)
    O.compress(st, x)
    np.testing.assert_array_equal(st.rows[:32, 0], 4 * np.arange(32) + 1.5)


@pytest.mark.parametrize("bf16", [True, False])
def test_pool_chunk_split_invariance(bf16):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 5)).astype(np.float32)
    ref = O.PoolingCacheState(dim=5, capacity=64, out_bf16=bf16)
    O.compress(ref, x)
    splits = [[64], [1, 63], [3, 61], [10, 54], [0, 64], [64, 0]]
    splits += [[a, b - a, 64 - b] for a, b in itertools.combinations(range(0, 65, 7), 2)]
    rs = np.random.default_rng(3)
    for _ in range(40):
        cuts = np.sort(rs.integers(0, 65, size=rs.integers(1, 9)))
        splits.append(list(np.diff(np.concatenate([[0], cuts, [64]]))))
    for parts in splits:
        st = O.PoolingCacheState(dim=5, capacity=64, out_bf16=bf16)
        pos = 0
        for n in parts:
            O.compress(st, x[pos:pos + n])
            pos += n
        assert st.n_rows == ref.n_rows == 16 and st.n_rem == ref.n_rem == 0
        np.testing.assert_array_equal(st.rows, ref.rows)


def test_pool_capacity_overflow_leaves_state():
    st = O.PoolingCacheState(dim=2, capacity=1)
    O.compress(st, np.ones((6, 2), np.float32))      # 1 row + 2 waiting
    before = (st.n_rows, st.rem.copy(), st.rows.copy())
    with pytest.raises(ValueError):
        O.compress(st, np.ones((3, 2), np.float32))  # 2 + 3 = 5 -> a second row: over
    assert st.n_rows == before[0]
    np.testing.assert_array_equal(st.rem, before[1])


# ------------------------------------------- ratio-128 pool (CompressedAttention)

def test_pool_ratio128_constant_and_ramp_closed_forms():
    st = O.PoolingCacheState(dim=3, capacity=4, ratio=128)
    O.compress(st, np.full((300, 3), 0.75, dtype=np.float32))
    assert st.n_rows == 2 and st.n_rem == 300 - 256
    assert np.all(st.rows[:2] == np.float32(0.75))
    # x_p = p: row s = mean(128s .. 128s+127) = 128s + 63.5.  Every partial sum
    # is an integer below 2^24, so the float32 result is exact; stored in
    # float32 it is the closed form, stored in bf16 it is that value rounded
    # by torch's own conversion.
    n = 128 * 5
    x = np.repeat(np.arange(n, dtype=np.float32)[:, None], 2, axis=1)
    want = 128 * np.arange(5) + 63.5
    st = O.PoolingCacheState(dim=2, capacity=5, out_bf16=False, ratio=128)
    O.compress(st, x)
    np.testing.assert_array_equal(st.rows[:, 1], want)
    st = O.PoolingCacheState(dim=2, capacity=5, out_bf16=True, ratio=128)
    O.compress(st, x)
    np.testing.assert_array_equal(
        st.rows[:, 0], torch.tensor(want, dtype=torch.float32).to(torch.bfloat16).float().numpy())


def test_pool_ratio128_order_left_to_right():
    # 1 followed by 127 copies of 2^-24: each add is a tie that rounds back to
    # 1, so the left-to-right float32 sum is exactly 1 and the mean 2^-7.  Any
    # pairwise or blocked order would collect the small terms first and land
    # above 1.
    x = np.full((128, 1), 2.0 ** -24, dtype=np.float32)
    x[0, 0] = 1.0
    st = O.PoolingCacheState(dim=1, capacity=1, out_bf16=False, ratio=128)
    O.compress(st, x)
    assert st.rows[0, 0] == np.float32(2.0 ** -7)
    assert float(np.sum(x.astype(np.float64))) / 128 > 2.0 ** -7


def test_pool_ratio128_chunk_split_invariance():
    rng = np.random.default_rng(71)
    n = 128 * 3 + 17
    x = rng.standard_normal((n, 4)).astype(np.float32)
    ref = O.PoolingCacheState(dim=4, capacity=3, ratio=128)
    O.compress(ref, x)
    assert ref.n_rows == 3 and ref.n_rem == 17
    rs = np.random.default_rng(5)
    for _ in range(12):
        cuts = np.sort(rs.integers(0, n + 1, size=rs.integers(1, 6)))
        st = O.PoolingCacheState(dim=4, capacity=3, ratio=128)
        pos = 0
        for m in np.diff(np.concatenate([[0], cuts, [n]])):
            O.compress(st, x[pos:pos + m])
            pos += m
        np.testing.assert_array_equal(st.rows, ref.rows)
        np.testing.assert_array_equal(st.rem, ref.rem)
    # the mean of a group is the float64 mean to within float32 summation error
    g = x[:128].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(ref.rows[0], g, atol=2e-2)


# ---------------------------------------------------------------- visibility

def test_visibility_against_token_enumeration():
    # A pooled row is visible once every token it summarises is at or before p.
    for p in range(0, 300):
        brute = 0
        s = 0
        while True:
            toks = [4 * s + i for i in range(4)]
            if max(toks) <= p:
                brute += 1
                s += 1
            else:
                break
        assert O.visible_rows(p) == brute
    assert O.visible_rows(2) == 0 and O.visible_rows(3) == 1


@pytest.mark.parametrize("ratio", [2, 128])
def test_visibility_other_ratios_against_enumeration(ratio):
    for p in range(0, 3 * ratio + 5):
        brute = sum(1 for s in range(p + 2) if ratio * s + ratio - 1 <= p)
        assert O.visible_rows(p, ratio) == brute
    assert O.visible_rows(ratio - 2, ratio) == 0 and O.visible_rows(ratio - 1, ratio) == 1


def test_visible_pairs_closed_form():
    # sum_{p=0}^{63} floor((p+1)/4) = 4*(0+1+...+15) + 16 = 496
    assert sum(O.visible_rows(p) for p in range(64)) == 496


# ---------------------------------------------------------------- path decision

def test_path_decision_rules():
    with pytest.raises(ValueError):
        O.indexer_path(5, 6, 8)
    assert O.indexer_path(0, 0, 8) == "empty"
    assert O.indexer_path(8, 8, 8) == "all_pooled"
    assert O.indexer_path(1, 1, 8) == "all_pooled"
    assert O.indexer_path(9, 9, 8) == "full"


def test_golden_10_tokens_sequential_selection():
    g = golden("p1_correctness_10tok_ratio4.json")
    T, topk = g["n_tokens"], 8
    idx = O.all_pooled_selection(T, 0, topk)
    for t in range(T):
        v = (t + 1) // 4
        assert list(idx[t, :v]) == list(range(v))
        assert np.all(idx[t, v:] == -1)
    assert idx[9, 0] == 0 and idx[9, 1] == 1 and idx[9, 2] == -1


def test_all_pooled_equals_full_selection():
    rng = np.random.default_rng(11)
    for S, topk in ((5, 8), (8, 8), (16, 16), (3, 64)):
        T = 4 * S
        q = rng.standard_normal((T, 3, 6))
        w = rng.random((T, 3))
        K = rng.standard_normal((S, 6))
        sc = O.indexer_scores(q, w, K, 0, S)
        full = O.topk_select(sc, 0, topk)
        np.testing.assert_array_equal(full, O.all_pooled_selection(T, 0, topk))
        got, ap = O.indexer_select(None, None, K, S, T, 0, topk, S)
        assert ap
        np.testing.assert_array_equal(got, full)


# ---------------------------------------------------------------- scores

def _brute_scores(q, w, K, q_pos0, S):
    T, H, D = q.shape
    out = [[0.0] * S for _ in range(T)]
    for t in range(T):
        for s in range(S):
            if 4 * (s + 1) > q_pos0 + t + 1:
                out[t][s] = -math.inf
                continue
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += float(q[t, h, d]) * float(K[s, d])
                if dot > 0:
                    tot += float(w[t, h]) * dot
            out[t][s] = tot
    return np.array(out)


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(5)
    T, H, D, S, q_pos0 = 9, 3, 4, 6, 15
    q = rng.standard_normal((T, H, D))
    w = rng.random((T, H)) * 2 - 0.5   # include negative weights
    K = rng.standard_normal((S, D))
    got = O.indexer_scores(q, w, K, q_pos0, S)
    want = _brute_scores(q, w, K, q_pos0, S)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)


def test_scores_reduce_to_matmul():
    rng = np.random.default_rng(6)
    T, D, S = 7, 5, 9
    q = rng.random((T, 1, D)) + 0.1       # positive entries: every dot > 0
    K = rng.random((S, D)) + 0.1
    w = np.ones((T, 1))
    got = O.indexer_scores(q, w, K, 10_000, S)
    np.testing.assert_allclose(got, np.matmul(q[:, 0, :], K.T), rtol=1e-13)


def test_scores_relu_and_weights():
    rng = np.random.default_rng(8)
    T, H, D, S = 4, 5, 6, 7
    q = rng.standard_normal((T, H, D))
    K = rng.standard_normal((S, D))
    w1 = rng.random((T, H))
    w2 = rng.random((T, H))
    z = O.indexer_scores(q, np.zeros((T, H)), K, 1000, S)
    assert np.all(z == 0.0)
    a = O.indexer_scores(q, w1, K, 1000, S)
    b = O.indexer_scores(q, w2, K, 1000, S)
    ab = O.indexer_scores(q, 2 * w1 + 3 * w2, K, 1000, S)
    np.testing.assert_allclose(ab, 2 * a + 3 * b, rtol=1e-12, atol=1e-12)
    assert np.all(a >= 0)
    # all dot products negative -> ReLU kills everything
    neg = O.indexer_scores(np.abs(q), w1, -np.abs(K), 1000, S)
    assert np.all(neg == 0.0)


def test_scores_mask_fold_equals_second_pass():
    rng = np.random.default_rng(9)
    T, H, D, S, q_pos0 = 12, 2, 3, 8, 20
    q = rng.standard_normal((T, H, D))
    w = rng.random((T, H))
    K = rng.standard_normal((S, D))
    folded = O.indexer_scores(q, w, K, q_pos0, S, fold_mask=True)
    raw = O.indexer_scores(q, w, K, q_pos0, S, fold_mask=False)
    assert np.all(np.isfinite(raw))
    second = O.apply_pooled_mask(raw, q_pos0)
    assert np.array_equal(folded, second)   # -inf == -inf compares equal
    for t in range(T):
        v = (q_pos0 + t + 1) // 4
        assert np.all(np.isneginf(folded[t, v:])) and np.all(np.isfinite(folded[t, :v]))


# ---------------------------------------------------------------- top-k

def _check_selection_characterisation(scores_row, n_vis, topk, sel):
    """Independent characterisation of the selection: exactly min(k, n_vis)
    distinct visible indices in ascending order then -1; every chosen row
    beats every unchosen visible row (higher score, or equal score and lower
    index)."""
    k_eff = min(topk, n_vis)
    chosen = [int(s) for s in sel if s >= 0]
    assert len(chosen) == k_eff
    assert all(s == -1 for s in sel[k_eff:])
    assert chosen == sorted(chosen) and len(set(chosen)) == k_eff
    assert all(0 <= s < n_vis for s in chosen)
    unchosen = [u for u in range(n_vis) if u not in set(chosen)]
    for c in chosen:
        for u in unchosen:
            assert scores_row[c] > scores_row[u] or (scores_row[c] == scores_row[u] and c < u)


def test_topk_brute_force_and_characterisation():
    rng = np.random.default_rng(12)
    for trial in range(60):
        n = int(rng.integers(0, 20))
        topk = int(rng.integers(1, 12))
        vals = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
        if trial % 3 == 0:
            vals = rng.standard_normal(n)
        row = np.concatenate([vals, np.full(5, -np.inf)])
        sel = O.topk_row(row, n, topk)
        _check_selection_characterisation(row, n, topk, sel)
        # brute force: sort all (score, index) pairs with Python's sorted
        order = sorted(range(n), key=lambda i: (-vals[i], i))[:min(topk, n)]
        assert [int(s) for s in sel if s >= 0] == sorted(order)


def test_topk_signed_zero_ties():
    row = np.array([0.0, -0.0, 0.0, -0.0, 1.0])
    sel = O.topk_row(row, 5, 3)
    assert list(sel) == [0, 1, 4]   # -0 == +0: lowest indices win


def test_topk_masked_never_selected():
    row = np.array([3.0, 2.0, 1.0, -np.inf, -np.inf])
    sel = O.topk_row(row, 3, 8)
    assert list(sel) == [0, 1, 2, -1, -1, -1, -1, -1]


def test_topk_tiled_equals_untiled():
    rng = np.random.default_rng(13)
    T, H, D, S, q_pos0, topk = 37, 3, 8, 30, 84, 6
    q = rng.standard_normal((T, H, D))
    w = rng.random((T, H))
    K = rng.standard_normal((S, D))
    full, _ = O.indexer_select(q, w, K, S, T, q_pos0, topk, S, tile_rows=0)
    for tile in (1, 5, 8, 16, 36, 37, 100):
        tiled, _ = O.indexer_select(q, w, K, S, T, q_pos0, topk, S, tile_rows=tile)
        np.testing.assert_array_equal(tiled, full)


def test_empty_pool_path():
    idx, ap = O.indexer_select(None, None, np.zeros((0, 4)), 0, 3, 0, 4, 0)
    assert not ap and np.all(idx == -1) and idx.shape == (3, 4)


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, mask):
    # torch CPU reference in float64 (independent library routine)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask)).numpy()


def test_attention_reduces_to_causal_sdpa():
    rng = np.random.default_rng(14)
    T, H, D = 10, 3, 8
    q = rng.standard_normal((T, H, D))
    raw = rng.standard_normal((T, D))
    pooled = np.zeros((0, D))
    scale = 1.0 / math.sqrt(D)
    # window >= p+1 and no pooled row visible (positions 0..2 see none; use
    # sel_idx of all -1 for the rest)
    sel = np.full((T, 4), -1, dtype=np.int32)
    got = O.sparse_prefill_attention(q, 0, raw, 0, T + 5, pooled, sel, scale)
    causal = np.tril(np.ones((T, T), dtype=bool))
    want = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(raw, (H, T, D)).copy(),
                 np.broadcast_to(raw, (H, T, D)).copy(), causal).transpose(1, 0, 2)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_with_pooled_matches_masked_sdpa():
    rng = np.random.default_rng(15)
    T, H, D, W, q_pos0 = 6, 2, 4, 3, 20
    q = rng.standard_normal((T, H, D))
    raw_pos0 = q_pos0 - W + 1
    raw = rng.standard_normal((T + W - 1, D))
    S = (q_pos0 + T) // 4
    pooled = rng.standard_normal((S, D))
    sel = np.full((T, 4), -1, dtype=np.int32)
    for t in range(T):
        v = (q_pos0 + t + 1) // 4
        pick = rng.choice(v, size=3, replace=False)
        sel[t, :3] = np.sort(pick)
    sel[0, 3] = S - 1  # a row not visible to the first query: must be ignored
    scale = 0.3
    got = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, scale)
    # SDPA over [all raw rows ; all pooled rows] with an explicit boolean mask
    keys = np.concatenate([raw, pooled], axis=0)
    mask = np.zeros((T, keys.shape[0]), dtype=bool)
    for t in range(T):
        p = q_pos0 + t
        for j in range(raw.shape[0]):
            pos = raw_pos0 + j
            mask[t, j] = (p - W < pos <= p)
        for s in sel[t]:
            if 0 <= s < (p + 1) // 4:
                mask[t, raw.shape[0] + s] = True
    KK = np.broadcast_to(keys, (H,) + keys.shape).copy()
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2)), torch.from_numpy(KK), torch.from_numpy(KK),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(16)
    T, H, D = 5, 2, 4
    q = rng.standard_normal((T, H, D))
    raw = rng.standard_normal((T, D))
    none = np.full((T, 2), -1, dtype=np.int32)
    # window 1, no pooled row: each query sees only its own raw row
    got = O.sparse_prefill_attention(q, 0, raw, 0, 1, np.zeros((0, D)), none, 0.5)
    for t in range(T):
        np.testing.assert_allclose(got[t], np.broadcast_to(raw[t], (H, D)), rtol=1e-14)
    # all keys equal -> output is that row
    same = np.tile(raw[:1], (T, 1))
    got = O.sparse_prefill_attention(q, 0, same, 0, 4, np.zeros((0, D)), none, 0.5)
    np.testing.assert_allclose(got, np.broadcast_to(raw[0], (T, H, D)), rtol=1e-13)


def test_attention_null_selection_and_trimmed_raw_buffer():
    rng = np.random.default_rng(17)
    T, H, D, W, q_pos0 = 7, 2, 4, 3, 33
    q = rng.standard_normal((T, H, D))
    S = (q_pos0 + T) // 4
    pooled = rng.standard_normal((S, D))
    raw_full = rng.standard_normal((q_pos0 + T, D))   # positions 0..
    seq = O.all_pooled_selection(T, q_pos0, S)
    a = O.sparse_prefill_attention(q, q_pos0, raw_full, 0, W, pooled, None, 0.4)
    b = O.sparse_prefill_attention(q, q_pos0, raw_full, 0, W, pooled, seq, 0.4)
    np.testing.assert_array_equal(a, b)
    # trimmed raw buffer starting just where the first window starts
    r0 = q_pos0 - W + 1
    c = O.sparse_prefill_attention(q, q_pos0, raw_full[r0:], r0, W, pooled, None, 0.4)
    np.testing.assert_array_equal(a, c)


def _masked_sdpa(q, keys, mask, scale):
    H = q.shape[1]
    KK = np.broadcast_to(keys, (H,) + keys.shape).copy()
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2)), torch.from_numpy(KK), torch.from_numpy(KK),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy().transpose(1, 0, 2)


def test_local_attention_is_banded_causal_sdpa():
    # Window-only mode (no pooled keys): sliding-window causal attention.
    rng = np.random.default_rng(18)
    T, H, D, W, q_pos0 = 9, 3, 8, 4, 11
    q = rng.standard_normal((T, H, D))
    raw_pos0 = 2
    raw = rng.standard_normal((q_pos0 + T - raw_pos0, D))
    got = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, None, None, 0.35)
    mask = np.zeros((T, raw.shape[0]), dtype=bool)
    for t in range(T):
        p = q_pos0 + t
        for j in range(raw.shape[0]):
            mask[t, j] = p - W < raw_pos0 + j <= p
    np.testing.assert_allclose(got, _masked_sdpa(q, raw, mask, 0.35), rtol=1e-10, atol=1e-12)
    # a pool of any size is ignored when it is passed as None, and an
    # all-empty selection over a real pool gives the same result
    S = (q_pos0 + T) // 4
    pooled = rng.standard_normal((S, D))
    empty = np.full((T, 3), -1, dtype=np.int32)
    same = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, empty, 0.35)
    np.testing.assert_array_equal(got, same)


def test_compressed_attention_ratio128_matches_masked_sdpa():
    # CompressedAttention: every pooled row whose 128 tokens are all at or
    # before the query is attended, together with the raw window.
    rng = np.random.default_rng(19)
    T, H, D, W = 6, 2, 4, 5
    q_pos0 = 128 * 3 - 3      # queries straddle the boundary 383 -> 384
    raw_pos0 = q_pos0 - W + 1
    raw = rng.standard_normal((T + W - 1, D))
    S = (q_pos0 + T) // 128
    pooled = rng.standard_normal((S, D))
    got = O.sparse_prefill_attention(q := rng.standard_normal((T, H, D)), q_pos0, raw,
                                     raw_pos0, W, pooled, None, 0.3, ratio=128)
    keys = np.concatenate([raw, pooled], axis=0)
    mask = np.zeros((T, keys.shape[0]), dtype=bool)
    for t in range(T):
        p = q_pos0 + t
        for j in range(raw.shape[0]):
            mask[t, j] = p - W < raw_pos0 + j <= p
        for s_ in range(S):
            mask[t, raw.shape[0] + s_] = 128 * s_ + 127 <= p
    assert mask[:, raw.shape[0]:].sum(axis=1).tolist() == [2, 2, 3, 3, 3, 3]
    np.testing.assert_allclose(got, _masked_sdpa(q, keys, mask, 0.3), rtol=1e-10, atol=1e-12)


def test_attention_repeated_slot_counts_once_per_listing():
    # Reading: a pooled row listed in two selection slots is two keys (each
    # slot is one key of the softmax).  SDPA over the key list [raw rows ;
    # pooled rows ; one more copy of every repeated row] with each copy
    # unmasked fixes that independently of the oracle's own loop.
    rng = np.random.default_rng(21)
    T, H, D, W, q_pos0 = 4, 3, 8, 3, 40
    raw_pos0 = q_pos0 - W + 1
    raw = rng.standard_normal((T + W - 1, D))
    S = (q_pos0 + T) // 4
    pooled = rng.standard_normal((S, D))
    q = rng.standard_normal((T, H, D))
    sel = np.full((T, 5), -1, dtype=np.int32)
    sel[0, :4] = [2, 7, 7, 9]          # row 7 twice
    sel[1, :5] = [5, 1, 5, 5, 3]       # row 5 three times, unsorted
    sel[2, :3] = [0, 0, 9]
    sel[3, :2] = [4, 8]                # no repeat
    scale = 0.4
    got = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, scale)
    extra = [(t, int(s)) for t in range(T) for j, s in enumerate(sel[t])
             if s >= 0 and s in sel[t, :j]]
    keys = np.concatenate([raw, pooled, np.stack([pooled[s] for _, s in extra])], axis=0)
    mask = np.zeros((T, keys.shape[0]), dtype=bool)
    for t in range(T):
        p = q_pos0 + t
        for j in range(raw.shape[0]):
            mask[t, j] = p - W < raw_pos0 + j <= p
        for s in set(int(s) for s in sel[t] if s >= 0):
            assert s < O.visible_rows(p)
            mask[t, raw.shape[0] + s] = True
    for e, (t, _) in enumerate(extra):
        mask[t, raw.shape[0] + S + e] = True
    assert len(extra) == 4
    np.testing.assert_allclose(got, _masked_sdpa(q, keys, mask, scale), rtol=1e-10, atol=1e-12)
    # and it differs from attending each distinct row once
    once = sel.copy()
    once[0, 2] = once[1, 2] = once[1, 3] = once[2, 1] = -1
    assert np.abs(O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, once, scale)
                  - got)[:3].max() > 1e-3


def test_tile_matrix_golden_scratch_sizes():
    # [P3 Summary; Suggested acceptance and benchmark matrix]: the score
    # scratch at 1M context is tile rows x pooled rows x 4 B.  The page
    # estimates about 4 GiB untiled at chunk 4,096 (262,146 rows); the
    # matrix lists the (global chunk, indexer tile) pairs to measure.
    g = golden("p3_tile_matrix.json")
    rows = g["compressed_rows_at_1M_context_approx"]
    untiled = 4096 * rows * 4
    assert round(untiled / 2 ** 30) == g["indexer_scores_bytes_at_chunk_4096_approx_GiB"]
    for chunk, tile in g["matrix"]:
        assert tile <= chunk and chunk % tile == 0
        # one reused scratch: the tile, not the chunk, sets its size
        assert tile * rows * 4 <= untiled
    assert [4096, 1024] in g["matrix"] and [1024, 1024] in g["matrix"]
    # the bench's (chunk, tile) matrix is the page's list
    import bench
    assert [list(m) for m in bench.MATRIX] == g["matrix"]
