"""GPU parity of the sibling attention modes that share the fused kernel
[P2 "perf(deepseek_v4): faster exact DeepSeek-V4 prefill", commit 1: one
kernel routed for LocalAttention, CompressedAttention and
SparseCompressedAttention], called through the C ABI, against the CPU oracle:

  * the ratio-128 compressor (CompressedAttention's pool), bit-exact over
    arbitrary chunk splits with the remainder carried between calls;
  * window-only attention (no pool: LocalAttention);
  * attention over every visible ratio-128 pooled row (CompressedAttention),
    alone and end to end after the ratio-128 compressor.

Attention outputs are compared with the fp64 oracle at the same bound as the
indexed path: max |gpu - ref| <= 2e-2.
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


# ====================================================================== ratio-128 compressor

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_compress_ratio128_any_split_is_bit_exact(dtype):
    rng = np.random.default_rng(128)
    n, dim = 128 * 5 + 37, 512
    x = rng.standard_normal((n, dim)).astype(np.float32) * 2
    if dtype == torch.bfloat16:
        x = SI.as_bf16_values(x)
    ref = O.PoolingCacheState(dim, 8, out_bf16=(dtype == torch.bfloat16), ratio=128)
    O.compress(ref, x)
    assert (ref.n_rows, ref.n_rem) == (5, 37)
    xd = torch.from_numpy(x).to(dtype).cuda()
    splits = [[n], [1] * 130 + [n - 130], [127, 1, 128, 300, 121], [0, 200, 0, 477]]
    for _ in range(4):
        cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(1, 8)))
        splits.append(list(np.diff(np.concatenate([[0], cuts, [n]]))))
    for parts in splits:
        c = dsv4.PoolCache(8, dim, dtype=dtype, ratio=128)
        pos = 0
        for p in parts:
            dsv4.dsv4_compress(c, xd[pos:pos + p])
            pos += p
        torch.cuda.synchronize()
        assert (c.n_rows, c.n_rem) == (5, 37), parts
        np.testing.assert_array_equal(c.rows[:5].float().cpu().numpy(), ref.rows[:5])
        np.testing.assert_array_equal(c.rem[:37].float().cpu().numpy(), ref.rem)


def test_compress_ratio128_ramp_closed_form():
    # x_p = p (exact in float32): row s = 128 s + 63.5 exactly
    n = 128 * 6
    x = np.repeat(np.arange(n, dtype=np.float32)[:, None], 64, axis=1)
    c = dsv4.PoolCache(6, 64, dtype=torch.float32, ratio=128)
    dsv4.dsv4_compress(c, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    got = c.rows.cpu().numpy()
    np.testing.assert_array_equal(got, np.repeat((128 * np.arange(6) + 63.5)[:, None], 64, axis=1))


# ====================================================================== local attention

def _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0):
    raw = SI.as_bf16_values(rng.standard_normal((q_pos0 + T - raw_pos0, D)).astype(np.float32))
    q = SI.as_bf16_values(rng.standard_normal((T, H, D)).astype(np.float32))
    return q, raw


def _run(q, q_pos0, raw, raw_pos0, W, cache, sel=None):
    T, H, D = q.shape
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_prefill_attn(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                  bf16_t(raw).cuda(), raw_pos0, W, cache, sel, out)
    return out


@pytest.mark.parametrize("T,q_pos0,H,D,W", [
    (50, 0, 64, 512, 128),    # first chunk: windows clipped at position 0
    (33, 1000, 64, 512, 128),  # full windows, ragged key tile tail (128 = 4 tiles exactly)
    (21, 400, 64, 512, 77),   # window not a multiple of the key tile
    (70, 10, 16, 64, 7),
    (1, 5000, 64, 512, 128),  # a single query
])
def test_local_attention_matches_oracle(T, q_pos0, H, D, W):
    rng = np.random.default_rng(T * 31 + W)
    raw_pos0 = max(0, q_pos0 - W + 1)
    q, raw = _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0)
    out = _run(q, q_pos0, raw, raw_pos0, W, None)
    torch.cuda.synchronize()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, None, None, 1 / math.sqrt(D))
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= ATTN_ATOL, err


def test_local_attention_equals_empty_selection_bitwise():
    # No pool, and a ratio-4 pool whose selection is all empty, walk the same
    # keys in the same order: the outputs are the same bits.
    T, q_pos0, H, D, W = 24, 700, 64, 512, 128
    rng = np.random.default_rng(3)
    raw_pos0 = q_pos0 - W + 1
    q, raw = _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0)
    S = (q_pos0 + T) // 4
    cache = dsv4.PoolCache(S, D)
    cache.rows.copy_(bf16_t(rng.standard_normal((S, D)).astype(np.float32)))
    cache.set_state(S, (q_pos0 + T) - 4 * S)
    empty = torch.full((T, 16), -1, dtype=torch.int32, device="cuda")
    a = _run(q, q_pos0, raw, raw_pos0, W, None)
    b = _run(q, q_pos0, raw, raw_pos0, W, cache, empty)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ====================================================================== compressed attention (ratio 128)

def _ratio128_cache(rng, q_pos0, T, D):
    S = (q_pos0 + T) // 128
    pooled = SI.as_bf16_values(rng.standard_normal((S, D)).astype(np.float32) * 0.5)
    cache = dsv4.PoolCache(S + 1, D, ratio=128)
    cache.rows[:S].copy_(bf16_t(pooled))
    cache.set_state(S, (q_pos0 + T) - 128 * S)
    return cache, pooled


@pytest.mark.parametrize("T,q_pos0,H,D,W", [
    (40, 128 * 8 - 20, 64, 512, 128),  # queries cross a pooled-row boundary
    (64, 128 * 300, 64, 512, 128),     # 300 pooled rows + full window
    (30, 100, 64, 512, 128),           # row 0 becomes visible mid-chunk (p = 127)
    (17, 128 * 40 + 5, 32, 256, 64),
])
def test_compressed_attention_matches_oracle(T, q_pos0, H, D, W):
    rng = np.random.default_rng(q_pos0 + T)
    raw_pos0 = max(0, q_pos0 - W + 1)
    q, raw = _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0)
    cache, pooled = _ratio128_cache(rng, q_pos0, T, D)
    out = _run(q, q_pos0, raw, raw_pos0, W, cache)
    torch.cuda.synchronize()
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, None,
                                     1 / math.sqrt(D), ratio=128)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= ATTN_ATOL, err


def test_compressed_attention_end_to_end_after_ratio128_compress():
    """A 300-token chunk behind 20 pooled rows and a 50-token remainder: the
    chunk goes through the ratio-128 compressor (device and oracle), then
    every query attends its window plus every visible pooled row."""
    rng = np.random.default_rng(2026)
    H, D, W, T = 64, 512, 128, 300
    n_prev, rem_prev = 20, 50
    q_pos0 = 128 * n_prev + rem_prev
    prefix = SI.as_bf16_values(rng.standard_normal((n_prev, D)).astype(np.float32) * 0.5)
    raw_pos0 = q_pos0 - W + 1
    q, raw = _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0)
    rem = raw[q_pos0 - rem_prev - raw_pos0:q_pos0 - raw_pos0]   # the 50 waiting tokens
    chunk = raw[q_pos0 - raw_pos0:]
    cache = dsv4.PoolCache(32, D, ratio=128)
    cache.rows[:n_prev].copy_(bf16_t(prefix))
    cache.rem[:rem_prev].copy_(bf16_t(rem))
    cache.set_state(n_prev, rem_prev)
    st = O.PoolingCacheState(D, 32, ratio=128)
    st.rows[:n_prev] = prefix
    st.n_rows = n_prev
    st.rem = rem.copy()
    dsv4.dsv4_compress(cache, bf16_t(chunk).cuda())
    O.compress(st, chunk)
    assert (cache.n_rows, cache.n_rem) == (st.n_rows, st.n_rem) == (22, 94)
    out = _run(q, q_pos0, raw, raw_pos0, W, cache)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cache.rows[:22].float().cpu().numpy(), st.rows[:22])
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, st.rows[:22], None,
                                     1 / math.sqrt(D), ratio=128)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= ATTN_ATOL, err


# ====================================================================== maximum sizes

def test_attention_at_maximum_topk():
    """top-k = DSV4_MAX_TOPK (4,096: the largest selection row the kernels hold
    in LDS) with H = 64, D = 512, through both attention entry points."""
    T, q_pos0, H, D, W, topk = 5, 4 * 6000, 64, 512, 128, 4096
    rng = np.random.default_rng(4096)
    raw_pos0 = q_pos0 - W + 1
    q, raw = _rand_q_raw(rng, T, q_pos0, H, D, raw_pos0)
    S = (q_pos0 + T) // 4
    pooled = SI.as_bf16_values(rng.standard_normal((S, D)).astype(np.float32) * 0.5)
    cache = dsv4.PoolCache(S, D)
    cache.rows.copy_(bf16_t(pooled))
    cache.set_state(S, (q_pos0 + T) - 4 * S)
    sel = np.full((T, topk), -1, np.int32)
    for t in range(T):
        v = (q_pos0 + t + 1) // 4
        sel[t] = np.sort(rng.choice(v, size=topk, replace=False))
    sel[2, topk - 1] = -1       # an empty last slot
    ref = O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, sel, 1 / math.sqrt(D))
    seld = torch.from_numpy(sel).cuda()
    a = _run(q, q_pos0, raw, raw_pos0, W, cache, seld)
    ns, nb = dsv4.dsv4_sparse_attn_narrow_plan(T, H, D, W, topk)
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    b = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_attn_narrow(bf16_t(q.reshape(T, H * D)).cuda().view(T, H, D), q_pos0,
                                 bf16_t(raw).cuda(), raw_pos0, W, cache, seld, b, ns, ws)
    torch.cuda.synchronize()
    assert np.abs(a.float().cpu().numpy() - ref).max() <= ATTN_ATOL
    assert np.abs(b.float().cpu().numpy() - ref).max() <= ATTN_ATOL


def test_compress_at_maximum_ratio_is_bit_exact():
    # ratio 256 (DSV4_MAX_RATIO): 2 rows + a 255-row remainder, then one more token
    rng = np.random.default_rng(256)
    n, dim = 256 * 3 - 1, 64
    x = SI.as_bf16_values(rng.standard_normal((n + 1, dim)).astype(np.float32))
    ref = O.PoolingCacheState(dim, 4, ratio=256)
    c = dsv4.PoolCache(4, dim, ratio=256)
    xd = bf16_t(x).cuda()
    O.compress(ref, x[:n])
    dsv4.dsv4_compress(c, xd[:n])
    assert (c.n_rows, c.n_rem) == (ref.n_rows, ref.n_rem) == (2, 255)
    O.compress(ref, x[n:])
    dsv4.dsv4_compress(c, xd[n:])
    torch.cuda.synchronize()
    assert (c.n_rows, c.n_rem) == (ref.n_rows, ref.n_rem) == (3, 0)
    np.testing.assert_array_equal(c.rows[:3].float().cpu().numpy(), ref.rows[:3])
