"""dsv4_indexer_select_noalloc (static per-GPU scratch, nothing allocated)
against dsv4_indexer_select with a caller scratch, through the C ABI:
bit-identical selections on consecutive calls, the second and third with
fewer rows, an oversized tile refused before anything is enqueued, and the
all-pooled path that needs no scratch."""
import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI

from parity_util import ChunkState

pytestmark = pytest.mark.gpu


def _ref(cs, T, q_pos0, rows, tile=0):
    wl = cs.wl
    S = cs.S
    nb = dsv4.dsv4_indexer_scratch_bytes(T if tile == 0 else tile, S)
    scratch = torch.empty(nb // 4, device="cuda")
    idx = torch.full((T, wl.topk), -7, dtype=torch.int32, device="cuda")
    assert not dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx[rows],
                                        cs.w[rows], T, q_pos0, wl.idx_heads, wl.topk, idx,
                                        scratch, tile)
    torch.cuda.synchronize()
    return idx


def _noalloc(cs, T, q_pos0, rows, tile=0):
    wl = cs.wl
    idx = torch.full((T, wl.topk), -7, dtype=torch.int32, device="cuda")
    ap = dsv4.dsv4_indexer_select_noalloc(cs.icache, cs.acache.n_rows, cs.q_idx[rows],
                                          cs.w[rows], T, q_pos0, wl.idx_heads, wl.topk, idx,
                                          tile)
    torch.cuda.synchronize()
    assert not ap
    return idx


def test_noalloc_select_matches_scratch_select():
    wl = SI.CTX_128K
    cs = ChunkState(wl, with_attn_q=False)
    T, q0 = wl.chunk, cs.q_pos0
    # 1: the whole 2,048-row chunk; the static 32 MiB holds 256 rows of
    # 32,768 pooled rows, so it runs in eight tiles
    ref = _ref(cs, T, q0, slice(0, T))
    got = _noalloc(cs, T, q0, slice(0, T))
    assert torch.equal(got, ref)
    # 2: a smaller call right after (64 rows from the middle of the chunk,
    # explicit 16-row tiles); the array still holds call 1's scores
    r = slice(1000, 1064)
    ref = _ref(cs, 64, q0 + 1000, r)
    got = _noalloc(cs, 64, q0 + 1000, r, tile=16)
    assert torch.equal(got, ref)
    # an explicit tile too large for the array: refused, nothing enqueued
    idx = torch.full((T, wl.topk), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(dsv4.DSV4Error) as e:
        dsv4.dsv4_indexer_select_noalloc(cs.icache, cs.acache.n_rows, cs.q_idx, cs.w, T, q0,
                                         wl.idx_heads, wl.topk, idx, 512)
    assert e.value.code == -5 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((idx == -7).all())


def test_noalloc_select_narrow_at_1m_and_all_pooled():
    wl = SI.CTX_1M
    cs = ChunkState(wl, with_attn_q=False)
    S = cs.S
    # 3: four rows at the end of the 1M context (the chunk-parallel top-k,
    # its workspace placed after the scores inside the static array)
    q0 = 4 * S - 4
    ref = _ref(cs, 4, q0, slice(0, 4))
    got = _noalloc(cs, 4, q0, slice(0, 4))
    assert torch.equal(got, ref)
    # all-pooled: no scoring, no scratch, q and w not read
    small = dsv4.PoolCache(64, wl.idx_dim)
    small.set_state(40, 0)
    idx = torch.full((8, 64), -7, dtype=torch.int32, device="cuda")
    assert dsv4.dsv4_indexer_select_noalloc(small, 40, None, None, 8, 152, wl.idx_heads, 64, idx)
    torch.cuda.synchronize()
    want = np.full((8, 64), -1, np.int32)
    for t in range(8):
        v = (152 + t + 1) // 4
        want[t, :v] = np.arange(v)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
