"""The hot path under HIP graph capture: the library allocates nothing and
enqueues only kernels on the caller's stream, so a whole step (both
compressions, the indexer select, the attention) can be captured once and
replayed.  Every replay, with eager work and synchronisations between the
replays, must give the eager step's outputs bit for bit (the kernels are
deterministic and a replay rewrites the same cache rows)."""
import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI

from parity_util import bf16_t

pytestmark = pytest.mark.gpu


def _state(wl, seed=0):
    inp = SI.make_inputs(wl, seed)
    n_prefix = wl.prefix_tokens // 4
    ic = dsv4.PoolCache(wl.capacity_rows, wl.idx_dim)
    ac = dsv4.PoolCache(wl.capacity_rows, wl.head_dim)
    ic.rows[:n_prefix].copy_(inp["prefix_idx_rows_t"])
    ac.rows[:n_prefix].copy_(inp["prefix_attn_rows_t"])
    return inp, n_prefix, ic, ac


@pytest.mark.parametrize("narrow", [False, True], ids=["chunk2048", "narrow-T2"])
def test_step_graph_replays_match_eager(narrow):
    wl = SI.CTX_4K
    inp, n_prefix, ic, ac = _state(wl)
    T = 2 if narrow else wl.chunk
    q_pos0 = wl.q_pos0
    raw_kv = inp["raw_kv_t"].cuda()
    chunk_kv = raw_kv[q_pos0 - inp["raw_pos0"]:][:T]
    idx_keys = inp["idx_keys_t"].cuda()[:T]
    q_idx, w = inp["q_idx_t"].cuda()[:T], inp["w_t"].cuda()[:T]
    q_attn = inp["q_attn_t"].cuda()[:T]
    S_after = (wl.prefix_tokens + T) // 4
    scratch = torch.empty(dsv4.dsv4_indexer_scratch_bytes(T, S_after) // 4, device="cuda")
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, wl.heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    ns, nb = dsv4.dsv4_sparse_attn_narrow_plan(T, wl.heads, wl.head_dim, wl.window, wl.topk)
    ws = torch.empty(max(nb // 4, 4), device="cuda")

    def step():
        ic.set_state(n_prefix, 0)
        ac.set_state(n_prefix, 0)
        dsv4.dsv4_compress(ac, chunk_kv)
        dsv4.dsv4_compress(ic, idx_keys)
        dsv4.dsv4_indexer_select(ic, ac.n_rows, q_idx, w, T, q_pos0, wl.idx_heads, wl.topk, idx,
                                 scratch, 0)
        if narrow:
            dsv4.dsv4_sparse_attn_narrow(q_attn, q_pos0, raw_kv, inp["raw_pos0"], wl.window, ac,
                                         idx, out, ns, ws)
        else:
            dsv4.dsv4_sparse_prefill_attn(q_attn, q_pos0, raw_kv, inp["raw_pos0"], wl.window, ac,
                                          idx, out)

    step()
    torch.cuda.synchronize()
    want = (idx.clone(), out.clone(), ic.rows.clone(), ac.rows.clone())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work between replays: clobber the outputs and the cache rows
        idx.fill_(-7)
        out.zero_()
        ic.rows[n_prefix:].zero_()
        ac.rows[n_prefix:].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want[0]), r
        assert torch.equal(out, want[1]), r
        assert torch.equal(ic.rows, want[2]) and torch.equal(ac.rows, want[3]), r


def test_long_row_select_graph_replays_match_eager():
    """The indexer select over rows longer than one 32,768-column chunk (the
    score kernel, then the two register top-k passes with the chunks' winners
    kept in the scratch) captured once and replayed, with the outputs and the
    scratch clobbered by eager work between replays."""
    T, S, topk = 64, 70000, 2048
    gen = torch.Generator(device="cuda").manual_seed(5)
    ic = dsv4.PoolCache(S, 128)
    ic.rows.copy_((torch.randn(S, 128, device="cuda", generator=gen) * 0.5).to(torch.bfloat16))
    ic.set_state(S)
    q_pos0 = 4 * S - T
    q = torch.randn(T, 64, 128, device="cuda", generator=gen).to(torch.bfloat16)
    w = torch.rand(T, 64, device="cuda", generator=gen)
    scratch = torch.empty(dsv4.dsv4_indexer_scratch_bytes(T, S) // 4, device="cuda")
    idx = torch.empty((T, topk), dtype=torch.int32, device="cuda")

    def step():
        assert not dsv4.dsv4_indexer_select(ic, S, q, w, T, q_pos0, 64, topk, idx, scratch, 0)

    step()
    torch.cuda.synchronize()
    want = idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        idx.fill_(-7)
        scratch.fill_(float(r) - 1.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want), r
