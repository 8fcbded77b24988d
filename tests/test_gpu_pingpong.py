"""Ping-pong score scratch with overlap, through the C ABI.

[P3 "[Discussion] Tile indexed-attention scoring independently of the global
prefill chunk", Possible design: score a bounded query-row tile into a
scratch, select, and reuse the scratch, optionally with ping-pong buffers or
careful overlap.]  A 4,096-row chunk at 1M tokens of context is scored in
1,024-row tiles on one stream into two alternating scratch buffers, while the
top-k of the previous tile runs on a second stream (two-pass split top-k,
with its own workspace per buffer); events order each buffer's reuse.  The
selection must be bit-identical to the library's serial one-scratch select,
and match the oracle on rows spread over every tile.
"""
import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import ChunkState, assert_selection_matches, spread_rows

pytestmark = pytest.mark.gpu


def test_pingpong_two_streams_matches_serial_and_oracle():
    wl = SI.CTX_1M
    cs = ChunkState(wl, with_attn_q=False)
    T, S, k, tile = wl.chunk, cs.S, wl.topk, wl.tile_rows
    q0 = cs.q_pos0
    stride = dsv4.dsv4_score_stride(S)
    # serial: one scratch reused by every tile
    scratch = torch.empty((tile, stride), device="cuda")
    ref_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    assert not dsv4.dsv4_indexer_select(cs.icache, cs.acache.n_rows, cs.q_idx, cs.w, T, q0,
                                        wl.idx_heads, k, ref_idx, scratch, tile)
    torch.cuda.synchronize()
    del scratch
    # ping-pong: two scratches, scores on `main`, top-k on `aux`
    bufs = [torch.empty((tile, stride), device="cuda") for _ in range(2)]
    nb_ws = dsv4.dsv4_topk_split_workspace_bytes(tile, q0 + T - tile, k)
    assert nb_ws > 0   # rows longer than one 32,768-column chunk: two passes
    wss = [torch.empty(nb_ws // 4, device="cuda") for _ in bufs]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    main, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    ev_sc = [torch.cuda.Event() for _ in bufs]
    ev_tk = [torch.cuda.Event() for _ in bufs]
    start = torch.cuda.Event()
    start.record(main)
    aux.wait_event(start)
    for i, t0 in enumerate(range(0, T, tile)):
        b = i % 2
        if i >= 2:
            main.wait_event(ev_tk[b])      # the buffer's previous top-k is done
        dsv4.dsv4_indexer_scores(cs.icache, cs.q_idx[t0:t0 + tile], cs.w[t0:t0 + tile],
                                 q0 + t0, bufs[b], True, stream=main)
        ev_sc[b].record(main)
        aux.wait_event(ev_sc[b])
        dsv4.dsv4_topk_select_split(bufs[b], q0 + t0, S, k, idx[t0:t0 + tile], wss[b],
                                    stream=aux)
        ev_tk[b].record(aux)
    for e in ev_tk:
        main.wait_event(e)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    gidx = idx.cpu().numpy()
    keys = cs.oracle_keys()
    for t in spread_rows(T, 32, tile=tile, seed=44):
        ref = O.indexer_scores(cs.inp["q_idx"][t:t + 1], cs.inp["w"][t:t + 1], keys, q0 + t, S)
        assert_selection_matches(gidx[t:t + 1], ref, q0 + t, k)
