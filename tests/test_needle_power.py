"""CPU checks of the needle attention cases the full-size GPU parity tests
use: every 32-key group of every query is decisive (leaving it out or
counting it twice moves the fp64 output by more than 4x the 2e-2 bar), and a
planted mistake in an output -- computed by the oracle with one group of
selection slots dropped, repeated or replaced -- fails the check.  The
ratio-128 mode's pooled rows are small (N(0, 1/128)), so there the bar is
a quarter of each head's own power instead (checked in check_needle_rows)."""
import math

import numpy as np
import pytest

import synthetic_inputs as SI
from oracle import dsv4_oracle as O

from parity_util import ATTN_ATOL, check_needle_rows, group_power, attention_keys, needle_queries


def _case(T=3, H=64, D=512, W=128, topk=512, q_pos0=4 * 8000, seed=5):
    rng = np.random.default_rng(seed)
    raw_pos0 = q_pos0 - W + 1
    raw = SI.as_bf16_values(rng.standard_normal((T + W - 1, D)).astype(np.float32))
    S = (q_pos0 + T) // 4
    pooled = SI.as_bf16_values((rng.standard_normal((S, D)) * 0.5).astype(np.float32))
    sel = np.full((T, topk), -1, np.int32)
    for t in range(T):
        v = O.visible_rows(q_pos0 + t)
        sel[t] = np.sort(rng.choice(v, size=topk, replace=False))
    scale = 1 / math.sqrt(D)
    q = needle_queries(T, q_pos0, H, W, raw, raw_pos0, pooled, sel, scale, seed=seed)
    return q, q_pos0, W, raw, raw_pos0, pooled, sel, scale


@pytest.mark.parametrize("topk", [512, 2048, 4096])
def test_every_group_is_decisive(topk):
    q, q_pos0, W, raw, raw_pos0, pooled, sel, scale = _case(T=2, topk=topk)
    for t in range(2):
        K, _ = attention_keys(t, q_pos0, W, raw, raw_pos0, pooled, sel)
        power = group_power(q[t], K, scale)
        assert np.all(power >= 4 * ATTN_ATOL), (topk, power.min())


def _planted(q, q_pos0, W, raw, raw_pos0, pooled, sel, scale, edit):
    bad = sel.copy()
    edit(bad)
    return O.sparse_prefill_attention(q, q_pos0, raw, raw_pos0, W, pooled, bad, scale)


@pytest.mark.parametrize("what", ["drop", "repeat", "replace", "none"])
def test_planted_group_mistake_fails(what):
    q, q_pos0, W, raw, raw_pos0, pooled, sel, scale = _case(T=2, topk=512)
    g = 7  # selection slots 32*(g-4) .. : the 8th group of keys (4 window groups first)
    a, b = 32 * (g - 4), 32 * (g - 3)

    def edit(s):
        if what == "drop":
            s[1, a:b] = -1
        elif what == "repeat":
            s[1, a + 32:b + 32] = s[1, a:b]     # the next group's slots replaced by this one's
        elif what == "replace":
            s[1, a:b] = (s[1, a:b] + 1000) % O.visible_rows(q_pos0 + 1)  # rows outside the group
    out = _planted(q, q_pos0, W, raw, raw_pos0, pooled, sel, scale, edit)
    run = lambda: check_needle_rows(out, [0, 1], q, q_pos0, W, raw, raw_pos0, pooled, sel, scale)
    if what == "none":
        run()
    else:
        with pytest.raises(AssertionError):
            run()
