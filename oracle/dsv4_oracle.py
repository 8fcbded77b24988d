"""Plain CPU oracle for DeepSeek-V4 indexed-attention prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports or calls it, and this
module imports nothing from the product path.

Everything here is the slow, obvious definition, written from the pages:

  [P1] "perf(deepseek-v4): skip redundant all-pooled indexer scoring"
       (oMLX pull request 2563) -- Summary, Correctness.
  [P2] "perf(deepseek_v4): faster exact DeepSeek-V4 prefill (wsdpa fusion +
       scheduler/cache amortization)" (oMLX pull request 2568) -- Summary
       commits 1, 4 and 5, Performance, Output-parity note.
  [P3] "[Discussion] Tile indexed-attention scoring independently of the
       global prefill chunk" (ds4 issue 644) -- Summary, Possible design,
       Correctness questions.

Floating point is fp64 except where a step's rounding is itself part of the
definition (the compressor stores fp32-accumulated, bf16-rounded rows, see
``compress``).  Readings taken where the pages are silent are marked
"Reading:" and each is listed with its reason in the design notes.

Pins: every function below is pinned by ``tests/test_oracle_pins.py`` against
worked examples from the pages (``tests/golden/``), closed forms, brute force
on tiny inputs and independent library routines.  The one part without such a
pin is agreement with the real DeepSeek-V4 model numerics (pooling function,
indexer scale, softmax scale): parity unpinned there, since no model weights
or model outputs exist to compare against.
"""
from __future__ import annotations

import math

import numpy as np

RATIO = 4  # [P1 Correctness]: ratio-4 compressor (10 tokens -> 2 rows + 2 left over)


# --------------------------------------------------------------------------
# Rounding helpers (definition of storage rounding, not of the method)
# --------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    Returns float32 values that are exactly representable in bfloat16.
    bfloat16 keeps the top 16 bits of an IEEE binary32 value; rounding adds
    0x7FFF plus the lowest kept bit before truncating (round half to even).
    Inputs are assumed finite (NaN/inf are out of scope).
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return rounded.astype(np.uint32).view(np.float32).reshape(a.shape)


# --------------------------------------------------------------------------
# Compressor and PoolingCache  [P1 Summary, Correctness; P2 commit 4]
# --------------------------------------------------------------------------

class PoolingCacheState:
    """Host model of one compressor's PoolingCache.

    Holds the pooled rows appended so far (``rows[:n_rows]``), and the raw
    tokens not yet pooled (``rem``, fewer than ``ratio`` of them).  Pooled rows
    are appended in place at offset ``n_rows`` [P2 commit 4].  ``ratio`` is 4
    on the indexer's path; the sibling CompressedAttention mode pools 128 rows
    [P2 commit 1 and the rebase note: ratio-128 prefill].
    """

    def __init__(self, dim: int, capacity: int, out_bf16: bool = True, ratio: int = RATIO):
        self.dim = dim
        self.capacity = capacity
        self.out_bf16 = out_bf16
        self.ratio = ratio
        self.rows = np.zeros((capacity, dim), dtype=np.float32)
        self.n_rows = 0
        self.rem = np.zeros((0, dim), dtype=np.float32)

    @property
    def n_rem(self) -> int:
        return int(self.rem.shape[0])

    @property
    def tokens_consumed(self) -> int:
        # Reading: groups are aligned to absolute position 0, so the stream
        # position of the next raw token is ratio * n_rows + n_rem.
        return self.ratio * self.n_rows + self.n_rem

    def copy(self) -> "PoolingCacheState":
        c = PoolingCacheState(self.dim, self.capacity, self.out_bf16, self.ratio)
        c.rows = self.rows.copy()
        c.n_rows = self.n_rows
        c.rem = self.rem.copy()
        return c


def pool_group(tokens_f32: np.ndarray, out_bf16: bool) -> np.ndarray:
    """One pooled row from ``r`` consecutive raw rows (r = the ratio, 4 or 128).

    Reading (pages name a ratio-4 "pooling" but give no formula): mean pool.
    The sum is taken in float32, strictly left to right, ((a+b)+c)+d..., each
    add rounded to float32, then multiplied by 1/r (exact for a power of two)
    and rounded to the storage type (bfloat16, ties to even).  No fused
    multiply-add.  The same reading serves the ratio-128 pool.
    """
    r = tokens_f32.shape[0]
    t = tokens_f32.astype(np.float32)
    acc = t[0].copy()
    for i in range(1, r):
        acc = (acc + t[i]).astype(np.float32)  # one float32 rounding per add
    mean = (acc * np.float32(1.0 / r)).astype(np.float32)
    return round_to_bf16(mean) if out_bf16 else mean


def compress(state: PoolingCacheState, x) -> int:
    """Feed ``x`` ([n_new, dim] raw rows) through the state's compressor.

    [P1 Correctness]: a non-aligned ratio-4 prefill of 10 tokens yields two
    pooled rows and a two-token remainder; the remainder is carried into the
    next call.  The concatenation (old remainder, new rows) is cut into groups
    of ``ratio``; each whole group becomes one pooled row appended at ``n_rows``
    [P2 commit 4]; what is left becomes the new remainder.
    Returns the number of rows appended.  Raises ValueError when the append
    would pass ``capacity`` (state unchanged).
    """
    x = np.asarray(x, dtype=np.float32).reshape(-1, state.dim)
    cat = np.concatenate([state.rem, x], axis=0)
    r = state.ratio
    groups = cat.shape[0] // r
    if state.n_rows + groups > state.capacity:
        raise ValueError("pooled rows would exceed capacity")
    for j in range(groups):
        state.rows[state.n_rows + j] = pool_group(cat[r * j: r * j + r], state.out_bf16)
    state.n_rows += groups
    state.rem = cat[r * groups:].copy()
    return groups


# --------------------------------------------------------------------------
# Pooled-row visibility  [P2 commit 1 and commit 5]
# --------------------------------------------------------------------------

def visible_rows(p: int, ratio: int = RATIO) -> int:
    """Number of pooled rows a query at absolute position ``p`` may see.

    [P2 commit 1] rebuilds pooled visibility from offsets; [P2 commit 5]
    names it the pooled-ratio causal mask.  Reading: with ratio r, pooled row
    s summarises tokens r*s .. r*s+r-1, and is visible to position p once all
    of them are at or before p, i.e. r*(s+1) <= p+1.  Counting those s gives
    floor((p+1)/r).
    """
    return (p + 1) // ratio


# --------------------------------------------------------------------------
# Indexer path decision  [P1 Summary, Correctness]
# --------------------------------------------------------------------------

def indexer_path(n_index_rows: int, n_attn_rows: int, topk: int) -> str:
    """Which indexer path a chunk takes.

    [P1 Summary]: guard against divergence of the attention and indexer
    compressor row counts; skip projection, scoring and top-k when every pooled
    row already fits within index_topk; keep the full path for empty pools and
    for pools larger than index_topk.
    """
    if n_index_rows != n_attn_rows:
        raise ValueError("attention / indexer pooled row counts diverge")
    if n_index_rows == 0:
        return "empty"
    if n_index_rows <= topk:
        return "all_pooled"
    return "full"


def all_pooled_selection(T: int, q_pos0: int, topk: int) -> np.ndarray:
    """[P1 Correctness]: the selection holds the sequential pooled indices.

    Row t (position q_pos0+t) lists 0 .. visible_rows(p)-1, then -1 padding.
    """
    out = np.full((T, topk), -1, dtype=np.int32)
    for t in range(T):
        v = visible_rows(q_pos0 + t)
        out[t, :v] = np.arange(v, dtype=np.int32)
    return out


# --------------------------------------------------------------------------
# Indexer score  [P2 commit 5, Performance; P3 Summary]
# --------------------------------------------------------------------------

def indexer_scores(q, w, K, q_pos0: int, S: int, fold_mask: bool = True) -> np.ndarray:
    """Indexer scores of T query rows against S pooled index keys, fp64.

    q: [T, H, D] indexer queries, w: [T, H] per-head weights, K: [>=S, D]
    pooled index keys (one key per pooled row shared by all heads -- reading).
    The DSA indexer [P2 Performance] scores every visible pooled row:
        score[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . K[s, :])
    With ``fold_mask`` the pooled-ratio causal mask [P2 commit 5] is applied:
    entries with s >= visible_rows(q_pos0 + t) are -inf (the sentinel --
    reading, the pages give no value).  Without it every s < S is scored.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Kd = np.asarray(K, dtype=np.float64)[:S]
    T = q.shape[0]
    out = np.empty((T, S), dtype=np.float64)
    for t in range(T):
        dots = q[t] @ Kd.T                      # [H, S]
        out[t] = w[t] @ np.maximum(dots, 0.0)   # sum over heads
    if fold_mask:
        out = apply_pooled_mask(out, q_pos0)
    return out


def apply_pooled_mask(scores, q_pos0: int) -> np.ndarray:
    """Second-pass form of the pooled-ratio causal mask [P2 commit 5]: the
    same sentinel (-inf) written where s >= visible_rows(q_pos0 + t)."""
    out = np.array(scores, dtype=np.float64, copy=True)
    for t in range(out.shape[0]):
        out[t, visible_rows(q_pos0 + t):] = -np.inf
    return out


# --------------------------------------------------------------------------
# Top-k selection  [P1 Summary; P3 Possible design step 3]
# --------------------------------------------------------------------------

def topk_row(scores_row, n_visible: int, topk: int) -> np.ndarray:
    """Selection for one query row.

    Takes the min(topk, n_visible) visible rows with the highest score; equal
    scores go to the lower index; the chosen indices are written in ascending
    order and the rest of the topk slots hold -1.  Masked rows are never
    chosen.  (Readings: order and tie rule are not on the pages; ascending
    order makes the result equal the sequential all-pooled selection of
    [P1 Correctness] whenever every visible row fits.)
    """
    s = np.asarray(scores_row, dtype=np.float64)[:n_visible]
    k_eff = min(topk, n_visible)
    idx = np.arange(n_visible)
    order = np.lexsort((idx, -s))  # primary: score descending; ties: index ascending
    chosen = np.sort(order[:k_eff])
    out = np.full(topk, -1, dtype=np.int32)
    out[:k_eff] = chosen
    return out


def topk_select(scores, q_pos0: int, topk: int) -> np.ndarray:
    """Row-wise ``topk_row`` over a [T, >=S] score block for queries at
    positions q_pos0 .. q_pos0+T-1."""
    scores = np.asarray(scores)
    T = scores.shape[0]
    out = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        out[t] = topk_row(scores[t], visible_rows(q_pos0 + t), topk)
    return out


def indexer_select(q, w, K, n_attn_rows: int, T: int, q_pos0: int, topk: int, S: int,
                   tile_rows: int = 0):
    """Whole indexer step for one chunk of T query rows: guard, path, then
    score + top-k in query-row tiles of ``tile_rows`` ([P3 Possible design]:
    score a tile, select, reuse the scratch for the next tile).
    Returns (idx [T, topk] int32, all_pooled flag).  q and w are not read on
    the all-pooled and empty paths [P1 Summary].
    """
    path = indexer_path(S, n_attn_rows, topk)
    if path == "empty":
        return np.full((T, topk), -1, dtype=np.int32), False
    if path == "all_pooled":
        return all_pooled_selection(T, q_pos0, topk), True
    q = np.asarray(q)
    tile = T if tile_rows <= 0 else tile_rows
    out = np.empty((T, topk), dtype=np.int32)
    for t0 in range(0, T, tile):
        t1 = min(T, t0 + tile)
        sc = indexer_scores(q[t0:t1], np.asarray(w)[t0:t1], K, q_pos0 + t0, S)
        out[t0:t1] = topk_select(sc, q_pos0 + t0, topk)
    return out, False


# --------------------------------------------------------------------------
# Fused windowed + pooled attention  [P2 commit 1; P3 Possible design step 4]
# --------------------------------------------------------------------------

def sparse_prefill_attention(q, q_pos0: int, raw_kv, raw_pos0: int, window: int,
                             pooled, sel_idx, scale: float, ratio: int = RATIO) -> np.ndarray:
    """Windowed + pooled attention for T queries, fp64.

    [P2 commit 1]: one attention over the sliding raw-token window plus the
    pooled rows (all visible ones on the small-pool path, the selected ones on
    the indexer top-k path), with causality, window and pooled visibility
    rebuilt from offsets.

    q: [T, H, D]; raw_kv: [n_raw, D] raw rows for positions raw_pos0.. ;
    pooled: [>=S, D] pooled rows, or None for the window-only mode (the
    LocalAttention sibling of [P2 commit 1]: no pooled keys at all); sel_idx:
    [T, k] int (-1 = empty slot) or None for "every visible pooled row" (the
    CompressedAttention sibling, ratio 128, and the small-pool path).
    ``ratio`` is the pool's ratio, used for pooled visibility.  Readings: keys
    and values are the same rows shared by all heads; the window holds
    positions p-window+1 .. p (clipped at 0); a pooled row is a key distinct
    from the raw rows (both are attended); no sink, no extra bias; softmax in
    fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    raw = np.asarray(raw_kv, dtype=np.float64)
    if pooled is not None:
        pooled = np.asarray(pooled, dtype=np.float64)
    T, H, D = q.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    for t in range(T):
        p = q_pos0 + t
        lo = max(0, p - window + 1)
        keys = [raw[j - raw_pos0] for j in range(lo, p + 1)]
        vis = 0 if pooled is None else visible_rows(p, ratio)
        if sel_idx is None:
            chosen = list(range(vis))
        else:
            chosen = [int(s) for s in np.asarray(sel_idx)[t] if 0 <= int(s) < vis]
        keys += [pooled[s] for s in chosen]
        Kt = np.stack(keys, axis=0)               # [n_keys, D]
        logits = scale * (q[t] @ Kt.T)            # [H, n_keys]
        logits -= logits.max(axis=1, keepdims=True)
        pr = np.exp(logits)
        pr /= pr.sum(axis=1, keepdims=True)
        out[t] = pr @ Kt                          # values are the keys
    return out
