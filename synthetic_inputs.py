"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and rounds them to the storage type; it holds
none of the method's arithmetic (no pooling, scoring, selection or attention),
so both the HIP path and the CPU oracle can be fed from it without sharing any
computation.

Every tensor has its own PCG64 stream, keyed by (seed, tensor name), so a
tensor's values do not depend on which other tensors were drawn first.

Workloads follow the context lengths and chunk sizes the pages measure at
(4K to 1M tokens of context, 2,048- and 4,096-token prefill chunks, index
top-k 512 / 2,048, 64 indexer heads x 128, attention B=1, H=64, D=512 bf16,
128-token sliding window).  Value distributions: raw keys, queries and KV
rows N(0, 1); head weights U(0, 1); pooled prefix rows N(0, 1/4), which is
the law of a mean of four independent N(0, 1) rows, drawn directly so that a
1M-token prefix does not have to be generated and pooled token by token.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np
import torch


def stream(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for one named tensor."""
    tag = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag])))


def normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    return (stream(seed, name).standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def uniform(seed: int, name: str, shape) -> np.ndarray:
    return stream(seed, name).random(size=shape, dtype=np.float32)


def as_bf16(a: np.ndarray):
    """(bf16 torch tensor on CPU, float32 numpy copy of exactly those values)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t, t.to(torch.float32).numpy()


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    prefix_tokens: int      # tokens already pooled before the measured chunk (multiple of 4)
    chunk: int              # query rows of the measured chunk (global prefill chunk)
    tile_rows: int          # indexer score/top-k tile (0 = whole chunk)
    topk: int
    idx_heads: int
    idx_dim: int
    heads: int
    head_dim: int
    window: int
    capacity_rows: int      # pooled-row capacity of each cache
    bf16: bool = True

    @property
    def q_pos0(self) -> int:
        return self.prefix_tokens

    @property
    def n_rows_after(self) -> int:
        return (self.prefix_tokens + self.chunk) // 4

    def visible_pairs(self) -> int:
        return sum((p + 1) // 4 for p in range(self.q_pos0, self.q_pos0 + self.chunk))


# Tiny CPU-checkable case: 64-token prefill from an empty cache.
TINY = Workload("tiny-64tok", 0, 64, 0, 8, 4, 32, 4, 32, 16, 16, bf16=False)
# 4K context: one 2,048-token chunk after a 2,048-token prefix -> 1,024 pooled rows.
CTX_4K = Workload("ctx4k-chunk2048", 2048, 2048, 0, 512, 64, 128, 64, 512, 128, 1024)
# 16K context, last of eight 2,048-token chunks (the first four take the all-pooled path).
CTX_16K = Workload("ctx16k-chunk2048", 14336, 2048, 0, 2048, 64, 128, 64, 512, 128, 4096)
# 128K context, last 2,048-token chunk -> 32,768 pooled rows.
CTX_128K = Workload("ctx128k-chunk2048", 129024, 2048, 0, 2048, 64, 128, 64, 512, 128, 32768)
# 1M context, last 4,096-token global chunk, score/top-k tiled at 1,024 rows.
CTX_1M = Workload("ctx1m-chunk4096-tile1024", 1044480, 4096, 1024, 2048, 64, 128, 64, 512, 128, 262144)

WORKLOADS = {w.name: w for w in (TINY, CTX_4K, CTX_16K, CTX_128K, CTX_1M)}


def make_inputs(wl: Workload, seed: int = 0, with_attn_q: bool = True) -> dict:
    """Host inputs for one chunk of ``wl``.

    Returns float32 numpy arrays whose values are exactly representable in
    bf16 when ``wl.bf16`` (tiny case: plain float32), plus the matching torch
    CPU tensors under ``*_t`` keys:

      prefix_idx_rows [prefix/4, idx_dim], prefix_attn_rows [prefix/4, head_dim]
      idx_keys  [chunk, idx_dim]     raw index keys of the chunk
      raw_kv    [chunk + window - 1, head_dim], raw_pos0 = q_pos0 - window + 1
                (clipped at 0): the raw rows the chunk's windows need
      q_idx     [chunk, idx_heads, idx_dim], w [chunk, idx_heads] (float32)
      q_attn    [chunk, heads, head_dim]
    """
    assert wl.prefix_tokens % 4 == 0
    n_prefix = wl.prefix_tokens // 4
    raw_pos0 = max(0, wl.q_pos0 - wl.window + 1)
    n_raw = wl.q_pos0 + wl.chunk - raw_pos0
    arrays = {
        "prefix_idx_rows": normal(seed, "prefix_idx_rows", (n_prefix, wl.idx_dim), 0.5),
        "prefix_attn_rows": normal(seed, "prefix_attn_rows", (n_prefix, wl.head_dim), 0.5),
        "idx_keys": normal(seed, "idx_keys", (wl.chunk, wl.idx_dim)),
        "raw_kv": normal(seed, "raw_kv", (n_raw, wl.head_dim)),
        "q_idx": normal(seed, "q_idx", (wl.chunk, wl.idx_heads, wl.idx_dim)),
    }
    if with_attn_q:
        arrays["q_attn"] = normal(seed, "q_attn", (wl.chunk, wl.heads, wl.head_dim))
    out = {"raw_pos0": raw_pos0, "q_pos0": wl.q_pos0}
    for k, a in arrays.items():
        if wl.bf16:
            t, v = as_bf16(a)
        else:
            t, v = torch.from_numpy(a), a
        out[k], out[k + "_t"] = v, t
    w = uniform(seed, "w", (wl.chunk, wl.idx_heads))
    out["w"], out["w_t"] = w, torch.from_numpy(w)
    return out


def prefix_rows_ratio(wl: Workload, seed: int, ratio: int):
    """Pooled prefix rows of a ratio-``ratio`` cache for ``wl`` (the
    CompressedAttention pool at ratio 128): [prefix_tokens // ratio,
    head_dim] drawn as N(0, 1/ratio), the law of a mean of ``ratio``
    independent N(0, 1) rows, rounded to bf16.  Returns (torch CPU tensor,
    float32 numpy values)."""
    n = wl.prefix_tokens // ratio
    a = normal(seed, f"prefix_attn_rows_r{ratio}", (n, wl.head_dim), float(1.0 / np.sqrt(ratio)))
    return as_bf16(a)


def as_bf16_values(a: np.ndarray) -> np.ndarray:
    """Values of ``a`` rounded to bf16 (used to feed a float32 tiny case to
    bf16-only kernels)."""
    return as_bf16(a)[1]
