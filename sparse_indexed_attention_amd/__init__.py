"""Python binding of libdsv4 (include/dsv4.h): DeepSeek-V4 indexed-attention
prefill on MI355X (gfx950).

Argument marshalling only.  Every function passes torch tensors' device
pointers, sizes and the current HIP stream to the C ABI of the same name;
all work runs in the HIP kernels of ``libdsv4.so``.  There is no fallback:
if the library is missing or fails to load, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "DSV4Error", "PoolCache", "lib", "header_functions",
    "dsv4_abi_version", "dsv4_last_error", "dsv4_indexer_all_pooled", "dsv4_score_stride",
    "dsv4_indexer_scratch_bytes", "dsv4_compress", "dsv4_indexer_scores", "dsv4_topk_select",
    "dsv4_indexer_select", "dsv4_sparse_prefill_attn", "dsv4_sparse_attn_narrow_plan",
    "dsv4_sparse_attn_narrow", "dsv4_topk_split_workspace_bytes", "dsv4_topk_select_split",
    "dsv4_indexer_select_noalloc", "DSV4_NOALLOC_SCRATCH_BYTES", "DSV4_MAX_EXTENT",
    "use_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsv4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dsv4.h")

DSV4_BF16 = 1
DSV4_F32 = 2
DSV4_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
DSV4_MAX_EXTENT = 1 << 40  # largest position / count / size / stride any call takes
RATIO = 4

c_i32, c_i64, c_vp, c_f32, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


class dsv4_pool_cache(ctypes.Structure):
    _fields_ = [("rows", c_vp), ("rem", c_vp), ("capacity", c_i64), ("n_rows", c_i64),
                ("n_rem", c_i32), ("ratio", c_i32), ("dim", c_i32), ("dtype", c_i32)]


class DSV4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dsv4 error {code}: {message}")
        self.code = code


_SIGNATURES = {
    "dsv4_abi_version": (c_i32, []),
    "dsv4_last_error": (ctypes.c_char_p, []),
    "dsv4_indexer_all_pooled": (c_i32, [c_i64, c_i32]),
    "dsv4_score_stride": (c_i64, [c_i64]),
    "dsv4_indexer_scratch_bytes": (c_i32, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "dsv4_compress": (c_i32, [ctypes.POINTER(dsv4_pool_cache), c_vp, c_i64, c_vp]),
    "dsv4_indexer_scores": (c_i32, [ctypes.POINTER(dsv4_pool_cache), c_vp, c_vp, c_i64, c_i64,
                                    c_i32, c_i32, c_vp, c_i64, c_vp]),
    "dsv4_topk_select": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp]),
    "dsv4_indexer_select": (c_i32, [ctypes.POINTER(dsv4_pool_cache), c_i64, c_vp, c_vp, c_i64,
                                    c_i64, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp,
                                    ctypes.POINTER(c_i32), c_vp]),
    "dsv4_sparse_prefill_attn": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_i32, c_f32, c_vp, c_i64,
                                         c_i64, c_i32, ctypes.POINTER(dsv4_pool_cache), c_vp,
                                         c_i32, c_vp, c_vp]),
    "dsv4_topk_split_workspace_bytes": (c_i32, [c_i64, c_i64, c_i32, ctypes.POINTER(c_sz)]),
    "dsv4_topk_select_split": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_sz,
                                       c_vp]),
    "dsv4_sparse_attn_narrow_plan": (c_i32, [c_i64, c_i32, c_i32, c_i32, c_i64,
                                             ctypes.POINTER(c_i32), ctypes.POINTER(c_sz)]),
    "dsv4_sparse_attn_narrow": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_i32, c_f32, c_vp, c_i64,
                                        c_i64, c_i32, ctypes.POINTER(dsv4_pool_cache), c_vp,
                                        c_i32, c_i32, c_vp, c_sz, c_vp, c_vp]),
    "dsv4_indexer_select_noalloc": (c_i32, [ctypes.POINTER(dsv4_pool_cache), c_i64, c_vp, c_vp,
                                            c_i64, c_i64, c_i32, c_i32, c_i32, c_vp,
                                            ctypes.POINTER(c_i32), c_vp]),
}

_lib = None


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m sparse_indexed_attention_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """Load libdsv4.so (built by ``python -m sparse_indexed_attention_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def use_library(path_or_handle) -> ctypes.CDLL:
    """Make the functions below call another build of the library (a path,
    or a handle this function returned before); returns the handle now in
    use.  Two builds can be loaded side by side, e.g. for an interleaved
    timing comparison in one process."""
    global _lib
    _lib = path_or_handle if isinstance(path_or_handle, ctypes.CDLL) else _load(path_or_handle)
    return _lib


def header_functions() -> list:
    """Names of the functions include/dsv4.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv4_[a-z_]+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        raise DSV4Error(rc, lib().dsv4_last_error().decode())


def _stream(stream):
    if stream is None:
        return c_vp(torch.cuda.current_stream().cuda_stream)
    return c_vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return None if t is None else c_vp(t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str, dims: int):
    if t.dtype != dtype or not t.is_contiguous() or t.dim() != dims or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {dims}-d {dtype} CUDA tensor, got "
                         f"{t.dtype} shape {tuple(t.shape)} contiguous={t.is_contiguous()} "
                         f"device={t.device}")


class PoolCache:
    """A PoolingCache: device rows [capacity, dim] and remainder
    [ratio - 1, dim] (torch tensors) plus the host struct the C ABI reads and
    updates.  ratio 4 serves the indexer and sparse attention, ratio 128 the
    CompressedAttention mode."""

    def __init__(self, capacity: int, dim: int, dtype=torch.bfloat16, device="cuda",
                 ratio: int = RATIO):
        self.rows = torch.zeros((capacity, dim), dtype=dtype, device=device)
        self.rem = torch.zeros((max(ratio - 1, 1), dim), dtype=dtype, device=device)
        self.struct = dsv4_pool_cache(self.rows.data_ptr(), self.rem.data_ptr(), capacity, 0, 0,
                                      ratio, dim, DSV4_BF16 if dtype == torch.bfloat16 else DSV4_F32)

    @property
    def n_rows(self) -> int:
        return int(self.struct.n_rows)

    @property
    def n_rem(self) -> int:
        return int(self.struct.n_rem)

    @property
    def dim(self) -> int:
        return int(self.struct.dim)

    @property
    def capacity(self) -> int:
        return int(self.struct.capacity)

    @property
    def ratio(self) -> int:
        return int(self.struct.ratio)

    def set_state(self, n_rows: int, n_rem: int = 0):
        """Declare rows [0, n_rows) and remainder [0, n_rem) valid (after the
        caller wrote them, e.g. restoring a saved state)."""
        self.struct.n_rows = n_rows
        self.struct.n_rem = n_rem

    def ref(self):
        return ctypes.byref(self.struct)


# ------------------------------------------------------------------ wrappers

def dsv4_abi_version() -> int:
    return int(lib().dsv4_abi_version())


def dsv4_last_error() -> str:
    return lib().dsv4_last_error().decode()


def dsv4_indexer_all_pooled(n_rows: int, topk: int) -> bool:
    return bool(lib().dsv4_indexer_all_pooled(n_rows, topk))


def dsv4_score_stride(n_rows: int) -> int:
    return int(lib().dsv4_score_stride(n_rows))


def dsv4_indexer_scratch_bytes(tile_rows: int, max_rows: int) -> int:
    b = c_sz(0)
    _check(lib().dsv4_indexer_scratch_bytes(tile_rows, max_rows, ctypes.byref(b)))
    return int(b.value)


def dsv4_compress(cache: PoolCache, x: torch.Tensor, stream=None) -> None:
    _need(x, cache.rows.dtype, "x", 2)
    _check(lib().dsv4_compress(cache.ref(), _ptr(x), x.shape[0], _stream(stream)))


def dsv4_indexer_scores(index_cache: PoolCache, q: torch.Tensor, w: torch.Tensor, q_pos0: int,
                        out: torch.Tensor, fold_mask: bool = True, stream=None) -> None:
    _need(q, torch.bfloat16, "q", 3)
    _need(w, torch.float32, "w", 2)
    _need(out, torch.float32, "out", 2)
    _check(lib().dsv4_indexer_scores(index_cache.ref(), _ptr(q), _ptr(w), q.shape[0], q_pos0,
                                     q.shape[1], 1 if fold_mask else 0, _ptr(out), out.shape[1],
                                     _stream(stream)))


def dsv4_topk_select(scores: torch.Tensor, q_pos0: int, n_cols: int, topk: int,
                     out_idx: torch.Tensor, stream=None) -> None:
    _need(scores, torch.float32, "scores", 2)
    _need(out_idx, torch.int32, "out_idx", 2)
    _check(lib().dsv4_topk_select(_ptr(scores), scores.shape[0], scores.shape[1], q_pos0, n_cols,
                                  topk, _ptr(out_idx), _stream(stream)))


def dsv4_topk_split_workspace_bytes(rows: int, q_pos0: int, topk: int) -> int:
    nb = c_sz(0)
    _check(lib().dsv4_topk_split_workspace_bytes(rows, q_pos0, topk, ctypes.byref(nb)))
    return int(nb.value)


def dsv4_topk_select_split(scores: torch.Tensor, q_pos0: int, n_cols: int, topk: int,
                           out_idx: torch.Tensor, workspace=None, stream=None) -> None:
    """Chunk-parallel top-k (same result as dsv4_topk_select); workspace: a
    CUDA tensor of at least dsv4_topk_split_workspace_bytes bytes, or None
    when that is 0."""
    _need(scores, torch.float32, "scores", 2)
    _need(out_idx, torch.int32, "out_idx", 2)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsv4_topk_select_split(_ptr(scores), scores.shape[0], scores.shape[1], q_pos0,
                                        n_cols, topk, _ptr(out_idx), _ptr(workspace), nbytes,
                                        _stream(stream)))


def dsv4_indexer_select(index_cache: PoolCache, n_attn_rows: int, q, w, T: int, q_pos0: int,
                        n_heads: int, topk: int, out_idx: torch.Tensor, scratch=None,
                        tile_rows: int = 0, stream=None) -> bool:
    """Returns True when the all-pooled path was taken (q, w unused)."""
    if q is not None:
        _need(q, torch.bfloat16, "q", 3)
    if w is not None:
        _need(w, torch.float32, "w", 2)
    _need(out_idx, torch.int32, "out_idx", 2)
    ap = c_i32(0)
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    _check(lib().dsv4_indexer_select(index_cache.ref(), n_attn_rows, _ptr(q), _ptr(w), T, q_pos0,
                                     n_heads, topk, tile_rows, _ptr(scratch), nbytes,
                                     _ptr(out_idx), ctypes.byref(ap), _stream(stream)))
    return bool(ap.value)


def dsv4_indexer_select_noalloc(index_cache: PoolCache, n_attn_rows: int, q, w, T: int,
                                q_pos0: int, n_heads: int, topk: int, out_idx: torch.Tensor,
                                tile_rows: int = 0, stream=None) -> bool:
    """dsv4_indexer_select with the library's static per-GPU scratch (no
    scratch argument, nothing allocated).  Returns True on the all-pooled
    path."""
    if q is not None:
        _need(q, torch.bfloat16, "q", 3)
    if w is not None:
        _need(w, torch.float32, "w", 2)
    _need(out_idx, torch.int32, "out_idx", 2)
    ap = c_i32(0)
    _check(lib().dsv4_indexer_select_noalloc(index_cache.ref(), n_attn_rows, _ptr(q), _ptr(w), T,
                                             q_pos0, n_heads, topk, tile_rows, _ptr(out_idx),
                                             ctypes.byref(ap), _stream(stream)))
    return bool(ap.value)


def dsv4_sparse_prefill_attn(q: torch.Tensor, q_pos0: int, raw_kv: torch.Tensor, raw_pos0: int,
                             window: int, attn_cache, sel_idx, out: torch.Tensor,
                             scale: float = 0.0, stream=None) -> None:
    """attn_cache: a PoolCache, or None for window-only attention (then
    sel_idx must be None too)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(raw_kv, torch.bfloat16, "raw_kv", 2)
    _need(out, torch.bfloat16, "out", 3)
    topk = 0
    if sel_idx is not None:
        _need(sel_idx, torch.int32, "sel_idx", 2)
        topk = sel_idx.shape[1]
    _check(lib().dsv4_sparse_prefill_attn(_ptr(q), q.shape[0], q_pos0, q.shape[1], q.shape[2],
                                          scale, _ptr(raw_kv), raw_pos0, raw_kv.shape[0], window,
                                          None if attn_cache is None else attn_cache.ref(),
                                          _ptr(sel_idx), topk, _ptr(out),
                                          _stream(stream)))


def dsv4_sparse_attn_narrow_plan(T: int, n_heads: int, head_dim: int, window: int,
                                 n_pooled_keys: int):
    """(n_splits, workspace_bytes) for narrow-query attention."""
    ns, nb = c_i32(0), c_sz(0)
    _check(lib().dsv4_sparse_attn_narrow_plan(T, n_heads, head_dim, window, n_pooled_keys,
                                              ctypes.byref(ns), ctypes.byref(nb)))
    return int(ns.value), int(nb.value)


def dsv4_sparse_attn_narrow(q: torch.Tensor, q_pos0: int, raw_kv: torch.Tensor, raw_pos0: int,
                            window: int, attn_cache, sel_idx, out: torch.Tensor, n_splits: int,
                            workspace=None, scale: float = 0.0, stream=None) -> None:
    """Narrow-query attention: as dsv4_sparse_prefill_attn, with each query's
    keys split over n_splits workgroups (workspace: a float32 CUDA tensor of
    at least the planned bytes, or None when n_splits == 1)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(raw_kv, torch.bfloat16, "raw_kv", 2)
    _need(out, torch.bfloat16, "out", 3)
    topk = 0
    if sel_idx is not None:
        _need(sel_idx, torch.int32, "sel_idx", 2)
        topk = sel_idx.shape[1]
    nbytes = 0
    if workspace is not None:
        _need(workspace, torch.float32, "workspace", 1)
        nbytes = workspace.numel() * 4
    _check(lib().dsv4_sparse_attn_narrow(_ptr(q), q.shape[0], q_pos0, q.shape[1], q.shape[2],
                                         scale, _ptr(raw_kv), raw_pos0, raw_kv.shape[0], window,
                                         None if attn_cache is None else attn_cache.ref(),
                                         _ptr(sel_idx), topk, n_splits, _ptr(workspace), nbytes,
                                         _ptr(out), _stream(stream)))
