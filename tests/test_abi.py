"""Host-only checks of the C-ABI library: it loads, exports every function
include/dsv4.h declares, and rejects bad arguments on the host before
anything touches HIP (every call below fails validation or needs no device;
none enqueues work)."""
import ctypes

import pytest

import sparse_indexed_attention_amd as dsv4
from sparse_indexed_attention_amd import dsv4_pool_cache

OK, INVALID, UNSUPPORTED, CAPACITY, MISMATCH, SCRATCH = 0, -1, -2, -3, -4, -5
FAKE = 0x1000  # never dereferenced: every call using it fails validation first


def test_library_exports_every_header_function():
    L = dsv4.lib()
    names = dsv4.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dsv4._SIGNATURES)


def test_use_library_switches_and_restores():
    # a second handle on the same build, then back to the first by handle
    first = dsv4.lib()
    second = dsv4.use_library(dsv4.LIB_PATH)
    try:
        assert second is not first
        assert dsv4.lib() is second
        assert second.dsv4_abi_version() == first.dsv4_abi_version()
        assert dsv4.dsv4_score_stride(1000) == first.dsv4_score_stride(1000)
    finally:
        assert dsv4.use_library(first) is first
    assert dsv4.lib() is first
    with pytest.raises(ImportError):
        dsv4.use_library("/nonexistent/libdsv4.so")
    assert dsv4.lib() is first


def test_abi_version_and_host_helpers():
    assert dsv4.dsv4_abi_version() == 6
    assert dsv4.dsv4_indexer_all_pooled(0, 8) is False
    assert dsv4.dsv4_indexer_all_pooled(1, 8) is True
    assert dsv4.dsv4_indexer_all_pooled(8, 8) is True
    assert dsv4.dsv4_indexer_all_pooled(9, 8) is False
    assert dsv4.dsv4_score_stride(1) == 64 and dsv4.dsv4_score_stride(64) == 64
    assert dsv4.dsv4_score_stride(65) == 128
    # one 1,024-row tile against 262,144 pooled rows: 1 GiB of fp32 scores
    assert dsv4.dsv4_indexer_scratch_bytes(1024, 262144) == 1 << 30
    # past the extent bound: -1, and sizes past it are refused
    ext = dsv4.DSV4_MAX_EXTENT
    assert dsv4.dsv4_score_stride(ext) == ext and dsv4.dsv4_score_stride(ext + 1) == -1
    with pytest.raises(dsv4.DSV4Error):
        dsv4.dsv4_indexer_scratch_bytes(1, ext + 1)
    with pytest.raises(dsv4.DSV4Error):  # 2^40 x 2^40 x 4 bytes do not fit a size_t
        dsv4.dsv4_indexer_scratch_bytes(ext, ext)


def test_binding_constants_match_header():
    """The binding's copies of the header's constants, read from the header."""
    import re
    text = open(dsv4.HEADER_PATH).read()

    def define(name):
        m = re.search(r"#define\s+%s\s+(.+)" % name, text)
        expr = re.sub(r"\(int64_t\)|(?<=\d)u\b", "", m.group(1).split("/*")[0])
        return eval(expr, {"__builtins__": {}})

    assert dsv4.DSV4_NOALLOC_SCRATCH_BYTES == define("DSV4_NOALLOC_SCRATCH_BYTES")
    assert dsv4.DSV4_MAX_EXTENT == define("DSV4_MAX_EXTENT")
    assert dsv4.dsv4_abi_version() == define("DSV4_ABI_VERSION")
    assert (dsv4.DSV4_BF16, dsv4.DSV4_F32) == (define("DSV4_BF16"), define("DSV4_F32"))


def _cache(n_rows=0, n_rem=0, cap=16, dim=128, dtype=1, ratio=4, rows=FAKE, rem=FAKE):
    return dsv4_pool_cache(rows, rem, cap, n_rows, n_rem, ratio, dim, dtype)


def _rc(name, *args):
    return getattr(dsv4.lib(), name)(*args)


def test_compress_validation_leaves_state():
    c = _cache(n_rows=15, n_rem=3)
    before = (c.n_rows, c.n_rem)
    # 3 waiting + 5 new = 2 rows -> 17 > 16
    assert _rc("dsv4_compress", ctypes.byref(c), ctypes.c_void_p(FAKE), 5, None) == CAPACITY
    assert (c.n_rows, c.n_rem) == before
    assert "capacity" in dsv4.dsv4_last_error()
    assert _rc("dsv4_compress", ctypes.byref(c), None, 1, None) == INVALID
    assert _rc("dsv4_compress", ctypes.byref(c), ctypes.c_void_p(FAKE), -1, None) == INVALID
    for r in (0, 1, 257):
        bad = _cache(ratio=r)
        assert _rc("dsv4_compress", ctypes.byref(bad), ctypes.c_void_p(FAKE), 4, None) == UNSUPPORTED
    # ratio 128: 100 waiting + 200 new = 2 rows -> 17 > 16; the remainder
    # bound follows the ratio (127 may wait, 128 may not)
    big = _cache(n_rows=15, n_rem=100, ratio=128)
    assert _rc("dsv4_compress", ctypes.byref(big), ctypes.c_void_p(FAKE), 200, None) == CAPACITY
    assert (big.n_rows, big.n_rem) == (15, 100)
    assert _rc("dsv4_compress", ctypes.byref(_cache(n_rem=128, ratio=128)),
               ctypes.c_void_p(FAKE), 4, None) == INVALID
    bad = _cache(n_rem=4)
    assert _rc("dsv4_compress", ctypes.byref(bad), ctypes.c_void_p(FAKE), 4, None) == INVALID
    assert _rc("dsv4_compress", None, ctypes.c_void_p(FAKE), 4, None) == INVALID
    # nothing to do: no enqueue, OK
    assert _rc("dsv4_compress", ctypes.byref(c), None, 0, None) == OK
    assert (c.n_rows, c.n_rem) == before


def test_select_guard_and_gates():
    c = _cache(n_rows=10, n_rem=0, cap=64)
    out = ctypes.c_void_p(FAKE)
    ap = ctypes.c_int32(7)
    args = lambda **kw: dict(dict(n_attn=10, q=FAKE, w=FAKE, T=8, q_pos0=32, heads=64, topk=4,
                                  tile=0, scratch=FAKE, sbytes=1 << 20), **kw)

    def call(**kw):
        a = args(**kw)
        return _rc("dsv4_indexer_select", ctypes.byref(c), a["n_attn"], ctypes.c_void_p(a["q"]),
                   ctypes.c_void_p(a["w"]), a["T"], a["q_pos0"], a["heads"], a["topk"], a["tile"],
                   ctypes.c_void_p(a["scratch"]), a["sbytes"], out, ctypes.byref(ap), None)
    assert call(n_attn=11) == MISMATCH            # row-count guard
    assert "pooled rows" in dsv4.dsv4_last_error()
    assert call(topk=0) == UNSUPPORTED
    assert call(topk=5000) == UNSUPPORTED
    assert call(q_pos0=40) == INVALID             # 40 + 8 > 4*10: ahead of the frontier
    assert call(heads=65) == UNSUPPORTED
    assert call(sbytes=10) == SCRATCH
    assert call(q=0) == INVALID
    assert ap.value == 7                          # untouched on every failure


def test_scores_and_topk_gates():
    c = _cache(n_rows=10, dim=96)
    assert _rc("dsv4_indexer_scores", ctypes.byref(c), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
               4, 0, 64, 1, ctypes.c_void_p(FAKE), 64, None) == UNSUPPORTED
    c = _cache(n_rows=10, dim=128, dtype=2)
    assert _rc("dsv4_indexer_scores", ctypes.byref(c), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
               4, 0, 64, 1, ctypes.c_void_p(FAKE), 64, None) == UNSUPPORTED
    c = _cache(n_rows=10, dim=128)
    assert _rc("dsv4_indexer_scores", ctypes.byref(c), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
               4, 0, 64, 1, ctypes.c_void_p(FAKE), 8, None) == INVALID  # stride < rows
    c = _cache(n_rows=10, dim=128, ratio=128)  # the indexer's mask is the ratio-4 rule
    assert _rc("dsv4_indexer_scores", ctypes.byref(c), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
               4, 0, 64, 1, ctypes.c_void_p(FAKE), 64, None) == UNSUPPORTED
    # top-k: visible prefix of the last row (position 99 -> 25 rows) exceeds 20 columns
    assert _rc("dsv4_topk_select", ctypes.c_void_p(FAKE), 4, 64, 96, 20, 8,
               ctypes.c_void_p(FAKE), None) == INVALID
    assert _rc("dsv4_topk_select", ctypes.c_void_p(FAKE), 4, 64, 0, 20, 0,
               ctypes.c_void_p(FAKE), None) == UNSUPPORTED


def test_attention_gates():
    c = _cache(n_rows=40, dim=512, cap=64)

    def call(T=4, q_pos0=100, heads=64, dim=512, raw_pos0=0, n_raw=104, window=128, cache=c,
             sel=FAKE, topk=16, out=FAKE):
        return _rc("dsv4_sparse_prefill_attn", ctypes.c_void_p(FAKE), T, q_pos0, heads, dim, 0.0,
                   ctypes.c_void_p(FAKE), raw_pos0, n_raw, window, ctypes.byref(cache),
                   ctypes.c_void_p(sel), topk, ctypes.c_void_p(out), None)
    assert call(dim=96) == UNSUPPORTED
    # the output is written in 16-byte vectors: an offset view is refused
    assert call(out=FAKE + 8) == INVALID
    assert "aligned" in dsv4.dsv4_last_error()
    assert call(dim=256) == INVALID           # cache dim differs
    assert call(heads=65) == UNSUPPORTED
    assert call(window=0) == INVALID
    assert call(raw_pos0=1, n_raw=103) == INVALID   # window of position 100 starts at 0
    assert call(n_raw=103) == INVALID          # does not reach position 103
    assert call(q_pos0=200, raw_pos0=73, n_raw=131) == INVALID  # sees 51 pooled rows > 40
    assert call(topk=0) == UNSUPPORTED
    f32 = _cache(n_rows=40, dim=512, cap=64, dtype=2)
    assert call(cache=f32) == UNSUPPORTED
    # ratio-128 pool: position 5119 sees 40 rows (fits), 5120+ sees 40 too,
    # 5247 sees 41 > 40
    r128 = _cache(n_rows=40, dim=512, cap=64, ratio=128)
    assert call(cache=r128, q_pos0=5244, raw_pos0=5117, n_raw=131) == INVALID
    assert "41 pooled rows" in dsv4.dsv4_last_error()
    # window-only mode: no pool, so no selection either
    assert _rc("dsv4_sparse_prefill_attn", ctypes.c_void_p(FAKE), 4, 100, 64, 512, 0.0,
               ctypes.c_void_p(FAKE), 0, 104, 128, None, ctypes.c_void_p(FAKE), 16,
               ctypes.c_void_p(FAKE), None) == INVALID
    assert "without a pool" in dsv4.dsv4_last_error()
    assert _rc("dsv4_sparse_prefill_attn", ctypes.c_void_p(FAKE), 4, 100, 64, 96, 0.0,
               ctypes.c_void_p(FAKE), 0, 104, 128, None, None, 0,
               ctypes.c_void_p(FAKE), None) == UNSUPPORTED


def test_narrow_attention_plan_and_gates():
    ns, nb = dsv4.dsv4_sparse_attn_narrow_plan(1, 64, 512, 128, 2048)
    assert ns == 34 and nb == 1 * 34 * 64 * (512 + 2) * 4     # 68 tiles, 2 per split
    assert dsv4.dsv4_sparse_attn_narrow_plan(4, 64, 512, 128, 2048)[0] == 34
    assert dsv4.dsv4_sparse_attn_narrow_plan(64, 64, 512, 128, 2048)[0] == 4   # 256 / 64
    assert dsv4.dsv4_sparse_attn_narrow_plan(1, 64, 512, 128, 0) == (2, 2 * 64 * 514 * 4)
    assert dsv4.dsv4_sparse_attn_narrow_plan(300, 64, 512, 128, 2048) == (1, 0)
    assert dsv4.dsv4_sparse_attn_narrow_plan(1, 64, 512, 128, 10 ** 6)[0] == 64  # cap
    with pytest.raises(dsv4.DSV4Error):
        dsv4.dsv4_sparse_attn_narrow_plan(1, 0, 512, 128, 0)
    c = _cache(n_rows=40, dim=512, cap=64)

    def call(n_splits=4, ws=FAKE, nbytes=1 << 30, sel=FAKE, T=4):
        return _rc("dsv4_sparse_attn_narrow", ctypes.c_void_p(FAKE), T, 100, 64, 512, 0.0,
                   ctypes.c_void_p(FAKE), 0, 104, 128, ctypes.byref(c), ctypes.c_void_p(sel), 16,
                   n_splits, ctypes.c_void_p(ws) if ws else None, nbytes,
                   ctypes.c_void_p(FAKE), None)
    assert call(n_splits=0) == UNSUPPORTED
    assert call(n_splits=65) == UNSUPPORTED
    assert call(ws=0) == INVALID
    assert call(ws=FAKE + 4) == INVALID                       # not 16-byte aligned
    assert _rc("dsv4_sparse_attn_narrow", ctypes.c_void_p(FAKE), 4, 100, 64, 512, 0.0,
               ctypes.c_void_p(FAKE), 0, 104, 128, ctypes.byref(c), ctypes.c_void_p(FAKE), 16,
               4, ctypes.c_void_p(FAKE), 1 << 30, ctypes.c_void_p(FAKE + 2), None) == INVALID
    assert call(nbytes=4 * 4 * 64 * 514 * 4 - 1) == SCRATCH   # one byte short
    assert "workspace" in dsv4.dsv4_last_error()
    assert call(T=0, n_splits=4, ws=0) == OK                  # nothing to do


def test_split_topk_sizing_and_gates():
    ws = dsv4.dsv4_topk_split_workspace_bytes
    # 1 row at position 2^20 - 4: 262,143 visible -> 8 chunks of 32,768
    assert ws(1, (1 << 20) - 4, 2048) == 2 * 8 * 2048 * 4
    assert ws(3, (1 << 20) - 4, 7) == 2 * ((3 * 8 * 7 * 4 + 15) // 16 * 16)
    assert ws(65, (1 << 20) - 4, 7) == 0              # too many rows for odd k: per-row kernel
    # whole tiles (last row sees 262,144 columns: 8 chunks) when k % 4 == 0 and
    # a row has at most 32,768 candidates
    assert ws(1024, (1 << 20) - 1024, 2048) == 2 * 1024 * 8 * 2048 * 4
    assert ws(65, (1 << 20) - 65, 4096) == 2 * 65 * 8 * 4096 * 4
    assert ws(65, (1 << 20) - 60, 4096) == 0          # 9 chunks x 4,096 candidates: too many
    assert ws(1, 4 * 32767, 2048) == 0                # one chunk
    # narrow tiles over long rows get room for the split top-k (sized for k = 4096)
    assert dsv4.dsv4_indexer_scratch_bytes(1, 262144) == 262144 * 4 + 2 * 8 * 4096 * 4
    assert dsv4.dsv4_indexer_scratch_bytes(64, 32768) == 64 * 32768 * 4
    assert dsv4.dsv4_indexer_scratch_bytes(65, 262144) == 65 * 262144 * 4

    def call(ws_ptr, nbytes, rows=2, q_pos0=(1 << 20) - 8):
        return _rc("dsv4_topk_select_split", ctypes.c_void_p(FAKE), rows, 262144, q_pos0, 262144,
                   2048, ctypes.c_void_p(FAKE), ctypes.c_void_p(ws_ptr) if ws_ptr else None,
                   nbytes, None)
    assert call(0, 0) == INVALID
    assert call(FAKE + 8, 1 << 20) == INVALID                 # misaligned
    assert call(FAKE, 2 * 2 * 8 * 2048 * 4 - 16) == SCRATCH
    assert "workspace" in dsv4.dsv4_last_error()
    assert call(FAKE, 1 << 20, q_pos0=(1 << 20) + 4) == INVALID   # sees past 262,144 columns
