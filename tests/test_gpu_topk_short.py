"""Top-k of rows held in registers (at most 32,768 visible columns: one wave
per row up to 4,096 columns, else 2, 4 or 8 waves of 4,096 columns each; few
rows of 2,049 - 16,384 columns take 2, 4 or 8 waves of 2,048):
parity with the oracle's selection and with the LDS-staged workgroup
kernel, which the same entry point takes when the row stride is not a
multiple of 4 floats or rows are longer.

Sizes put the longest row exactly at, and one past, each register layout's
limit (1,024 / 2,048 / 4,096 columns in one wave, 8,192 / 16,384 / 32,768 in
2 / 4 / 8 waves; 32,769 goes to the LDS-staged kernel).
Row contents cover the selection's hard cases: several digit passes (few
distinct values), a single value, signed zeros, keys spanning the sign bit
and infinities, and k at or above the visible count.
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_indexed_attention_amd as dsv4
from oracle import dsv4_oracle as O

pytestmark = pytest.mark.gpu


def _rows(kind, rows, n_cols, rng):
    shape = (rows, n_cols)
    if kind == "relu_sum":      # indexer-like: non-negative, tightly packed exponents
        s = np.zeros(shape, np.float32)
        for _ in range(8):
            s += np.maximum(rng.standard_normal(shape, dtype=np.float32), 0)
    elif kind == "uniform":
        s = rng.random(shape)
    elif kind == "normal":
        s = rng.standard_normal(shape)
    elif kind == "levels3":
        s = rng.integers(0, 3, size=shape)
    elif kind == "levels40":
        s = rng.integers(0, 40, size=shape) * 0.25
    elif kind == "constant":
        s = np.full(shape, 0.75)
    elif kind == "signed_zero":
        s = np.where(rng.random(shape) < 0.5, -0.0, 0.0)
        s[:, ::37] = 2.0
    elif kind == "wide":        # mixed signs, huge range, infinities
        s = rng.standard_normal(shape, dtype=np.float32) * np.exp2(
            rng.integers(-90, 90, size=shape).astype(np.float32))
        s[:, ::53] = np.inf
        s[:, 7::61] = -np.inf
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


def _select(scores, q_pos0, n_cols, topk, stride):
    rows = scores.shape[0]
    buf = np.full((rows, stride), np.float32(3e38), np.float32)  # garbage past the prefix
    buf[:, :n_cols] = scores
    for t in range(rows):
        buf[t, O.visible_rows(q_pos0 + t):n_cols] = np.float32(3e38)
    d = torch.from_numpy(buf).cuda()
    out = torch.full((rows, topk), 77, dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select(d, q_pos0, n_cols, topk, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), buf


@pytest.mark.parametrize("max_vis", [1024, 1025, 2048, 2049, 4096, 4097, 8192, 8193, 16384,
                                     16385, 32768, 32769])
@pytest.mark.parametrize("kind", ["relu_sum", "uniform", "normal", "levels3", "levels40",
                                  "constant", "signed_zero", "wide"])
def test_short_rows_match_oracle(max_vis, kind):
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{max_vis}".encode()))
    rows = 70  # one wave per row (18 workgroups, the last partial) up to 2,048 columns
    q_pos0 = 4 * max_vis - rows               # the last row sees exactly max_vis columns
    n_cols = max_vis
    topk = 512 if max_vis <= 2049 else 2048
    s = _rows(kind, rows, n_cols, rng)
    got, buf = _select(s, q_pos0, n_cols, topk, stride=n_cols + (-n_cols) % 4)
    want = O.topk_select(buf.astype(np.float64), q_pos0, topk)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("max_vis,rows", [(2049, 1100), (3000, 1100), (4096, 1100),
                                          (4097, 1100), (8192, 1100), (8193, 600), (16384, 600)])
@pytest.mark.parametrize("kind", ["relu_sum", "levels3", "constant", "wide"])
def test_many_rows_keep_4096_columns_per_wave(max_vis, rows, kind):
    """Past 1,024 rows (512 beyond 8,192 columns) rows keep one wave per 4,096
    columns; fewer rows take waves of 2,048, covered above with 70 rows."""
    rng = np.random.default_rng(zlib.crc32(f"many/{kind}/{max_vis}".encode()))
    q_pos0 = 4 * max_vis - rows
    n_cols = max_vis
    s = _rows(kind, rows, n_cols, rng)
    got, buf = _select(s, q_pos0, n_cols, 2048, stride=n_cols + (-n_cols) % 4)
    np.testing.assert_array_equal(got, O.topk_select(buf.astype(np.float64), q_pos0, 2048))


@pytest.mark.parametrize("topk", [1, 2, 63, 64, 65, 1000, 1023, 1024, 4096])
def test_short_rows_k_around_visible(topk):
    """k below, at and above the visible count of every row (rows see 768..1,023
    columns here; k >= visible chooses every visible column)."""
    rng = np.random.default_rng(topk)
    rows, q_pos0 = 1024, 3072 - 1
    n_cols = (q_pos0 + rows) // 4
    s = _rows("relu_sum", rows, n_cols, rng)
    got, buf = _select(s, q_pos0, n_cols, topk, stride=n_cols + (-n_cols) % 4)
    np.testing.assert_array_equal(got, O.topk_select(buf.astype(np.float64), q_pos0, topk))


def test_short_rows_from_the_first_token():
    """Rows 0-2 see no pooled row (all -1); row 3 sees one."""
    rng = np.random.default_rng(5)
    rows, q_pos0, topk = 200, 0, 16
    n_cols = 52
    s = _rows("normal", rows, n_cols, rng)
    got, buf = _select(s, q_pos0, n_cols, topk, stride=52)
    assert (got[:3] == -1).all() and got[3, 0] == 0 and (got[3, 1:] == -1).all()
    np.testing.assert_array_equal(got, O.topk_select(buf.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("kind", ["relu_sum", "levels3", "wide"])
def test_short_rows_match_workgroup_kernel(kind):
    """A whole 2,048-row tile at a 16K-token context (4,096 pooled rows, k =
    2,048): the wave-per-row kernel (row stride 4,096) against the
    workgroup-per-row kernel (row stride 4,097, not a multiple of 4)."""
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    rows, q_pos0, topk = 2048, 16384 - 2048, 2048
    n_cols = (q_pos0 + rows) // 4
    s = _rows(kind, rows, n_cols, rng)
    a, _ = _select(s, q_pos0, n_cols, topk, stride=n_cols)
    b, _ = _select(s, q_pos0, n_cols, topk, stride=n_cols + 1)
    np.testing.assert_array_equal(a, b)
    pick = rng.choice(rows, 64, replace=False)
    for t in pick:
        vis = O.visible_rows(q_pos0 + int(t))
        np.testing.assert_array_equal(a[t], O.topk_row(s[t].astype(np.float64), vis, topk))


@pytest.mark.parametrize("kind", ["relu_sum", "levels40", "wide"])
def test_long_rows_match_workgroup_kernel(kind):
    """A whole 2,048-row tile at a 128K-token context (32,768 pooled rows, k =
    2,048): the 8-wave register kernel (row stride 32,768) against the
    LDS-staged kernel (row stride 32,769), and sampled rows against the oracle."""
    rng = np.random.default_rng(zlib.crc32(("long/" + kind).encode()))
    rows, q_pos0, topk = 2048, 131072 - 2048, 2048
    n_cols = (q_pos0 + rows) // 4
    s = _rows(kind, rows, n_cols, rng)
    a, _ = _select(s, q_pos0, n_cols, topk, stride=n_cols)
    b, _ = _select(s, q_pos0, n_cols, topk, stride=n_cols + 1)
    np.testing.assert_array_equal(a, b)
    for t in rng.choice(rows, 24, replace=False):
        vis = O.visible_rows(q_pos0 + int(t))
        np.testing.assert_array_equal(a[t], O.topk_row(s[t].astype(np.float64), vis, topk))


@pytest.mark.parametrize("max_vis,topk", [(32768, 4096), (16384, 4096), (4096, 4095),
                                          (2048, 1023), (32768, 3), (1024, 1)])
def test_register_rows_large_and_odd_k(max_vis, topk):
    """The largest k (its output slots fill most of a multi-wave row's LDS
    area), odd k (the scalar copy-out), and tiny k."""
    rng = np.random.default_rng(max_vis + topk)
    rows = 40
    q_pos0 = 4 * max_vis - rows
    s = _rows("relu_sum", rows, max_vis, rng)
    got, buf = _select(s, q_pos0, max_vis, topk, stride=max_vis)
    np.testing.assert_array_equal(got, O.topk_select(buf.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("max_vis", [1024, 4096, 32768])
def test_register_rows_unaligned_output(max_vis):
    """An output row block that starts 4 bytes past a 16-byte boundary takes
    the element-wise copy-out."""
    rng = np.random.default_rng(max_vis)
    rows, topk = 36, 512
    q_pos0 = 4 * max_vis - rows
    s = _rows("normal", rows, max_vis, rng)
    d = torch.from_numpy(s).cuda()
    flat = torch.full((rows * topk + 1,), 77, dtype=torch.int32, device="cuda")
    out = flat[1:].view(rows, topk)
    assert out.data_ptr() % 16 == 4
    dsv4.dsv4_topk_select(d, q_pos0, max_vis, topk, out)
    torch.cuda.synchronize()
    assert int(flat[0]) == 77                 # nothing written before the block
    np.testing.assert_array_equal(out.cpu().numpy(),
                                  O.topk_select(s.astype(np.float64), q_pos0, topk))


@pytest.mark.parametrize("case", range(24))
def test_random_shapes_match_oracle(case):
    """Seeded random shapes across every top-k path: row counts, positions
    (visible prefixes from a few columns up to three 32,768-column chunks),
    k (odd or a multiple of 4, below or above the visible count), aligned or
    unaligned strides, and tie-prone or continuous values; both the per-row
    entry point and the two-pass one (with its workspace) against the oracle."""
    rng = np.random.default_rng(1000 + case)
    rows = int(rng.integers(1, 40))
    max_vis = int(rng.choice([int(rng.integers(4, 600)), int(rng.integers(600, 4200)),
                              int(rng.integers(4200, 33000)), int(rng.integers(33000, 72000))]))
    q_pos0 = max(0, 4 * max_vis - rows)
    n_cols = (q_pos0 + rows) // 4
    topk = int(rng.choice([int(rng.integers(1, 9)), 4 * int(rng.integers(1, 400)),
                           int(rng.integers(1, 4097))]))
    stride = n_cols + int(rng.choice([0, (-n_cols) % 4, 1, 7]))
    kind = rng.choice(["relu_sum", "levels40", "normal"])
    s = _rows(str(kind), rows, max(n_cols, 1), rng)[:, :n_cols]
    got, buf = _select(s, q_pos0, n_cols, topk, stride=max(stride, 1))
    want = O.topk_select(buf.astype(np.float64), q_pos0, topk)
    np.testing.assert_array_equal(got, want)
    # the two-pass entry point on the same buffer
    d = torch.from_numpy(buf).cuda()
    nb = dsv4.dsv4_topk_split_workspace_bytes(rows, q_pos0, topk)
    ws = torch.empty(max(nb // 4, 4), dtype=torch.float32, device="cuda")
    out = torch.full((rows, topk), 55, dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select_split(d, q_pos0, n_cols, topk, out, ws if nb else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("case", range(12))
def test_random_long_rows_two_pass_match_oracle(case):
    """Seeded random long rows (2 or 3 chunks of 32,768 columns) with aligned
    strides and k % 4 == 0, so that the two register passes run: the per-row
    entry point (LDS-staged kernel) and the two-pass one with its workspace,
    at row counts on both sides of 64, against the oracle."""
    rng = np.random.default_rng(2000 + case)
    rows = int(rng.integers(1, 90))
    max_vis = int(rng.integers(33000, 72000))
    q_pos0 = 4 * max_vis - rows
    n_cols = (q_pos0 + rows) // 4
    topk = 4 * int(rng.integers(1, 1025))
    stride = n_cols + (-n_cols) % 4 + 4 * int(rng.integers(0, 3))
    kind = str(rng.choice(["relu_sum", "levels40", "normal"]))
    s = _rows(kind, rows, n_cols, rng)
    got, buf = _select(s, q_pos0, n_cols, topk, stride=stride)
    want = O.topk_select(buf.astype(np.float64), q_pos0, topk)
    np.testing.assert_array_equal(got, want)
    d = torch.from_numpy(buf).cuda()
    nb = dsv4.dsv4_topk_split_workspace_bytes(rows, q_pos0, topk)
    assert nb > 0
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    out = torch.full((rows, topk), 55, dtype=torch.int32, device="cuda")
    dsv4.dsv4_topk_select_split(d, q_pos0, n_cols, topk, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want)
