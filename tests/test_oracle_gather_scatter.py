"""Pins of the C oracle's row gather and gradient scatter-add — no GPU.

Gather is pinned to torch.index_select on the CPU (textbook routine), bit for
bit.  Scatter-add is pinned to its one-hot definition (index_add_ in fp64 on
the CPU), to the row histogram when every gradient is 1, and to exact sums
when gradients are small integers."""
import numpy as np
import pytest
import torch

from oracle import c_oracle


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_equals_index_select(dtype):
    rng = np.random.default_rng(0)
    num_rows, dim, row_begin = 1000, 160, 5000
    t = rng.normal(0, 0.02, size=(num_rows, dim)).astype(np.float32)
    table = t if dtype == "f32" else bf16_bits(t)
    rows = rng.integers(row_begin, row_begin + num_rows, size=(3, 7, 16)).astype(np.int64)
    out, bad = c_oracle.gather(table, rows, row_begin)
    assert bad == -1 and out.shape == (3, 7, 16, dim)
    ref = torch.index_select(torch.from_numpy(table.view(np.int32 if dtype == "f32" else np.int16)), 0,
                             torch.from_numpy(rows.reshape(-1) - row_begin)).numpy()
    assert np.array_equal(out.reshape(-1, dim).view(ref.dtype), ref)


def test_gather_out_of_range():
    table = np.arange(40, dtype=np.float32).reshape(10, 4) + 1
    rows = np.array([3, 4, 12, 2, 1, 13], dtype=np.int64)   # owned rows are [2, 12)
    out, bad = c_oracle.gather(table, rows, row_begin=2)
    assert bad == 2
    assert np.array_equal(out[2], np.zeros(4, np.float32)) and np.array_equal(out[4], np.zeros(4, np.float32))
    assert np.array_equal(out[0], table[1]) and np.array_equal(out[3], table[0])


def one_hot_sum(rows, dy64, num_rows, row_begin):
    ok = (rows >= row_begin) & (rows < row_begin + num_rows)
    g = torch.zeros(num_rows, dy64.shape[1], dtype=torch.float64)
    g.index_add_(0, torch.from_numpy(rows[ok] - row_begin), torch.from_numpy(dy64[ok]))
    return g.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_equals_one_hot(dtype):
    rng = np.random.default_rng(1)
    num_rows, dim, row_begin, n = 300, 160, 100, 5000
    rows = (row_begin + rng.zipf(1.3, size=n) % num_rows).astype(np.int64)
    rows[::97] = 7                                            # below the owned range
    dy32 = rng.standard_normal((n, dim)).astype(np.float32)
    dy = dy32 if dtype == "f32" else bf16_bits(dy32)
    dy64 = dy32.astype(np.float64) if dtype == "f32" else bits_to_f64(dy)
    ref = one_hot_sum(rows, dy64, num_rows, row_begin)
    gin = rng.standard_normal((num_rows, dim)).astype(np.float32)
    dense, bad = c_oracle.scatter_add_dense(rows, dy, num_rows, row_begin, gin)
    assert bad == 0
    np.testing.assert_allclose(dense, ref + gin.astype(np.float64), rtol=1e-12, atol=1e-12)
    ur, ug, bad = c_oracle.scatter_add_compact(rows, dy, num_rows, row_begin)
    assert bad == 0
    ok = rows[(rows >= row_begin) & (rows < row_begin + num_rows)]
    assert np.array_equal(ur, np.unique(ok))
    np.testing.assert_allclose(ug, ref[ur - row_begin], rtol=1e-12, atol=1e-12)


def test_scatter_ones_is_histogram():
    rng = np.random.default_rng(2)
    rows = rng.integers(0, 50, size=20000).astype(np.int64)
    dy = np.ones((rows.size, 8), dtype=np.float32)
    ur, ug, bad = c_oracle.scatter_add_compact(rows, dy, 50)
    counts = np.bincount(rows, minlength=50)
    assert bad == -1
    assert np.array_equal(ur, np.nonzero(counts)[0])
    assert np.array_equal(ug, np.repeat(counts[ur][:, None], 8, axis=1).astype(np.float64))


def test_scatter_integer_grads_exact():
    """Small-integer gradients have exact sums in fp64 and in fp32 (|sum| < 2**24)."""
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 64, size=30000).astype(np.int64)
    dy = rng.integers(-8, 9, size=(rows.size, 16)).astype(np.float32)
    dense, _ = c_oracle.scatter_add_dense(rows, bf16_bits(dy), 64)
    exact = np.zeros((64, 16), dtype=np.int64)
    np.add.at(exact, rows, dy.astype(np.int64))
    assert np.array_equal(dense, exact.astype(np.float64))


def test_scatter_empty_and_all_invalid():
    dy = np.ones((3, 4), dtype=np.float32)
    ur, ug, bad = c_oracle.scatter_add_compact(np.array([], dtype=np.int64), dy[:0], 10)
    assert ur.size == 0 and bad == -1
    ur, ug, bad = c_oracle.scatter_add_compact(np.array([10, 11, -1], dtype=np.int64), dy, 10)
    assert ur.size == 0 and bad == 0
