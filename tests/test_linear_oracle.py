"""Pins of the oracle's integer-only linear layer (CPU).

The integer product is pinned to numpy's int64 matrix product (a library
special case) and the requantisation to exact integer floor division, on
shapes with ragged sizes and extreme dyadic pairs; the head-split layout is a
pure permutation checked here too.
"""
import numpy as np
import pytest

import oracle
from integer_only_quantized_int8_amd import workloads as W


def _expected(x, w, b, c):
    acc = x.astype(np.int64) @ w.astype(np.int64).T
    # exact floor((b * acc) / 2^c) in Python integers, then the symmetric clip
    y = np.array([[(int(b) * int(a)) // (1 << c) for a in row] for row in acc], dtype=np.int64)
    return np.clip(y, -127, 127).astype(np.int8)


@pytest.mark.parametrize("rows,fin,fout,b,c", [
    (1, 1, 1, 1, 0), (3, 5, 7, 20000, 16), (17, 64, 9, (1 << 15) - 1, 22),
    (5, 33, 4, (1 << 31) - 1, 40), (8, 128, 64, 1 << 14, 24), (2, 7, 3, 12345, 62),
])
def test_linear_matches_matmul_and_floor(rows, fin, fout, b, c):
    rng = np.random.default_rng(rows * 131 + fin)
    x = rng.integers(-127, 128, (rows, fin)).astype(np.int8)
    w = rng.integers(-127, 128, (fout, fin)).astype(np.int8)
    assert np.array_equal(oracle.linear(x, w, b, c), _expected(x, w, b, c))


def test_linear_row_range_and_extremes():
    x = np.full((4, 64), -127, np.int8)
    w = np.full((2, 64), 127, np.int8)
    full = oracle.linear(x, w, 1, 0)
    assert np.all(full == -127)                      # saturates low
    assert np.all(oracle.linear(-x, w, 1, 0) == 127)  # and high
    # exact zero and the floor of a negative quotient
    x2 = np.zeros((1, 64), np.int8); x2[0, 0] = -1
    w2 = np.ones((1, 64), np.int8)
    assert oracle.linear(x2, w2, 1, 1)[0, 0] == -1    # floor(-1/2) = -1
    assert oracle.linear(x2, w2, 1, 0)[0, 0] == -1
    assert np.array_equal(oracle.linear(x, w, 3, 2, rows=(1, 3)), full[1:3] * 0 - 127)


def test_linear_workload_generator_and_head_split_permutation():
    lw = W.make_linear(2 * 3, 64, 3 * 2 * 64, seed=5, qkv_heads=(2, 3, 2, 64))
    assert lw.x.shape == (6, 64) and lw.w.shape == (384, 64)
    assert lw.params["layout"] == 1 and len(lw.params["b"]) == 3
    for bi, ci in zip(lw.params["b"], lw.params["c"]):
        assert (1 << 14) <= bi < (1 << 15) and 0 < ci < 63
    # the head split of a [rows, 3 C] result is a permutation of its entries
    y = np.arange(6 * 384).reshape(6, 384)
    q = y.reshape(2, 3, 3, 2, 64).transpose(2, 0, 3, 1, 4)   # [which, b, h, t, i]
    assert sorted(q.reshape(-1).tolist()) == list(range(6 * 384))
    assert q[1, 1, 0, 2, 5] == y[1 * 3 + 2, 1 * 128 + 0 * 64 + 5]
