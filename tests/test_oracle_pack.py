"""Pins for the oracle's fragment-ordered weight layout (a permutation of the
codes, no arithmetic), each against something other than the function:

- numpy's reshape / transpose route: (groups, 16 rows, steps, 4 quarters,
  2 halves, 16 bytes) -> (groups, steps, halves, quarters, rows, bytes);
- a permutation: every code appears exactly once, the padding rows past N
  are zero codes, and the inverse map recovers the row-major codes;
- single-element probes: a one-hot matrix lands at the position the layout
  formula gives.
"""
import numpy as np
import pytest


def numpy_route(q):
    N, K = q.shape
    G = -(-N // 16)
    qq = np.zeros((G * 16, K), np.uint8)
    qq[:N] = q
    t = qq.reshape(G, 16, K // 128, 4, 2, 16)        # g, row, step, quarter, half, byte
    return t.transpose(0, 2, 4, 3, 1, 5).reshape(-1)  # g, step, half, lane = quarter*16 + row, byte


@pytest.mark.parametrize("shape", [(16, 128), (48, 384), (37, 256), (5, 128)])
def test_matches_numpy_route(orc, shape):
    q = np.random.default_rng(shape[0]).integers(0, 256, shape).astype(np.uint8)
    assert np.array_equal(orc.pack_weights16(q), numpy_route(q))


def test_is_a_permutation_with_zero_padding(orc):
    N, K = 37, 256
    ids = np.arange(N * K, dtype=np.int64)
    q = (ids % 251 + 1).astype(np.uint8)  # nonzero codes
    p = orc.pack_weights16(q.reshape(N, K))
    assert p.size == 48 * K
    assert np.count_nonzero(p) == N * K   # the 11 padding rows are zeros
    assert np.array_equal(np.sort(p[p != 0]), np.sort(q))


def test_one_hot_positions(orc):
    N, K = 32, 256
    for (n, k) in [(0, 0), (5, 17), (16, 200), (31, 255), (9, 128 + 32 * 3 + 16 + 7)]:
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 0x5A
        p = orc.pack_weights16(q)
        G, r = divmod(n, 16)
        s, kk = divmod(k, 128)
        quarter, rem = divmod(kk, 32)
        h, b = divmod(rem, 16)
        lane = quarter * 16 + r
        pos = (G * (K // 128) + s) * 2048 + h * 1024 + lane * 16 + b
        assert np.flatnonzero(p).tolist() == [pos]
