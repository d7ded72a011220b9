"""Pins of the oracle's cast-transpose (quantize once, codes written both
row-major and K-major), each against something other than the function
itself:

- the transposed codes equal numpy's transpose of the row-major codes, on
  non-square shapes (an index swap or a wrong leading dimension fails);
- transposition invariance: cast-transposing X with groups (gr, gc) gives the
  codes, scales, amax and counters of quantizing X^T with groups (gc, gr),
  since a group's maximum and each element's product do not depend on the
  orientation;
- per-column groups on a tiny matrix, brute-forced: numpy column maxima, the
  pinned scale rule and the nearest-code search over all 256 codes."""
import numpy as np
import pytest

from workloads import to_bf16_bits

GRANS = [(0, 0), (1, 0), (0, 1), (16, 32)]


def make_x(seed, rows, cols, dtype):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(g.uniform(-4, 4, (1, cols))).astype(np.float32)  # per-column spread
    x[:, g.integers(0, cols)] = 0.0                                 # an all-zero column
    x[g.integers(0, rows), g.integers(0, cols)] = 1e30              # a saturating outlier
    return to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", GRANS)
def test_transposed_codes_are_the_transpose(orc, dtype, fmt, gran):
    x = make_x(1, 48, 80, dtype)
    q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, gran)
    assert qt.shape == (80, 48)
    assert np.array_equal(qt, np.ascontiguousarray(q.T))
    q2, s2, r2, am2, cnt2 = orc.quantize(x, fmt, gran)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(cnt, cnt2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("mode", ["dynamic", "given"])
def test_transposition_invariance(orc, dtype, fmt, gran, mode):
    x = make_x(2, 64, 96, dtype)
    xt = np.ascontiguousarray(x.T)
    gt = (gran[1], gran[0])
    if mode == "dynamic":
        q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, gran)
        q_t, s_t, r_t, am_t, cnt_t = orc.quantize(xt, fmt, gt)
    else:
        G = (orc.ngroups(64, gran[0]), orc.ngroups(96, gran[1]))
        sg = np.exp(np.random.default_rng(3).uniform(-6, 2, G)).astype(np.float32)
        q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, gran, mode=orc.GIVEN, scale=sg)
        q_t, s_t, r_t, am_t, cnt_t = orc.quantize(xt, fmt, gt, mode=orc.GIVEN,
                                                  scale=np.ascontiguousarray(sg.T))
    assert np.array_equal(qt, q_t)
    assert np.array_equal(s.T, s_t) and np.array_equal(r.T, r_t)
    assert np.array_equal(am.T.view(np.uint32), am_t.view(np.uint32))
    assert np.array_equal(cnt, cnt_t)


@pytest.mark.parametrize("fmt", [0, 1])
def test_per_column_groups_brute_force(orc, fmt):
    g = np.random.default_rng(4)
    x = (g.standard_normal((8, 6)) * np.exp(g.uniform(-3, 3, (1, 6)))).astype(np.float32)
    q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, (0, 1))
    F = orc.fmax(fmt)
    for j in range(6):
        a = np.float32(np.abs(x[:, j]).max())
        assert am[0, j] == a
        assert s[0, j] == np.float32(np.float64(a) / F)
        assert r[0, j] == np.float32(F / np.float64(a))
        for i in range(8):
            v = np.float32(np.float64(x[i, j]) * np.float64(r[0, j]))
            code = orc.encode_bruteforce(float(np.clip(v, -F, F)), fmt)
            assert q[i, j] == code and qt[j, i] == code
