"""Parity of the HIP cast-transpose (fp8_quantize_transpose) with the CPU
oracle: bit-exact row-major codes, K-major codes, scales, inverse scales, amax
and counters, on shapes that span several 128 x 128 tiles with ragged edges,
strided operands and special values (NaN, Inf, zero rows, outliers)."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, same_f32
from workloads import case_seed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def make_input(seed, rows, cols, dtype, special=False):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(g.uniform(-5, 5, (rows, 1))).astype(np.float32)
    x *= np.exp(g.uniform(-3, 3, (1, cols))).astype(np.float32)
    x[g.integers(0, rows), :] = 0.0
    if special:
        x[g.integers(0, rows), g.integers(0, cols)] = np.inf
        x[g.integers(0, rows), g.integers(0, cols)] = -np.inf
        x[g.integers(0, rows), g.integers(0, cols)] = np.nan
        x[g.integers(0, rows), g.integers(0, cols)] = 3e38
    if dtype == "bf16":
        from workloads import to_bf16_bits
        return to_bf16_bits(x)
    return x


def run(rt, x_np, gran, fmt, mode, s_given=None, r_given=None, amax=True, counts=True, pad=0):
    rows, cols = x_np.shape
    if pad:
        xs = np.zeros((rows, cols + pad), x_np.dtype)
        xs[:, :cols] = x_np
        X = dev(xs)[:, :cols]
    else:
        X = dev(x_np)
    G = (1 if gran[0] == 0 else rows // gran[0], 1 if gran[1] == 0 else cols // gran[1])
    S = dev(s_given) if s_given is not None else torch.full(G, float("nan"), device="cuda")
    R = (dev(r_given) if r_given is not None else
         (torch.full(G, float("nan"), device="cuda") if mode == rt.DYNAMIC else None))
    Q = torch.full((rows, cols + pad), 0xAA, dtype=torch.uint8, device="cuda")[:, :cols]
    QT = torch.full((cols, rows + pad), 0xAA, dtype=torch.uint8, device="cuda")[:, :rows]
    A = torch.full(G, float("nan"), device="cuda") if amax else None
    C = torch.full((2,), -1, dtype=torch.int64, device="cuda") if counts else None
    rt.fp8_quantize_transpose(X, gran, fmt, mode, 1e-12, False, S, R, Q, QT, A, C)
    torch.cuda.synchronize()
    return (host(Q), host(QT), host(S), None if R is None else host(R),
            None if A is None else host(A), None if C is None else host(C))


SHAPES = [(16, 16), (144, 272), (256, 1024), (1040, 48)]
GRANS = [(0, 0), (1, 0), (0, 1)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", GRANS)
def test_dynamic_bit_exact(rt, orc, shape, dtype, fmt, gran):
    x = make_input(case_seed(shape, dtype, fmt, gran), *shape, dtype)
    q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, gran)
    Q, QT, S, R, A, C = run(rt, x, gran, fmt, rt.DYNAMIC)
    assert np.array_equal(Q, q), "row-major codes"
    assert np.array_equal(QT, qt), "K-major codes"
    assert same_f32(S, s) and same_f32(R, r) and same_f32(A, am)
    assert C.tolist() == cnt.astype(np.int64).tolist()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("with_inv", [True, False])
def test_given_bit_exact_strided_special(rt, orc, dtype, fmt, gran, with_inv):
    rows, cols = 272, 400
    x = make_input(7 + fmt, rows, cols, dtype, special=True)
    G = (1 if gran[0] == 0 else rows, 1 if gran[1] == 0 else cols)
    sg = np.exp(np.random.default_rng(8).uniform(-8, 4, G)).astype(np.float32)
    rg = (1.0 / sg.astype(np.float64)).astype(np.float32) * np.float32(1.0000001) if with_inv else None
    q, qt, s, r, am, cnt = orc.quantize_transpose(x, fmt, gran, mode=orc.GIVEN, scale=sg, inv_scale=rg)
    Q, QT, S, R, A, C = run(rt, x, gran, fmt, rt.GIVEN, s_given=sg, r_given=rg, pad=32)
    assert np.array_equal(Q, q), "row-major codes"
    assert np.array_equal(QT, qt), "K-major codes"
    assert same_f32(A, am)
    assert C.tolist() == cnt.astype(np.int64).tolist()


@pytest.mark.parametrize("gran", GRANS)
def test_null_optional_outputs(rt, orc, gran):
    x = make_input(11, 128, 256, "bf16")
    q, qt, s, r, am, cnt = orc.quantize_transpose(x, 0, gran)
    Q, QT, S, R, A, C = run(rt, x, gran, 0, rt.DYNAMIC, amax=False, counts=False)
    assert np.array_equal(Q, q) and np.array_equal(QT, qt) and same_f32(S, s)
