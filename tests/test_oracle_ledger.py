"""Pins for the oracle's quantization-error statistics (the granularity
ledger's sums), each against something other than the function itself:

- the weight sums against numpy float64 on the pinned dequantization
  (oracle.dequantize): sum e^2, sum w^2, max |e|;
- the output sums against numpy float64 matrix products x W^T and x W_hat^T;
- a weight already on the FP8 grid (w = s dec(q) exactly) has zero error,
  y_q = y_ref and therefore sum y_q^2 = sum y_ref^2 = sum y_ref y_q;
- scaling the weight and its scales by 2^j scales sum e^2 by exactly 4^j;
- NaN in the weight propagates to the error sums and max |e|.
"""
import numpy as np
import pytest

from workloads import case_seed, to_bf16_bits


def bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make(orc, seed, N, K, M, fmt, gran, dtype):
    g = np.random.default_rng(seed)
    wf = (g.standard_normal((N, K)) * np.exp(g.uniform(-3, 3, (N, 1)))).astype(np.float32)
    w = to_bf16_bits(wf) if dtype == "bf16" else wf
    q, s, _, _, _ = orc.quantize(w, fmt, gran)
    x = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    return w, q, s, x


def wdouble(w):
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", [(0, 0), (1, 0), (1, 32), (16, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_against_numpy(orc, fmt, gran, dtype):
    N, K, M = 24, 64, 5
    w, q, s, x = make(orc, case_seed(fmt, gran, dtype), N, K, M, fmt, gran, dtype)
    st = orc.quant_error(w, q, fmt, s, gran, x)
    wh = orc.dequantize(q, fmt, s, gran).astype(np.float64)
    wd = wdouble(w)
    e = wh - wd
    assert np.isclose(st[0], (e * e).sum(), rtol=1e-12, atol=0)
    assert np.isclose(st[1], (wd * wd).sum(), rtol=1e-12, atol=0)
    assert st[2] == np.abs(e).max()
    xd = bf16_to_f64(x)
    yr = xd @ wd.T
    yq = xd @ wh.T
    d = xd @ e.T
    ref = [(d * d).sum(), (yr * yr).sum(), (yq * yq).sum(), (yr * yq).sum()]
    assert np.allclose(st[3:], ref, rtol=1e-9, atol=0)
    st0 = orc.quant_error(w, q, fmt, s, gran, None)
    assert np.array_equal(st0[:3], st[:3]) and not st0[3:].any()


def test_weight_on_grid_has_no_error(orc):
    N, K, M = 16, 48, 4
    w, q, s, x = make(orc, 3, N, K, M, 0, (1, 16), "f32")
    exact = orc.dequantize(q, 0, s, (1, 16))       # w = s dec(q), binary32
    q2, s2, _, _, _ = orc.quantize(exact, 0, (1, 16), mode=orc.GIVEN, scale=s)
    assert np.array_equal(q2, q)
    st = orc.quant_error(exact, q, 0, s, (1, 16), x)
    assert st[0] == 0 and st[2] == 0 and st[3] == 0
    assert st[4] == st[5] == st[6]


def test_power_of_two_scaling(orc):
    N, K = 12, 32
    w, q, s, _ = make(orc, 5, N, K, 1, 0, (1, 0), "f32")
    base = orc.quant_error(w, q, 0, s, (1, 0))
    for j in (-3, 4):
        st = orc.quant_error((w * np.float32(2.0 ** j)).astype(np.float32), q, 0,
                             (s * np.float32(2.0 ** j)).astype(np.float32), (1, 0))
        assert st[0] == base[0] * 4.0 ** j and st[1] == base[1] * 4.0 ** j
        assert st[2] == base[2] * 2.0 ** j


def test_nan_propagates(orc):
    w, q, s, x = make(orc, 9, 8, 32, 2, 0, (1, 0), "f32")
    w = w.copy()
    w[3, 5] = np.nan
    st = orc.quant_error(w, q, 0, s, (1, 0), x)
    assert np.isnan(st[0]) and np.isnan(st[2]) and np.isnan(st[3])
