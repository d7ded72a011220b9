"""Pins for the oracle's weight-only FP8 GEMM (FP8 weights with their scales,
BF16 activations, the weight restored inside the GEMM), each against
something other than the function itself:

- a library route: torch's float8 decode, the weight scales expanded per
  element, a numpy float64 matmul x (s_w o dec(W))^T, for tensor, channel,
  K-group and 2-D block scales, bf16 and fp32 activations;
- reduction to the FP8 x FP8 reference: when every activation is exactly an
  E4M3 value, the weight-only result equals the scaled GEMM reference with
  those codes as A and a unit activation scale, bit for bit (every product is
  exact and both sum in k order);
- closed forms: the identity weight gives the activations back (plus bias);
  K = 1 gives one product;
- factorisation: K-group scales that are equal along a row give the
  per-channel result bit for bit.
"""
import numpy as np
import pytest
import torch

from workloads import case_seed, to_bf16_bits

TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def lib_decode(codes, f):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TORCH[f]).to(torch.float64).numpy()


def expand(s, rows, cols, gran):
    er = rows if gran[0] <= 0 else gran[0]
    ec = cols if gran[1] <= 0 else gran[1]
    s = np.asarray(s, np.float64).reshape(-(-rows // er), -(-cols // ec))
    return np.repeat(np.repeat(s, er, axis=0), ec, axis=1)[:rows, :cols]


def finite_codes(g, shape, f):
    c = g.integers(0, 256, shape).astype(np.uint8)
    d = lib_decode(c, f)
    c[~np.isfinite(d)] = 0x3C
    return c


def bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def n_groups(n, g):
    return -(-n // (n if g <= 0 else g))


@pytest.mark.parametrize("fw", [0, 1])
@pytest.mark.parametrize("gw", [(0, 0), (1, 0), (1, 16), (4, 8)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_library_route(orc, fw, gw, xdt):
    g = np.random.default_rng(case_seed(fw, gw, xdt))
    M, N, K = 5, 7, 40
    xf = (g.standard_normal((M, K)) * np.exp(g.uniform(-3, 3, (M, 1)))).astype(np.float32)
    x = to_bf16_bits(xf) if xdt == "bf16" else xf
    xd = bf16_to_f64(x) if xdt == "bf16" else xf.astype(np.float64)
    w = finite_codes(g, (N, K), fw)
    sw = np.exp(g.uniform(-6, 2, (n_groups(N, gw[0]), n_groups(K, gw[1])))).astype(np.float32)
    bias = (g.standard_normal(N) * 0.1).astype(np.float32)
    y, S = orc.wonly_gemm_full(x, w, fw, sw, gw, bias=bias)
    wd = lib_decode(w, fw) * expand(sw, N, K, gw)
    ref = xd @ wd.T + bias[None, :].astype(np.float64)
    sref = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(y - ref) <= 1e-13 * (sref + np.abs(bias)[None, :]))
    assert np.allclose(S, sref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fw", [0, 1])
@pytest.mark.parametrize("gw", [(0, 0), (1, 0), (1, 16)])
def test_reduces_to_fp8_gemm(orc, fw, gw):
    g = np.random.default_rng(7 + fw)
    M, N, K = 6, 9, 48
    a = finite_codes(g, (M, K), 0)
    x = lib_decode(a, 0).astype(np.float32)  # exact E4M3 values, also exact in bf16
    w = finite_codes(g, (N, K), fw)
    sw = np.exp(g.uniform(-6, 2, (n_groups(N, gw[0]), n_groups(K, gw[1])))).astype(np.float32)
    one = np.ones((1, 1), np.float32)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y8, S8 = orc.gemm_points(a, 0, one, (0, 0), w, fw, sw, gw, mm.ravel(), nn.ravel())
    assert np.array_equal(bf16_to_f64(to_bf16_bits(x)), x.astype(np.float64))
    for xin in (x, to_bf16_bits(x)):
        y, S = orc.wonly_gemm_full(xin, w, fw, sw, gw)
        assert np.array_equal(y.ravel(), y8) and np.array_equal(S.ravel(), S8)


@pytest.mark.parametrize("fw", [0, 1])
def test_identity_weight(orc, fw):
    g = np.random.default_rng(3)
    M, K = 4, 32
    x = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    one = 0x38 if fw == 0 else 0x3C  # 1.0 in E4M3 / E5M2
    w = np.where(np.eye(K, dtype=bool), one, 0).astype(np.uint8)
    bias = to_bf16_bits((g.standard_normal(K) * 0.1).astype(np.float32))
    y, _ = orc.wonly_gemm_full(x, w, fw, np.ones((1, 1), np.float32), (0, 0), bias=bias)
    assert np.array_equal(y, bf16_to_f64(x) + bf16_to_f64(bias)[None, :])


def test_k1_single_product(orc):
    x = np.array([[3.0], [-0.5]], np.float32)
    w = np.array([[0x44], [0xB0]], np.uint8)  # E4M3: 3.0 and -0.5
    sw = np.array([[0.25], [8.0]], np.float32)
    y, S = orc.wonly_gemm_full(x, w, 0, sw, (1, 0))
    assert np.array_equal(y, np.array([[2.25, -12.0], [-0.375, 2.0]]))
    assert np.array_equal(S, np.abs(y))


@pytest.mark.parametrize("fw", [0, 1])
def test_equal_group_scales_are_per_channel(orc, fw):
    g = np.random.default_rng(11)
    M, N, K = 3, 8, 64
    x = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = finite_codes(g, (N, K), fw)
    sc = np.exp(g.uniform(-4, 2, (N, 1))).astype(np.float32)
    y1, S1 = orc.wonly_gemm_full(x, w, fw, sc, (1, 0))
    y2, S2 = orc.wonly_gemm_full(x, w, fw, np.repeat(sc, 4, axis=1), (1, 16))
    assert np.array_equal(y1, y2) and np.array_equal(S1, S2)
