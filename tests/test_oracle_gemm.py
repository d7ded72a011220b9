"""Pins for the oracle's scaled GEMM reference.

- exact integer (__int128) inner sums per constant-scale K-run, compared with
  the plain binary64 accumulation;
- a library route: torch's float8 decode, scales expanded per element, and a
  numpy float64 matmul, (A o S_A)(B o S_B)^T;
- closed forms: B = identity gives the dequantized A; K = 1 gives one product.
"""
import numpy as np
import pytest
import torch
from workloads import case_seed

TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def lib_decode(codes, f):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TORCH[f]).to(torch.float64).numpy()


def expand(s, rows, cols, gran):
    er = rows if gran[0] <= 0 else gran[0]
    ec = cols if gran[1] <= 0 else gran[1]
    s = np.asarray(s, np.float64).reshape(-(-rows // er), -(-cols // ec))
    return np.repeat(np.repeat(s, er, axis=0), ec, axis=1)[:rows, :cols]


def random_case(g, M, N, K, fa, fb, ga, gb):
    def codes(shape, f):
        c = g.integers(0, 256, shape).astype(np.uint8)
        bad = np.isnan(lib_decode(c, f)) | np.isinf(lib_decode(c, f))
        c[bad] = 0x3C
        return c
    a = codes((M, K), fa)
    b = codes((N, K), fb)
    nga = (-(-M // (M if ga[0] <= 0 else ga[0])), -(-K // (K if ga[1] <= 0 else ga[1])))
    ngb = (-(-N // (N if gb[0] <= 0 else gb[0])), -(-K // (K if gb[1] <= 0 else gb[1])))
    sa = np.exp(g.uniform(-6, 2, nga)).astype(np.float32)
    sb = np.exp(g.uniform(-6, 2, ngb)).astype(np.float32)
    return a, b, sa, sb


CASES = [
    (0, 0, (0, 0), (0, 0)),
    (0, 0, (1, 0), (1, 0)),
    (0, 0, (1, 128), (128, 128)),
    (0, 0, (1, 32), (1, 32)),
    (1, 0, (0, 0), (0, 0)),
    (1, 0, (1, 128), (1, 0)),
]


@pytest.mark.parametrize("fa,fb,ga,gb", CASES)
def test_gemm_binary64_matches_exact_integer_sums(orc, fa, fb, ga, gb):
    g = np.random.default_rng(case_seed(fa, fb, ga, gb))
    M, N, K = 37, 150, 416
    a, b, sa, sb = random_case(g, M, N, K, fa, fb, ga, gb)
    m = g.integers(0, M, 600)
    n = g.integers(0, N, 600)
    y, S = orc.gemm_points(a, fa, sa, ga, b, fb, sb, gb, m, n)
    ye = orc.gemm_points_exact(a, fa, sa, ga, b, fb, sb, gb, m, n)
    assert np.all(np.abs(y - ye) <= 1e-13 * S + 1e-300)


@pytest.mark.parametrize("fa,fb,ga,gb", CASES)
def test_gemm_matches_library_route(orc, fa, fb, ga, gb):
    g = np.random.default_rng(7 + fa)
    M, N, K = 19, 140, 288
    a, b, sa, sb = random_case(g, M, N, K, fa, fb, ga, gb)
    bias = g.standard_normal(N).astype(np.float32)
    A = lib_decode(a, fa) * expand(sa, M, K, ga)
    B = lib_decode(b, fb) * expand(sb, N, K, gb)
    ref = A @ B.T + bias.astype(np.float64)
    y, S = orc.gemm_full(a, fa, sa, ga, b, fb, sb, gb, bias=bias)
    assert np.all(np.abs(y - ref) <= 1e-13 * S + 1e-300)
    assert np.allclose(S, np.abs(A) @ np.abs(B).T, rtol=1e-13)


def test_gemm_identity_b_gives_dequantized_a(orc):
    g = np.random.default_rng(1)
    M, K = 24, 64
    a, _, sa, _ = random_case(g, M, K, K, 0, 0, (1, 0), (0, 0))
    b = np.zeros((K, K), np.uint8)
    np.fill_diagonal(b, 0x38)                 # E4M3 1.0
    sb = np.array([[1.0]], np.float32)
    y, _ = orc.gemm_full(a, 0, sa, (1, 0), b, 0, sb, (0, 0))
    deq = orc.dequantize(a, 0, sa, (1, 0))    # fl32(s * dec); s * dec is exact in binary64
    assert np.array_equal(y, lib_decode(a, 0) * sa.astype(np.float64).reshape(M, 1))
    assert np.array_equal(y.astype(np.float32), deq)


def test_gemm_k1_single_product_and_bf16_bias(orc):
    a = np.array([[0x44], [0xB0]], np.uint8)   # E4M3 3.0, -0.5
    b = np.array([[0x3D], [0xC0]], np.uint8)   # E5M2 1.25, -2.0
    sa = np.array([[0.5]], np.float32)
    sb = np.array([[4.0]], np.float32)
    bias = np.array([0x3F80, 0xC000], np.uint16)  # bf16 1.0, -2.0
    y, S = orc.gemm_full(a, 0, sa, (0, 0), b, 1, sb, (0, 0), bias=bias)
    assert y.tolist() == [[0.5 * 4 * 3.0 * 1.25 + 1.0, 0.5 * 4 * 3.0 * -2.0 - 2.0],
                          [0.5 * 4 * -0.5 * 1.25 + 1.0, 0.5 * 4 * -0.5 * -2.0 - 2.0]]
    assert S.tolist() == [[7.5, 12.0], [1.25, 2.0]]
