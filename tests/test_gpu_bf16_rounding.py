"""BF16 output rounding of every GEMM route, bit for bit.

"FP8 formats and scaling for LLM inference", section "The full precision
contract of one FP8 GEMM": the GEMM accumulates in FP32 and writes BF16.  The
kernels convert their binary32 result to BF16 (the large, K-blocked, decode and
weight-only kernels with the hardware conversion, the general kernel with an
integer rounding); this test pins that conversion as round-to-nearest-even on
every finite input, the subnormal range and the rounding overflow to Inf
included.

The operands make the binary32 result known exactly: A (or the activations)
holds one code 1.0 per row, at k = 0, and B holds 1.0 at k = 0 of every row,
so the accumulator is exactly 1 and y[m, n] = s_a(m) s_b(n) with one binary32
rounding at most (every order of multiplying s_a, s_b and an exact 1 rounds
once).  s_b(n) walks every value of the 17 low significand bits (the rounded
away half and the kept last bit) under a seeded high part, one in eight of
them all ones so that rounding carries into the exponent; s_a(m) = +-2^e with
e from -149 to 127, so results span the binary32 subnormals down to the
smallest one and the top binade.  The reference is the oracle's BF16 rounding of fl32(s_a s_b)
(orc_dequantize with one scale per element on the code 1.0), which equals the
rounding of the exact product: rounding to binary32 first is innocuous for a
format of 8 significant bits (24 >= 2 * 8 + 2).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from workloads import case_seed

pytestmark = pytest.mark.gpu

ONE_E4M3 = 0x38      # 1.0 in E4M3 (exponent 7 = bias, mantissa 0)
NPAT = 1 << 17       # every value of the low 17 significand bits


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    return rt


def column_scales(seed):
    """s_b(n) in [1, 2): low 17 significand bits = n, the 6 bits above seeded
    (all ones for one column in eight)."""
    g = np.random.default_rng(seed)
    n = np.arange(NPAT, dtype=np.uint32)
    hi = g.integers(0, 64, NPAT, dtype=np.uint32)
    hi[g.integers(0, 8, NPAT) == 0] = 63
    bits = np.uint32(0x3F800000) | (hi << np.uint32(17)) | n
    return bits.view(np.float32)


def row_scales(M, lo=-149):
    """s_a(m) = (-1)^m 2^e, e spread over [lo, 127] (the last row at 127): no
    product rounds to zero, whose sign a kernel's zero bias may change."""
    e = np.round(np.linspace(lo, 127, M)).astype(np.int64)
    return (np.where(np.arange(M) % 2 == 0, 1.0, -1.0) * np.exp2(e.astype(np.float64))).astype(np.float32)


def expected_bits(orc, sa, sb):
    prod = (sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :]).astype(np.float32)
    ones = np.full(prod.shape, ONE_E4M3, np.uint8)
    return orc.dequantize(ones, orc.E4M3, prod, (1, 1), orc.BF16)


def one_hot_codes(rows, K):
    q = np.zeros((rows, K), np.uint8)
    q[:, 0] = ONE_E4M3
    return q


def compare(y_bits, ref_bits):
    bad = np.flatnonzero(y_bits.ravel() != ref_bits.ravel())
    assert bad.size == 0, "%d of %d BF16 outputs differ from round-to-nearest-even; first: got %#06x want %#06x" % (
        bad.size, y_bits.size, int(y_bits.ravel()[bad[0]]), int(ref_bits.ravel()[bad[0]]))


# (route, M, K, A granularity): the large kernel (per-row scales, K a multiple
# of 256, M >= 65), the K-blocked kernel (1 x 128 groups on A), the general
# kernel (K = 128 is not a multiple of 256) and the decode kernel (M <= 64).
ROUTES = [("large", 128, 256, (1, 0)), ("kblocked", 128, 256, (1, 128)), ("general", 128, 128, (1, 0)),
          ("decode", 64, 128, (1, 0))]


@pytest.mark.parametrize("route,M,K,ga", ROUTES, ids=[r[0] for r in ROUTES])
def test_scaled_gemm_bf16_output_is_rne(rt, orc, route, M, K, ga):
    sb = column_scales(case_seed("bf16-rne", route))
    sa = row_scales(M)
    a = one_hot_codes(M, K)
    b = one_hot_codes(NPAT, K)
    if ga == (1, 0):
        sa_arr = sa.reshape(M, 1)
    else:                               # 1 x 128 groups: group 0 carries the row's scale, the rest multiply zeros
        sa_arr = np.ones((M, K // 128), np.float32)
        sa_arr[:, 0] = sa
    y = torch.empty((M, NPAT), dtype=torch.bfloat16, device="cuda")
    rt.fp8_scaled_gemm(dev(a), rt.E4M3, ga, dev(sa_arr), dev(b), rt.E4M3, (1, 0), dev(sb.reshape(NPAT, 1)), y)
    torch.cuda.synchronize()
    compare(host(y), expected_bits(orc, sa, sb))


def test_weight_only_gemm_bf16_output_is_rne(rt, orc):
    M, K = 16, 128
    sb = column_scales(case_seed("bf16-rne", "weight-only"))
    # activations: x[m, 0] = s_a(m), a normal power of two (exact in bf16; the
    # matrix cores' handling of subnormal bf16 inputs is not what is tested)
    sa = row_scales(M, lo=-126)
    x = np.zeros((M, K), np.uint16)
    x[:, 0] = (sa.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((x[:, 0].astype(np.uint32) << 16).view(np.float32), sa)
    w = one_hot_codes(NPAT, K)
    y = torch.empty((M, NPAT), dtype=torch.bfloat16, device="cuda")
    rt.fp8_weight_only_gemm(dev(x), dev(w), rt.E4M3, (1, 0), dev(sb.reshape(NPAT, 1)), y)
    torch.cuda.synchronize()
    compare(host(y), expected_bits(orc, sa, sb))
