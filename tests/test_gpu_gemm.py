"""Parity of the HIP scaled GEMM with the CPU oracle (binary64 reference) on
every output element, at sizes that span several 128x128 tiles with ragged
M, N and K tails.  Operands are FP8 codes and scales produced by the ORACLE's
quantizer from seeded normal data (the GEMM under test never feeds its own
inputs).  Acceptance: fp32 |y - y_ref| <= 1e-5 * sum_k |s_a s_b a_k b_k| + T_hw,
bf16 within one bf16 ulp of the rounded reference (see gpu_helpers), where
T_hw bounds the truncation of the matrix cores' FP8 dot product (measured:
8-product groups aligned to their largest exponent sum keep 13 bits below
it).  The count of elements that need T_hw is printed and bounded."""
import numpy as np
import pytest
import torch

from gpu_helpers import check_gemm, dev, host
from workloads import case_seed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    return rt


def operands(orc, seed, M, N, K, fa, fb, ga, gb, pow2):
    g = np.random.default_rng(seed)
    xa = g.standard_normal((M, K)).astype(np.float32)
    xb = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    a, sa, _, _, _ = orc.quantize(xa, fa, ga, pow2=pow2)
    b, sb, _, _, _ = orc.quantize(xb, fb, gb, pow2=pow2)
    return a, sa, b, sb


def run_gemm(rt, a, fa, ga, sa, b, fb, gb, sb, out, bias=None, flags=0):
    M, N = a.shape[0], b.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                   device="cuda")
    rt.fp8_scaled_gemm(dev(a), fa, ga, dev(sa), dev(b), fb, gb, dev(sb), y,
                       bias=None if bias is None else dev(bias), flags=flags)
    torch.cuda.synchronize()
    return host(y)


SHAPES = [(200, 300, 320), (64, 256, 1024), (16, 512, 1024), (5, 200, 2048), (7, 203, 1024), (257, 129, 256),
          (300, 520, 512), (520, 776, 1024)]
SCALES = [((0, 0), (0, 0)), ((1, 0), (1, 0)), ((1, 128), (128, 128)), ((1, 128), (1, 0)),
          ((0, 0), (128, 128))]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fa", [0, 1])
@pytest.mark.parametrize("grans", SCALES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_matches_oracle(rt, orc, shape, fa, grans, out):
    M, N, K = shape
    ga, gb = grans
    a, sa, b, sb = operands(orc, case_seed(shape, fa, grans), M, N, K, fa, 0, ga, gb, False)
    bias = None
    if out == "bf16":
        from workloads import to_bf16_bits
        bias = to_bf16_bits((np.random.default_rng(1).standard_normal(N) * 0.1).astype(np.float32))
    y = run_gemm(rt, a, fa, ga, sa, b, 0, gb, sb, out, bias)
    yref, S = orc.gemm_full(a, fa, sa, ga, b, 0, sb, gb, bias=bias)
    thw = orc.dot_truncation_bound_full(a, fa, sa, ga, b, 0, sb, gb)
    bias_f = None if bias is None else orc.bf16_bits_to_f32(bias)
    ok, st = check_gemm(y, yref, S, out == "bf16", orc, t_hw=thw,
                        bias=None if bias is None else np.broadcast_to(bias_f, yref.shape))
    print("gemm", shape, fa, grans, out, st)
    assert ok, st


@pytest.mark.parametrize("shape", [(200, 300, 320), (128, 256, 512), (300, 520, 512), (520, 776, 1024),
                                   (16, 512, 1024), (40, 1003, 1024), (64, 4160, 512)])
@pytest.mark.parametrize("fa", [0, 1])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_mx32_pow2(rt, orc, shape, fa, out):
    """1x32 power-of-two scales on both operands: the general kernel, the
    large kernel (split K parts on the small grids) and the decode kernel
    (M <= 64: one to four row tiles of A per workgroup, a ragged N)."""
    M, N, K = shape
    ga = gb = (1, 32)
    a, sa, b, sb = operands(orc, 3 + fa, M, N, K, fa, 0, ga, gb, True)
    y = run_gemm(rt, a, fa, ga, sa, b, 0, gb, sb, out, flags=rt.POW2_SCALES)
    yref, S = orc.gemm_full(a, fa, sa, ga, b, 0, sb, gb)
    thw = orc.dot_truncation_bound_full(a, fa, sa, ga, b, 0, sb, gb)
    ok, st = check_gemm(y, yref, S, out == "bf16", orc, t_hw=thw)
    print("gemm mx32", shape, fa, out, st)
    assert ok, st


def test_gemm_fp32_bias_and_strided_output(rt, orc):
    M, N, K = 96, 200, 384
    a, sa, b, sb = operands(orc, 9, M, N, K, 0, 0, (1, 0), (1, 0), False)
    bias = np.random.default_rng(2).standard_normal(N).astype(np.float32)
    yb = torch.full((M, N + 56), float("nan"), device="cuda")
    y = yb[:, :N]
    rt.fp8_scaled_gemm(dev(a), 0, (1, 0), dev(sa), dev(b), 0, (1, 0), dev(sb), y, bias=dev(bias))
    torch.cuda.synchronize()
    yref, S = orc.gemm_full(a, 0, sa, (1, 0), b, 0, sb, (1, 0), bias=bias)
    thw = orc.dot_truncation_bound_full(a, 0, sa, (1, 0), b, 0, sb, (1, 0))
    ok, st = check_gemm(host(y), yref, S, False, orc, t_hw=thw, bias=np.broadcast_to(bias, yref.shape))
    assert ok, st
    assert np.all(np.isnan(host(yb)[:, N:]))          # nothing written past N


def test_gemm_identity_weight_reproduces_dequantized_a(rt, orc):
    M, K = 130, 256
    g = np.random.default_rng(4)
    a, sa, _, _, _ = orc.quantize(g.standard_normal((M, K)).astype(np.float32), 0, (1, 0))
    b = np.zeros((K, K), np.uint8)
    np.fill_diagonal(b, 0x38)
    sb = np.ones((1, 1), np.float32)
    y = run_gemm(rt, a, 0, (1, 0), sa, b, 0, (0, 0), sb, "f32")
    assert np.array_equal(y, orc.dequantize(a, 0, sa, (1, 0)))


def test_fp8_dot_unit_truncation_model(rt, orc):
    """Documents the matrix-core behaviour the tolerance term rests on: in a
    row [X, d, 0, ...] times a column of ones, d survives when X / d <= 2^13
    and is dropped when X / d >= 2^14 (same 8-product group); a d placed in
    another group is kept."""
    K = 128
    rows = []
    expect = []
    for ex in range(-9, 9):
        for ed in range(-9, ex + 1):
            X, d = 2.0 ** ex, 2.0 ** ed
            same = np.zeros(K, np.float32)
            same[0], same[1] = X, d
            other = np.zeros(K, np.float32)
            other[0], other[8] = X, d
            rows += [same, other]
            expect += [X + d if ex - ed <= 13 else X, X + d]
    A = np.array([[orc.encode(v, 0) for v in r] for r in rows], np.uint8)
    B = np.full((16, K), 0x38, np.uint8)
    one = np.ones((1, 1), np.float32)
    y = run_gemm(rt, A, 0, (0, 0), one, B, 0, (0, 0), one, "f32")
    assert np.array_equal(y[:, 0], np.array(expect, np.float32))


@pytest.mark.parametrize("fa", [0, 1])
@pytest.mark.parametrize("grans", [((0, 0), (0, 0)), ((1, 0), (1, 0))])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_split_last_wave(rt, orc, fa, grans, out):
    """4096 x 4300 x 1024: 16 x 17 = 272 tiles of 256 x 256 on 256 CUs, so the
    last 16 tiles run as K-split units plus a reduction.  Whole rows and
    columns through the split tiles (rows 3072-4095, columns 3328-4299) and
    through whole tiles, plus random points, against the oracle."""
    M, N, K = 4096, 4300, 1024
    ga, gb = grans
    a, sa, b, sb = operands(orc, 11 + fa, M, N, K, fa, 0, ga, gb, False)
    bias = None
    if out == "bf16":
        from workloads import to_bf16_bits
        bias = to_bf16_bits((np.random.default_rng(2).standard_normal(N) * 0.1).astype(np.float32))
    y = run_gemm(rt, a, fa, ga, sa, b, 0, gb, sb, out, bias)
    rows = np.array([3072, 3583, 4095, 17])
    cols = np.array([3328, 3999, 4299, 5])
    g = np.random.default_rng(5)
    m = np.concatenate([np.repeat(rows, N), np.repeat(np.arange(M), len(cols)), g.integers(0, M, 8192)])
    n = np.concatenate([np.tile(np.arange(N), len(rows)), np.tile(cols, M), g.integers(0, N, 8192)])
    yref, S = orc.gemm_points(a, fa, sa, ga, b, 0, sb, gb, m, n, bias=bias)
    thw = orc.dot_truncation_bound(a, fa, sa, ga, b, 0, sb, gb, m, n)
    bias_f = None if bias is None else orc.bf16_bits_to_f32(bias)[n]
    ok, st = check_gemm(y[m, n], yref, S, out == "bf16", orc, t_hw=thw, bias=bias_f)
    print("split", fa, grans, out, st)
    assert ok, st


def test_k32_per_row_scales_are_not_mx_blocks(rt, orc):
    """At K = 32 a {1, 32} group is the whole row: per-token x per-channel
    scales, accepted without the power-of-two flag and computed as per-row."""
    M, N, K = 40, 72, 32
    a, sa, b, sb = operands(orc, 21, M, N, K, 0, 0, (1, 0), (1, 0), False)
    y = run_gemm(rt, a, 0, (1, 32), sa, b, 0, (1, 32), sb, "f32")
    yref, S = orc.gemm_full(a, 0, sa, (1, 0), b, 0, sb, (1, 0))
    thw = orc.dot_truncation_bound_full(a, 0, sa, (1, 0), b, 0, sb, (1, 0))
    ok, st = check_gemm(y, yref, S, False, orc, t_hw=thw)
    assert ok, st


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("N", [256, 1152], ids=["exact-products", "fp8-cores"])
def test_decode_gemm_special_codes(rt, orc, N, packed):
    """E5M2 activation codes holding +Inf, -Inf and NaN in the decode kernel,
    with K = 1024: eight 128-deep steps over 16 waves, so every wave that has
    a step also passes its odd-count tail, which must add nothing (no 0 x Inf).
    Non-finite outputs (Inf of either sign, NaN from Inf - Inf, 0 x Inf or a
    NaN code) must sit exactly where the binary64 reference has them, the rest
    within the acceptance rule.  N = 256 runs the exact-product variant
    (automatic for small weights), N = 1152 the FP8 matrix cores."""
    M, K = 16, 1024
    a, sa, b, sb = operands(orc, case_seed("special", N), M, N, K, 1, 0, (1, 0), (1, 0), False)
    a = a.copy()
    a[0, 7 * 128 + 5] = 0x7C                  # +Inf in the last step
    a[1, 3 * 128 + 70] = 0xFC                 # -Inf
    a[2, 1000] = 0x7E                         # NaN
    a[3, 10], a[3, 900] = 0x7C, 0xFC          # +Inf and -Inf in one row
    a[4, 1023] = 0x7C                         # +Inf at the last K
    b = b.copy()
    b[7, :] = 0                               # a zero weight row: 0 x Inf
    bd = dev(b)
    if packed:
        bd = rt.fp8_pack_weights16(bd)
    y = torch.full((M, N), 12345.0, dtype=torch.float32, device="cuda")
    rt.fp8_scaled_gemm(dev(a), 1, (1, 0), dev(sa), bd, 0, (1, 0), dev(sb), y)
    torch.cuda.synchronize()
    y = host(y)
    yref, S = orc.gemm_full(a, 1, sa, (1, 0), b, 0, sb, (1, 0))
    fin = np.isfinite(yref)
    assert np.array_equal(np.isnan(y), np.isnan(yref))
    assert np.array_equal(np.isposinf(y), np.isposinf(yref))
    assert np.array_equal(np.isneginf(y), np.isneginf(yref))
    assert (~fin).sum() >= 4 * N - 8
    t_hw = None if N * K <= rt.EXACT_AUTO_BYTES else orc.dot_truncation_bound_full(a, 1, sa, (1, 0), b, 0, sb, (1, 0))
    rows = fin.all(axis=1)
    ok, st = check_gemm(y[rows], yref[rows], S[rows], False, orc, t_hw=None if t_hw is None else t_hw[rows])
    assert ok, st


SPECIAL_ROUTES = [  # name, M, N, K, ga, gb
    ("general-ragged-k", 96, 160, 528, (1, 0), (1, 0)),
    ("large", 256, 384, 512, (1, 0), (1, 0)),
    ("kblock", 256, 256, 512, (1, 128), (128, 128)),
]


@pytest.mark.parametrize("route", SPECIAL_ROUTES, ids=[r[0] for r in SPECIAL_ROUTES])
def test_gemm_special_codes_other_kernels(rt, orc, route):
    """The same special E5M2 codes through the general kernel (a ragged last
    K step, padded on both operands), the large kernel and the K-blocked
    kernel: non-finite outputs exactly where the reference has them."""
    name, M, N, K, ga, gb = route
    a, sa, b, sb = operands(orc, case_seed("special-other", name), M, N, K, 1, 0, ga, gb, False)
    a = a.copy()
    a[0, K - 1] = 0x7C
    a[1, K // 2] = 0xFC
    a[2, 3] = 0x7E
    a[3, 10], a[3, K - 20] = 0x7C, 0xFC
    b = b.copy()
    b[7, :] = 0
    y = run_gemm(rt, a, 1, ga, sa, b, 0, gb, sb, "f32")
    yref, S = orc.gemm_full(a, 1, sa, ga, b, 0, sb, gb)
    assert np.array_equal(np.isnan(y), np.isnan(yref))
    assert np.array_equal(np.isposinf(y), np.isposinf(yref))
    assert np.array_equal(np.isneginf(y), np.isneginf(yref))
    rows = np.isfinite(yref).all(axis=1)
    t_hw = orc.dot_truncation_bound_full(a, 1, sa, ga, b, 0, sb, gb)
    ok, st = check_gemm(y[rows], yref[rows], S[rows], False, orc, t_hw=t_hw[rows])
    assert ok, st


@pytest.mark.parametrize("M", [16, 64])
def test_decode_mx32_full_size(rt, orc, M):
    """The decode kernel with 1x32 power-of-two scales at the decode layer's
    size (M x 8192 x 8192, bf16 out, bias): A and W quantized on the device
    (1x32 groups, power-of-two round-up), then every row on a column sample
    (the first and last 256 columns and 512 random ones) against the oracle
    under the one acceptance rule."""
    N = K = 8192
    print("decode mx32 full size, M =", M, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(case_seed("decode-mx32-full", M))
    x = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    bias = (torch.randn(N, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    A = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    B = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 32), device="cuda")
    sb = torch.empty((N, K // 32), device="cuda")
    rt.fp8_quantize(x, (1, 32), 0, rt.DYNAMIC, 1e-12, True, sa, None, A)
    rt.fp8_quantize(w, (1, 32), 0, rt.DYNAMIC, 1e-12, True, sb, None, B)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_scaled_gemm(A, 0, (1, 32), sa, B, 0, (1, 32), sb, y, bias=bias, flags=rt.POW2_SCALES)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([np.arange(256), np.arange(N - 256, N), rng.integers(256, N - 256, 512)]))
    m = np.repeat(np.arange(M), len(cols))
    n = np.tile(cols, M)
    a, b, ha, hb = host(A), host(B), host(sa), host(sb)
    bias_bits = host(bias)
    yref, S = orc.gemm_points(a, 0, ha, (1, 32), b, 0, hb, (1, 32), m, n, bias=bias_bits)
    thw = orc.dot_truncation_bound(a, 0, ha, (1, 32), b, 0, hb, (1, 32), m, n)
    bias_f = orc.bf16_bits_to_f32(bias_bits).astype(np.float64)[n]
    ok, st = check_gemm(host(y)[m, n], yref, S, True, orc, t_hw=thw, bias=bias_f)
    print("decode mx32", M, st)
    assert ok, st
