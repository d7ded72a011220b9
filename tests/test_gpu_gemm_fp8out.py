"""Parity of the FP8-output GEMM (fp8_scaled_gemm_fp8out) with the CPU
oracle.  The binary32 GEMM result is fixed only up to the GEMM tolerance T
(FP32 accumulation order, the matrix cores' dot-product truncation), so each
output code must lie, in signed code order, between the oracle's codes of
y_ref - T and y_ref + T (both cast by the oracle's GIVEN-mode quantize with
the same output scale; the bounds rounded outward to binary32).  amax_y must
be within T of max |y_ref|, and each counter between the number of elements
certain to be counted and the number that may be.  Shapes exercise the
general kernel, the decode kernel (one to four row tiles, per-step block
scales, a ragged last column group), the large kernel and its 1x32 (MX)
path; on the fragment-ordered weight image the decode kernel must give the
row-major call's codes, amax and counters bit for bit."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from workloads import case_seed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    return rt


def operands(orc, seed, M, N, K, fa, ga, gb, pow2):
    g = np.random.default_rng(seed)
    xa = g.standard_normal((M, K)).astype(np.float32)
    xb = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    a, sa, _, _, _ = orc.quantize(xa, fa, ga, pow2=pow2)
    b, sb, _, _, _ = orc.quantize(xb, 0, gb, pow2=pow2)
    return a, sa, b, sb


def order(c):
    c = np.asarray(c).astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


CASES = [  # (shape, ga, gb, pow2)
    ((200, 300, 320), (0, 0), (0, 0), False),    # general kernel, ragged
    ((520, 776, 1024), (0, 0), (1, 0), False),   # large kernel, per-channel B
    ((16, 512, 1024), (1, 0), (1, 0), False),    # decode kernel
    ((40, 1003, 1024), (0, 0), (1, 0), False),   # decode kernel, two row tiles, ragged N
    ((64, 4160, 512), (1, 0), (1, 0), False),    # decode kernel, four row tiles in one workgroup
    ((16, 640, 1024), (1, 128), (128, 128), False),  # decode kernel, per-step block scales
    ((264, 400, 512), (1, 128), (128, 128), False),  # K-blocked scales (general kernel)
    ((520, 776, 1024), (1, 32), (1, 32), True),  # 1x32 power-of-two scales (large kernel)
    ((40, 1003, 1024), (1, 32), (1, 32), True),  # 1x32 power-of-two scales (decode kernel)
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("fy", [0, 1])
@pytest.mark.parametrize("with_inv", [True, False])
def test_fp8_output_within_tolerance(rt, orc, case, fy, with_inv):
    check_fp8out(rt, orc, case, fy, with_inv)


@pytest.mark.parametrize("fy,with_inv", [(0, False), (1, True)])
def test_fp8_output_split_last_wave(rt, orc, fy, with_inv):
    """520 x 22000 x 512: 3 x 86 = 258 tiles of 256 x 256 on 256 CUs, so the
    last two tiles (columns 21760-21999, rows 256-519, the second ragged in
    both dimensions) run as K-split units; the reduction kernel requantizes
    them and supplies their statistics partials."""
    check_fp8out(rt, orc, ((520, 22000, 512), (1, 0), (1, 0), False), fy, with_inv)


IMAGE_CASES = [  # decode shapes: (shape, ga, gb)
    ((16, 512, 1024), (1, 0), (1, 0)),
    ((40, 1003, 1024), (0, 0), (1, 0)),        # two row tiles, ragged N (a short last 16-row group)
    ((64, 4160, 512), (1, 0), (1, 0)),         # four row tiles in one workgroup
    ((16, 640, 1024), (1, 128), (128, 128)),   # per-step block scales
    ((16, 8192, 8192), (1, 0), (1, 0)),        # the decode layer's size
]


@pytest.mark.parametrize("case", IMAGE_CASES, ids=[str(c) for c in IMAGE_CASES])
@pytest.mark.parametrize("fy", [0, 1])
def test_fp8_output_on_weight_image(rt, case, fy):
    """FP8 output with B as the fragment-ordered image: the decode kernel reads
    the same bytes in the same order, so codes, amax and counters equal the
    row-major call's bit for bit (that call is checked against the oracle
    above)."""
    (M, N, K), ga, gb = case
    g = torch.Generator(device="cuda")
    g.manual_seed(case_seed("fp8out-image", case, fy))
    x = torch.randn((M, K), device="cuda", generator=g)
    w = torch.randn((N, K), device="cuda", generator=g) * 0.02
    sa = torch.empty(rt.scale_shape((M, K), ga), device="cuda")
    sb = torch.empty(rt.scale_shape((N, K), gb), device="cuda")
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    rt.fp8_quantize(x, ga, 0, rt.DYNAMIC, 1e-12, False, sa, None, a)
    rt.fp8_quantize(w, gb, 0, rt.DYNAMIC, 1e-12, False, sb, None, b)
    bias = torch.randn(N, device="cuda", generator=g).to(torch.bfloat16)
    # an output scale that saturates the largest outputs: half of max |y| / F_max
    am0 = torch.zeros(1, device="cuda")
    rt.fp8_scaled_gemm_fp8out(a, 0, ga, sa, b, 0, gb, sb, torch.empty((M, N), dtype=torch.uint8, device="cuda"),
                              fy, torch.ones((1, 1), device="cuda"), None, am0, None, bias=bias)
    sy = (am0 * 0.5 / (448.0 if fy == 0 else 57344.0)).reshape(1, 1)
    out = []
    for B in (b, rt.fp8_pack_weights16(b)):
        yq = torch.full((M, N), 0xAA, dtype=torch.uint8, device="cuda")
        amax = torch.full((1,), float("nan"), device="cuda")
        cnt = torch.full((2,), -1, dtype=torch.int64, device="cuda")
        rt.fp8_scaled_gemm_fp8out(a, 0, ga, sa, B, 0, gb, sb, yq, fy, sy, None, amax, cnt, bias=bias)
        out.append((yq, amax, cnt))
    torch.cuda.synchronize()
    (q0, a0, c0), (q1, a1, c1) = out
    assert torch.equal(q0, q1)
    assert torch.equal(a0.view(torch.int32), a1.view(torch.int32))
    assert c0.tolist() == c1.tolist() and c0[0].item() > 0


def check_fp8out(rt, orc, case, fy, with_inv):
    (M, N, K), ga, gb, pow2 = case
    fa = 0
    a, sa, b, sb = operands(orc, case_seed(case, fy), M, N, K, fa, ga, gb, pow2)
    from workloads import to_bf16_bits
    bias = to_bf16_bits((np.random.default_rng(3).standard_normal(N) * 0.1).astype(np.float32))
    yref, S = orc.gemm_full(a, fa, sa, ga, b, 0, sb, gb, bias=bias)
    thw = orc.dot_truncation_bound_full(a, fa, sa, ga, b, 0, sb, gb)
    bias_f = orc.bf16_bits_to_f32(bias).astype(np.float64)
    T = 1e-5 * S + thw + 2.0 ** -24 * np.abs(bias_f)[None, :]
    F = orc.fmax(fy)
    # an output scale that saturates the largest outputs and underflows the smallest
    sy = np.array([[0.8 * np.abs(yref).max() / F]], np.float32)
    ry = (np.array([[np.float32(1.0) / sy[0, 0]]], np.float32) * np.float32(1.0000001)) if with_inv else None
    yq = torch.full((M, N), 0xAA, dtype=torch.uint8, device="cuda")
    amax = torch.full((1,), float("nan"), device="cuda")
    cnt = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    rt.fp8_scaled_gemm_fp8out(dev(a), fa, ga, dev(sa), dev(b), 0, gb, dev(sb), yq, fy, dev(sy),
                              None if ry is None else dev(ry), amax, cnt, bias=dev(bias),
                              flags=rt.POW2_SCALES if pow2 else 0)
    torch.cuda.synchronize()
    q = host(yq)
    lo = np.nextafter((yref - T).astype(np.float32), np.float32(-np.inf))
    hi = np.nextafter((yref + T).astype(np.float32), np.float32(np.inf))
    qlo = orc.quantize(lo, fy, (0, 0), mode=orc.GIVEN, scale=sy, inv_scale=ry)[0]
    qhi = orc.quantize(hi, fy, (0, 0), mode=orc.GIVEN, scale=sy, inv_scale=ry)[0]
    ok = (order(qlo) <= order(q)) & (order(q) <= order(qhi))
    print("fp8out", case, fy, with_inv, "bad", int((~ok).sum()), "of", q.size)
    assert ok.all(), np.argwhere(~ok)[:5]
    # amax of y, before the cast
    am = float(host(amax)[0])
    assert abs(am - np.abs(yref).max()) <= T.max(), (am, np.abs(yref).max())
    # counters between certain and possible
    r = float(ry[0, 0]) if ry is not None else float(np.float32(1.0) / sy[0, 0])
    mag_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)).astype(np.float64))
    mag_hi = np.maximum(np.abs(lo), np.abs(hi)).astype(np.float64)
    edge = 2.0 ** -10 if fy == 0 else 2.0 ** -17
    sat_certain = int((mag_lo * r > F * (1 + 1e-6)).sum())
    sat_possible = int((mag_hi * r > F * (1 - 1e-6)).sum())
    under_certain = int(((mag_lo > 0) & (mag_hi * r < edge * (1 - 1e-6))).sum())
    under_possible = int((mag_lo * r <= edge * (1 + 1e-6)).sum())
    c = host(cnt).tolist()
    assert sat_certain <= c[0] <= sat_possible, (c, sat_certain, sat_possible)
    assert under_certain <= c[1] <= under_possible, (c, under_certain, under_possible)
    if sat_certain == sat_possible:  # no output near the threshold: the count is fixed
        assert c[0] == sat_certain
    assert c[0] > 0, "the chosen scale saturates some outputs"
