"""Race check: every cross-thread combine in the library is exact (integer
max of |x| bit patterns, integer sums of counts, a fixed FP32 summation
order per kernel), so repeating a call on the same inputs must reproduce
every output bit for bit.  Each entry point runs three times, with other
work between the calls, on shapes that use several hundred workgroups."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from workloads import case_seed, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    return rt


def bits(t):
    a = host(t)
    return a.view(np.uint8).copy()


def repeat3(fn, outs):
    got = []
    junk = torch.empty(1 << 24, device="cuda")
    for _ in range(3):
        for o in outs:  # poison the outputs first
            o.fill_(float("nan") if o.dtype.is_floating_point else 0x5A)
        fn()
        junk.fill_(1.0)  # other work between the calls
        torch.cuda.synchronize()
        got.append([bits(o) for o in outs])
    return got


def assert_same(got):
    for rep in got[1:]:
        for a, b in zip(got[0], rep):
            assert np.array_equal(a, b)


def bf16(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return dev(to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


@pytest.mark.parametrize("gran", [(0, 0), (1, 0), (1, 128), (128, 128), (1, 32)])
@pytest.mark.parametrize("mode", ["dynamic", "given"])
def test_quantize_repeats_bit_for_bit(rt, gran, mode):
    X = bf16((2048, 4096), case_seed("det-q", gran, mode))
    q = torch.empty((2048, 4096), dtype=torch.uint8, device="cuda")
    gs = rt.scale_shape((2048, 4096), gran)
    s = torch.empty(gs, device="cuda")
    r = torch.empty(gs, device="cuda")
    am = torch.empty(gs, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    if mode == "given":
        rt.fp8_quantize(X, gran, rt.E4M3, rt.DYNAMIC, 1e-12, False, s, r, q)
        fn = lambda: rt.fp8_quantize(X, gran, rt.E4M3, rt.GIVEN, 1e-12, False, s, r, q, am, cnt)
        outs = [q, am, cnt]
    else:
        fn = lambda: rt.fp8_quantize(X, gran, rt.E4M3, rt.DYNAMIC, 1e-12, gran == (1, 32), s, r, q, am, cnt)
        outs = [q, s, r, am, cnt]
    assert_same(repeat3(fn, outs))


GEMMS = [  # M, N, K, ga, gb, flags, out
    (4096, 4352, 1024, (0, 0), (0, 0), 0, torch.bfloat16),      # large kernel, split last wave
    (1024, 2048, 2048, (1, 0), (1, 0), 0, torch.float32),       # large kernel, per-row scales
    (1024, 1024, 2048, (1, 128), (128, 128), 0, torch.bfloat16),  # K-blocked kernel
    (512, 768, 1024, (1, 32), (1, 32), 1, torch.bfloat16),      # 1x32 power-of-two scales
    (96, 1000, 1040, (0, 0), (1, 0), 0, torch.float32),         # general kernel (K not a multiple of 256)
    (96, 1000, 1024, (0, 0), (1, 0), 0, torch.float32),         # large kernel, every tile split along K
    (16, 8192, 4096, (1, 0), (1, 0), 0, torch.bfloat16),        # decode kernel
]


@pytest.mark.parametrize("case", GEMMS, ids=lambda c: "%dx%dx%d" % c[:3])
def test_gemm_repeats_bit_for_bit(rt, case):
    M, N, K, ga, gb, flags, out = case
    pow2 = flags != 0
    A, W = bf16((M, K), case_seed("det-a", case[:3])), bf16((N, K), case_seed("det-w", case[:3]), 0.02)
    Aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    Wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa, sw = torch.empty(rt.scale_shape((M, K), ga), device="cuda"), torch.empty(rt.scale_shape((N, K), gb), device="cuda")
    rt.fp8_quantize(A, ga, rt.E4M3, rt.DYNAMIC, 1e-12, pow2, sa, None, Aq)
    rt.fp8_quantize(W, gb, rt.E4M3, rt.DYNAMIC, 1e-12, pow2, sw, None, Wq)
    y = torch.empty((M, N), dtype=out, device="cuda")
    fn = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, ga, sa, Wq, rt.E4M3, gb, sw, y, flags=rt.POW2_SCALES if pow2 else 0)
    assert_same(repeat3(fn, [y]))


def test_fp8_output_gemm_and_weight_only_repeat_bit_for_bit(rt):
    M, N, K = 1024, 2048, 2048
    A, W = bf16((M, K), 5), bf16((N, K), 6, 0.02)
    Aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    Wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa, sw = torch.empty((1, 1), device="cuda"), torch.empty((N, 1), device="cuda")
    rt.fp8_quantize(A, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sa, None, Aq)
    rt.fp8_quantize(W, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, None, Wq)
    yq = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sy = torch.full((1, 1), 0.01, device="cuda")
    amy = torch.empty((1, 1), device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    fn = lambda: rt.fp8_scaled_gemm_fp8out(Aq, rt.E4M3, (0, 0), sa, Wq, rt.E4M3, (1, 0), sw, yq, rt.E4M3, sy, None,
                                           amy, cnt)
    assert_same(repeat3(fn, [yq, amy, cnt]))
    X = A[:16].contiguous()
    yw = torch.empty((16, N), dtype=torch.bfloat16, device="cuda")
    assert_same(repeat3(lambda: rt.fp8_weight_only_gemm(X, Wq, rt.E4M3, (1, 0), sw, yw), [yw]))
    Xt = torch.empty((K, M), dtype=torch.uint8, device="cuda")
    sc, rc = torch.empty((1, K), device="cuda"), torch.empty((1, K), device="cuda")
    ct = lambda: rt.fp8_quantize_transpose(A, (0, 1), rt.E5M2, rt.DYNAMIC, 1e-12, False, sc, rc, Aq, Xt)
    assert_same(repeat3(ct, [Aq, Xt, sc, rc]))
