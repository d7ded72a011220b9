"""fp8_scaled_gemm_noalloc, the GEMM entry point that allocates nothing (its
scratch is the library's fixed 16 MiB device array), against fp8_scaled_gemm
through the C ABI.  Each case runs two calls in a row on the allocation-free
entry point, the second with a smaller input, so the second reads an array
that still holds the first call's contents:
  - 1x32 power-of-two scales (repacked exponents in the array) and 1x128 /
    128x128 block scales (transposed A scales in the array): bit-identical to
    fp8_scaled_gemm;
  - a split last wave whose FP32 parts (32 MiB at 2 parts) do not fit: run
    unsplit, so only the FP32 summation order differs; within the GEMM
    tolerance of the oracle, like fp8_scaled_gemm's own result;
  - a shape whose exponent table needs more than 16 MiB is refused with
    FP8RT_ESCRATCH before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import check_gemm, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def operands(orc, seed, M, N, K, ga, gb, pow2):
    g = np.random.default_rng(seed)
    xa = g.standard_normal((M, K)).astype(np.float32)
    xb = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    a, sa, _, _, _ = orc.quantize(xa, orc.E4M3, ga, pow2=pow2)
    b, sb, _, _, _ = orc.quantize(xb, orc.E4M3, gb, pow2=pow2)
    return a, sa, b, sb


def both(rt, a, sa, ga, b, sb, gb, flags, out=torch.bfloat16):
    M, N = a.shape[0], b.shape[0]
    A, SA, B, SB = dev(a), dev(sa), dev(b), dev(sb)
    y0 = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    y1 = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    rt.fp8_scaled_gemm(A, rt.E4M3, ga, SA, B, rt.E4M3, gb, SB, y0, flags=flags)
    rt.fp8_scaled_gemm_noalloc(A, rt.E4M3, ga, SA, B, rt.E4M3, gb, SB, y1, flags=flags)
    torch.cuda.synchronize()
    return host(y0), host(y1)


@pytest.mark.parametrize("case", [
    # 4096 x 4096: one whole wave of tiles, no split; the smaller shapes:
    # one or two tiles, each split in 2 K parts on both paths (the parts
    # fit the fixed array)
    ("mx32", [(4096, 4096, 512), (256, 384, 512)], (1, 32), (1, 32), True),
    ("kblock", [(4096, 4096, 512), (256, 256, 512)], (1, 128), (128, 128), False),
], ids=lambda c: c[0])
def test_noalloc_bit_identical(rt, orc, case):
    name, shapes, ga, gb, pow2 = case
    flags = rt.POW2_SCALES if pow2 else 0
    for i, (M, N, K) in enumerate(shapes):            # the second call is smaller
        a, sa, b, sb = operands(orc, wl.case_seed("noalloc", name, i), M, N, K, ga, gb, pow2)
        y0, y1 = both(rt, a, sa, ga, b, sb, gb, flags)
        assert np.array_equal(y0, y1), (name, M, N, K)
        m, n = wl.sample_points(M, N, i, n_random=2048, n_rows=2, n_cols=2)
        yref, S = orc.gemm_points(a, orc.E4M3, sa, ga, b, orc.E4M3, sb, gb, m, n)
        thw = orc.dot_truncation_bound(a, orc.E4M3, sa, ga, b, orc.E4M3, sb, gb, m, n)
        ok, st = check_gemm(y1[m, n], yref, S, True, orc, t_hw=thw)
        assert ok, (name, M, N, K, st)


def test_noalloc_unsplit_last_wave(rt, orc):
    """4096 x 6144 x 1024: 384 tiles, 128 in a last wave that fp8_scaled_gemm
    splits in 2 K parts (32 MiB of FP32 parts); the fixed array holds 16 MiB,
    so the allocation-free call runs those tiles whole.  Then a smaller split
    shape (4096 x 4352: 16 tiles x 4 parts = 16 MiB) that fits: identical."""
    for M, N, K, identical in [(4096, 6144, 1024, False), (4096, 4352, 1024, True)]:
        a, sa, b, sb = operands(orc, wl.case_seed("noalloc-split", N), M, N, K, (0, 0), (0, 0), False)
        y0, y1 = both(rt, a, sa, (0, 0), b, sb, (0, 0), 0, out=torch.float32)
        if identical:
            assert np.array_equal(y0, y1)
        m, n = wl.sample_points(M, N, 5, n_random=4096, n_rows=1, n_cols=1)
        m = np.concatenate([m, np.full(N, M - 1)])    # a row through the last wave's tiles
        n = np.concatenate([n, np.arange(N)])
        yref, S = orc.gemm_points(a, orc.E4M3, sa, (0, 0), b, orc.E4M3, sb, (0, 0), m, n)
        thw = orc.dot_truncation_bound(a, orc.E4M3, sa, (0, 0), b, orc.E4M3, sb, (0, 0), m, n)
        for y in (y0, y1):
            ok, st = check_gemm(y[m, n], yref, S, False, orc, t_hw=thw)
            assert ok, (M, N, K, st)


def test_noalloc_refuses_oversized_scratch(rt):
    """1x32 exponents of a 16384 x N x 8192 GEMM take (ceil(M/256) + ceil(N/256))
    * 64 * 1024 bytes: exactly 16 MiB at N = 49152, more at N = 49408, which is
    refused with FP8RT_ESCRATCH before anything is enqueued."""
    M, K = 16384, 8192
    for N, expect in [(49408, rt.ESCRATCH)]:
        A = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        B = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sa = torch.ones((M, K // 32), device="cuda")
        sb = torch.ones((N, K // 32), device="cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        L = rt.lib()
        st = L.fp8_scaled_gemm_noalloc(rt._ptr(A), rt.E4M3, K, rt.Gran(1, 32), rt._ptr(sa), rt._ptr(B),
                                       rt.E4M3, K, rt.Gran(1, 32), rt._ptr(sb), M, N, K, None, rt.F32,
                                       rt._ptr(y), rt.BF16, N, rt.POW2_SCALES, None)
        assert st == expect
        del A, B, sa, sb, y
        torch.cuda.empty_cache()
