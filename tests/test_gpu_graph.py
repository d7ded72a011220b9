"""The hot path under HIP graph capture: one prefill step (per-tensor DYNAMIC
quantize of X, scaled GEMM with a split last wave) and one decode step
(per-token quantize of A, GEMM on the fragment-ordered weight image) are
captured once and replayed on new inputs.  Every replay must equal, bit for
bit, the eager calls on the same inputs (codes, scales, amax, counters,
output), with the program's own eager work and synchronizations between
replays; the eager prefill codes are also checked against the oracle.

The library allocates its per-stream workspace and scratch on first use, so
each test warms its entry points up eagerly on the stream it then captures."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def same(a, b):
    a, b = host(a), host(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    elif a.dtype == np.uint16 or a.dtype == np.int16:
        a, b = a.view(np.uint16), b.view(np.uint16)
    return np.array_equal(a, b)


def bf16_input(seed, shape, scale=1.0):
    g = np.random.default_rng(seed)
    return dev(to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


def test_prefill_step_graph(rt, orc):
    M, N, K = 1024, 1536, 1024  # 24 output tiles: one ragged wave, split along K
    s = torch.cuda.Stream()
    X = bf16_input(1, (M, K))
    Wb = bf16_input(2, (N, K), 0.02)
    with torch.cuda.stream(s):
        Wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sw = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        rw = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        rt.fp8_quantize(Wb, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, rw, Wq)
        Xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sx = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        rx = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        am = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step():
            rt.fp8_quantize(X, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sx, rx, Xq, amax_out=am,
                            sat_underflow=cnt)
            rt.fp8_scaled_gemm(Xq, rt.E4M3, (0, 0), sx, Wq, rt.E4M3, (0, 0), sw, Y)

        step()  # first use on this stream: workspace and scratch
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    outs = (Xq, sx, rx, am, cnt, Y)
    for rep in range(4):
        X.copy_(bf16_input(10 + rep, (M, K), 1.0 + rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        with torch.cuda.stream(s):
            step()  # eager, same inputs
        s.synchronize()
        for name, a, b in zip(("codes", "scale", "inv_scale", "amax", "counts", "Y"), got, outs):
            assert same(a, b), "replay %d: %s differs from the eager call" % (rep, name)
        if rep == 0:
            q, sref, _, _, _ = orc.quantize(host(X), orc.E4M3, (0, 0))
            assert np.array_equal(host(Xq), q) and same(sx, torch.from_numpy(np.asarray(sref, np.float32)).reshape(1, 1))


def test_decode_step_graph_packed(rt, orc):
    M, N, K = 16, 2048, 4096
    s = torch.cuda.Stream()
    A = bf16_input(3, (M, K))
    Wb = bf16_input(4, (N, K), 0.02)
    bias = bf16_input(5, (N,), 0.1)
    with torch.cuda.stream(s):
        Wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sw = torch.empty((N, 1), dtype=torch.float32, device="cuda")
        rt.fp8_quantize(Wb, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, None, Wq)
        P = rt.fp8_pack_weights16(Wq)
        Aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sa = torch.empty((M, 1), dtype=torch.float32, device="cuda")
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        Yw = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step():
            rt.fp8_quantize(A, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sa, None, Aq)
            rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), sa, P, rt.E4M3, (1, 0), sw, Y, bias=bias)
            rt.fp8_weight_only_gemm(A, P, rt.E4M3, (1, 0), sw, Yw, bias=bias)

        step()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        A.copy_(bf16_input(20 + rep, (M, K), 2.0 ** rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (Aq, sa, Y, Yw)]
        with torch.cuda.stream(s):
            step()
        s.synchronize()
        for name, a, b in zip(("codes", "scales", "Y", "Y weight-only"), got, (Aq, sa, Y, Yw)):
            assert same(a, b), "replay %d: %s differs from the eager call" % (rep, name)
