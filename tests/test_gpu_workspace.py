"""Lifetime of the library's per-stream device memory under HIP graph capture.

A prefill step whose GEMM splits its last wave along K (4096 x 4352 x 1024:
272 tiles of 256 x 256 on 256 CUs, the last 16 in 4 K parts, 16 MiB of FP32
parts in the stream's scratch) is captured.  Then a larger GEMM runs eagerly
on the same stream (4096 x 6144 x 1024: 384 tiles, 128 split in 2 parts,
64 MiB), which makes the scratch grow.  The graph captured the old scratch
address, so the library must keep that memory alive: every replay afterwards
must equal the eager step on the same inputs bit for bit and the oracle
within the GEMM tolerance."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import check_gemm, dev, host
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def bf16(seed, shape, scale=1.0):
    g = np.random.default_rng(seed)
    return dev(to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


def test_graph_replay_after_scratch_growth(rt, orc):
    M, N, K = 4096, 4352, 1024
    N2 = 6144
    s = torch.cuda.Stream()
    X = bf16(1, (M, K))
    W = bf16(2, (N, K), 0.02)
    W2 = bf16(3, (N2, K), 0.02)
    with torch.cuda.stream(s):
        Wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sw = torch.empty((1, 1), device="cuda")
        rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, None, Wq)
        W2q = torch.empty((N2, K), dtype=torch.uint8, device="cuda")
        sw2 = torch.empty((1, 1), device="cuda")
        rt.fp8_quantize(W2, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw2, None, W2q)
        Xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sx = torch.empty((1, 1), device="cuda")
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        Y2 = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")

        def step():
            rt.fp8_quantize(X, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sx, None, Xq)
            rt.fp8_scaled_gemm(Xq, rt.E4M3, (0, 0), sx, Wq, rt.E4M3, (0, 0), sw, Y)

        step()  # warm-up: the stream's workspace and a 16 MiB scratch
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    with torch.cuda.stream(s):
        # larger split: the scratch grows past what the graph captured
        rt.fp8_scaled_gemm(Xq, rt.E4M3, (0, 0), sx, W2q, rt.E4M3, (0, 0), sw2, Y2)
        filler = torch.full((64 << 20,), 7, dtype=torch.uint8, device="cuda")   # new allocations
    s.synchronize()
    wq_h, sw_h = host(Wq), host(sw)
    for rep in range(3):
        X.copy_(bf16(10 + rep, (M, K), 1.0 + rep))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        got_q, got_s, got_y = Xq.clone(), sx.clone(), Y.clone()
        with torch.cuda.stream(s):
            step()
        s.synchronize()
        assert torch.equal(got_q, Xq) and torch.equal(got_s.view(torch.int32), sx.view(torch.int32))
        assert torch.equal(got_y.view(torch.int16), Y.view(torch.int16)), "replay %d differs from eager" % rep
        m, n = wl.sample_points(M, N, 100 + rep, n_random=4096, n_rows=2, n_cols=2)
        m = np.concatenate([m, np.full(N, 4095), np.full(N, 3072)])   # rows through the split tiles
        n = np.concatenate([n, np.arange(N), np.arange(N)])
        a, sa = host(got_q), host(got_s)
        yref, S = orc.gemm_points(a, 0, sa, (0, 0), wq_h, 0, sw_h, (0, 0), m, n)
        thw = orc.dot_truncation_bound(a, 0, sa, (0, 0), wq_h, 0, sw_h, (0, 0), m, n)
        ok, st = check_gemm(host(got_y)[m, n], yref, S, True, orc, t_hw=thw)
        print("replay", rep, st)
        assert ok, st
    assert int(filler[12345]) == 7
