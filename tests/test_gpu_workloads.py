"""Full-size parity of the five workloads, in the call sequence the benchmark
times: every FP8 code, scale, amax, saturation / underflow counter and
history entry of the HIP path is compared bit-exactly with the CPU oracle on
the whole tensor; GEMM outputs are compared with the oracle's binary64 dot
products on a sample of points (whole rows, whole columns and random points,
workloads.sample_points) under the same acceptance rule as the small GEMM
tests.  The GEMM reference is computed from the oracle's own codes and scales,
which the first half of each test shows equal to the GPU's.

Inputs are the seeded synthetic workloads of the workloads module at their
full shapes (the delayed chain runs its first 10 steps, spike included, at
the full 8192 x 8192 shape and all 32 steps at 256 rows)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import check_gemm, dev, host, same_f32

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def f32(*shape):
    return torch.empty(shape, dtype=torch.float32, device="cuda")


def u8(*shape):
    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def assert_codes(q_gpu, q_orc, what):
    qg = host(q_gpu)
    bad = np.flatnonzero(qg.ravel() != q_orc.ravel())
    assert bad.size == 0, "%s: %d codes differ, first at flat index %d (gpu %d, oracle %d)" % (
        what, bad.size, bad[0], qg.ravel()[bad[0]], q_orc.ravel()[bad[0]])


def gemm_sampled(orc, y_gpu, a, fa, sa, ga, b, fb, sb, gb, out_bf16, seed, bias=None):
    M, N = a.shape[0], b.shape[0]
    m, n = wl.sample_points(M, N, seed, n_random=16384, n_rows=4, n_cols=4)
    yref, S = orc.gemm_points(a, fa, sa, ga, b, fb, sb, gb, m, n, bias=bias)
    thw = orc.dot_truncation_bound(a, fa, sa, ga, b, fb, sb, gb, m, n)
    bias_f = None if bias is None else orc.bf16_bits_to_f32(bias)[n]
    ok, st = check_gemm(host(y_gpu)[m, n], yref, S, out_bf16, orc, bias=bias_f, t_hw=thw)
    print("gemm sample", (M, N, a.shape[1]), st, flush=True)
    assert ok, st


def test_tiny_per_tensor(rt, orc):
    c = wl.C1Tiny()
    d = c.make()
    x, w = d["x"], d["w"]
    xq, sx, rx, amx, cnx = orc.quantize(x, orc.E4M3, (0, 0))
    wq, sw, rw, _, _ = orc.quantize(w, orc.E4M3, (1, 0))
    X, W = dev(x), dev(w)
    Xq, Wq = u8(*x.shape), u8(*w.shape)
    s_x, r_x, a_x = f32(1, 1), f32(1, 1), f32(1, 1)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    s_w, r_w = f32(w.shape[0], 1), f32(w.shape[0], 1)
    rt.fp8_quantize(X, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_x, r_x, Xq, a_x, cnt)
    rt.fp8_quantize(W, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_w, r_w, Wq)
    y = f32(c.M_gemm, c.N)
    rt.fp8_scaled_gemm(Xq[:c.M_gemm], rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (1, 0), s_w, y)
    torch.cuda.synchronize()
    assert same_f32(host(a_x), amx) and same_f32(host(s_x), sx) and same_f32(host(r_x), rx)
    assert host(cnt).tolist() == cnx.astype(np.int64).tolist()
    assert same_f32(host(s_w), sw) and same_f32(host(r_w), rw)
    assert_codes(Xq, xq, "X codes")
    assert_codes(Wq, wq, "W codes")
    a = xq[:c.M_gemm]
    yref, S = orc.gemm_full(a, orc.E4M3, sx, (0, 0), wq, orc.E4M3, sw, (1, 0))
    thw = orc.dot_truncation_bound_full(a, orc.E4M3, sx, (0, 0), wq, orc.E4M3, sw, (1, 0))
    ok, st = check_gemm(host(y), yref, S, False, orc, t_hw=thw)
    print("tiny gemm", st, flush=True)
    assert ok, st


def test_decode_per_token_per_channel(rt, orc):
    c = wl.C2Decode()
    d = c.make()
    M, N, K = c.M, c.N, c.K
    aq, sa, ra, _, _ = orc.quantize(d["a"], orc.E4M3, (1, 0))
    wq, sw, rw, _, _ = orc.quantize(d["w"], orc.E4M3, (1, 0))
    A, W, bias = dev(d["a"]), dev(d["w"]), dev(d["bias"])
    Aq, Wq = u8(M, K), u8(N, K)
    s_a, r_a, s_w, r_w = f32(M, 1), f32(M, 1), f32(N, 1), f32(N, 1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_quantize(A, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_a, r_a, Aq)
    rt.fp8_quantize(W, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_w, r_w, Wq)
    rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), s_a, Wq, rt.E4M3, (1, 0), s_w, y, bias=bias)
    torch.cuda.synchronize()
    assert same_f32(host(s_a), sa) and same_f32(host(r_a), ra)
    assert same_f32(host(s_w), sw) and same_f32(host(r_w), rw)
    assert_codes(Aq, aq, "A codes")
    assert_codes(Wq, wq, "W codes")
    # every output of the 16 x 8192 result
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    m, n = mm.ravel(), nn.ravel()
    yref, S = orc.gemm_points(aq, orc.E4M3, sa, (1, 0), wq, orc.E4M3, sw, (1, 0), m, n, bias=d["bias"])
    thw = orc.dot_truncation_bound(aq, orc.E4M3, sa, (1, 0), wq, orc.E4M3, sw, (1, 0), m, n)
    ok, st = check_gemm(host(y).ravel(), yref, S, True, orc, t_hw=thw,
                        bias=orc.bf16_bits_to_f32(d["bias"])[n])
    print("decode gemm", st, flush=True)
    assert ok, st


def test_prefill_per_tensor(rt, orc):
    c = wl.C3Prefill()
    M, N, K = c.M, c.N, c.K
    x_bits = c.make_x()
    w_bits = c.make_w()
    # oracle: dynamic X; static W scale from W's own amax, then GIVEN-mode cast
    xq, sx, rx, amx, cnx = orc.quantize(x_bits, orc.E4M3, (0, 0))
    amw = orc.amax(w_bits)
    sw, rw = orc.compute_scale(amw, orc.E4M3)
    wq, _, _, amw2, cnw = orc.quantize(w_bits, orc.E4M3, (0, 0), mode=orc.GIVEN, scale=sw, inv_scale=rw)
    print("oracle done", flush=True)
    X, W = dev(x_bits), dev(w_bits)
    del w_bits
    a_w, s_w, r_w, am_w = f32(1, 1), f32(1, 1), f32(1, 1), f32(1, 1)
    cnt_w = torch.zeros(2, dtype=torch.int64, device="cuda")
    Wq = u8(N, K)
    rt.fp8_amax(W, (0, 0), a_w)
    rt.fp8_compute_scale(a_w, rt.E4M3, 1e-12, False, s_w, r_w)
    rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.GIVEN, 1e-12, False, s_w, r_w, Wq, am_w, cnt_w)
    del W
    Xq = u8(M, K)
    s_x, r_x, am_x = f32(1, 1), f32(1, 1), f32(1, 1)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_quantize(X, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_x, r_x, Xq, am_x, cnt)
    rt.fp8_scaled_gemm(Xq, rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (0, 0), s_w, y)
    torch.cuda.synchronize()
    assert same_f32(host(a_w), amw) and same_f32(host(am_w), amw2)
    assert same_f32(host(s_w), sw) and same_f32(host(r_w), rw)
    assert host(cnt_w).tolist() == cnw.astype(np.int64).tolist()
    assert same_f32(host(am_x), amx) and same_f32(host(s_x), sx) and same_f32(host(r_x), rx)
    assert host(cnt).tolist() == cnx.astype(np.int64).tolist()
    assert_codes(Xq, xq, "X codes")
    assert_codes(Wq, wq, "W codes")
    del Xq, Wq
    gemm_sampled(orc, y, xq, orc.E4M3, sx, (0, 0), wq, orc.E4M3, sw, (0, 0), True, 3)


def delayed_chain(rt, orc, c, steps, w_gemm_step=None):
    """Runs the first `steps` steps of the delayed E5M2 chain on both sides:
    step 0 current scaling (cold start), then GIVEN with the scale of the
    history; every step pushes its observed amax.  Returns the last step's
    oracle codes and scale."""
    fmt = orc.E5M2
    hist_o = np.zeros(c.history, np.float32)
    head_o = 0
    hist = torch.zeros(c.history, dtype=torch.float32, device="cuda")
    head = torch.zeros(1, dtype=torch.int32, device="cuda")
    s_g, r_g, am = f32(1, 1), f32(1, 1), f32(1, 1)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    Gq = u8(c.M, c.K)
    s_o = r_o = None
    out = None
    for t in range(steps):
        g_bits = c.make_g(t)
        G = dev(g_bits)
        if t == 0:
            q_o, s0, r0, a_o, cn_o = orc.quantize(g_bits, fmt, (0, 0))
            rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.DYNAMIC, 1e-12, False, s_g, r_g, Gq, am, cnt)
            s_used = s0
        else:
            q_o, _, _, a_o, cn_o = orc.quantize(g_bits, fmt, (0, 0), mode=orc.GIVEN,
                                                scale=np.array([[s_o]], np.float32),
                                                inv_scale=np.array([[r_o]], np.float32))
            rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, s_g, r_g, Gq, am, cnt)
            s_used = np.array([[s_o]], np.float32)
        torch.cuda.synchronize()
        assert same_f32(host(am).ravel(), a_o.ravel()), t
        assert host(cnt).tolist() == cn_o.astype(np.int64).tolist(), (t, host(cnt), cn_o)
        assert_codes(Gq, q_o, "G codes step %d" % t)
        if t == steps - 1:
            out = (q_o, s_used, Gq)
        head_o, s_o, r_o = orc.history_update(hist_o, head_o, float(a_o.ravel()[0]), fmt)
        rt.fp8_amax_history_update(hist, head, am, rt.E5M2, 1e-12, False, s_g, r_g)
        torch.cuda.synchronize()
        assert int(host(head)[0]) == head_o
        assert same_f32(host(hist), hist_o), t
        assert same_f32(host(s_g).ravel(), [s_o]) and same_f32(host(r_g).ravel(), [r_o]), t
        print("delayed step", t, "amax", float(a_o.ravel()[0]), "sat/under", cn_o.tolist(), flush=True)
        del G, g_bits
    return out


def test_delayed_chain_full_rows(rt, orc):
    c = wl.C4Delayed()
    _, spikes = c.sigmas()
    steps = int(spikes.max()) + 2  # through the spike and the step after it
    q_o, s_g, Gq = delayed_chain(rt, orc, c, steps)
    # the backward GEMM of the last step: G (E5M2) x W (E4M3, per tensor) -> fp32
    w_bits = c.make_w()
    wq, sw, rw, _, _ = orc.quantize(w_bits, orc.E4M3, (0, 0))
    W = dev(w_bits)
    Wq = u8(c.N, c.K)
    s_w, r_w = f32(1, 1), f32(1, 1)
    rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_w, r_w, Wq)
    S_g = dev(s_g)
    y = f32(c.M, c.N)
    rt.fp8_scaled_gemm(Gq, rt.E5M2, (0, 0), S_g, Wq, rt.E4M3, (0, 0), s_w, y)
    torch.cuda.synchronize()
    assert same_f32(host(s_w), sw)
    assert_codes(Wq, wq, "W codes")
    gemm_sampled(orc, y, q_o, orc.E5M2, s_g, (0, 0), wq, orc.E4M3, sw, (0, 0), False, 4)


def test_delayed_chain_32_steps(rt, orc):
    c = wl.C4Delayed(M=256)
    delayed_chain(rt, orc, c, c.steps)


@pytest.mark.parametrize("variant", ["block128", "mx32"])
def test_block_scaled(rt, orc, variant):
    c = wl.C5Block()
    M, N, K = c.M, c.N, c.K
    a_bits = c.make_a()
    w_bits = c.make_w()
    if variant == "block128":
        ga, gb, pow2, flags = (1, 128), (128, 128), False, 0
    else:
        ga, gb, pow2, flags = (1, 32), (1, 32), True, rt.POW2_SCALES
    aq, sa, _, _, _ = orc.quantize(a_bits, orc.E4M3, ga, pow2=pow2)
    wq, sw, _, _, _ = orc.quantize(w_bits, orc.E4M3, gb, pow2=pow2)
    print("oracle done", flush=True)
    A, W = dev(a_bits), dev(w_bits)
    del a_bits, w_bits
    Aq, Wq = u8(M, K), u8(N, K)
    s_a, s_w = f32(*sa.shape), f32(*sw.shape)
    rt.fp8_quantize(A, ga, rt.E4M3, rt.DYNAMIC, 1e-12, pow2, s_a, None, Aq)
    rt.fp8_quantize(W, gb, rt.E4M3, rt.DYNAMIC, 1e-12, pow2, s_w, None, Wq)
    del A, W
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_scaled_gemm(Aq, rt.E4M3, ga, s_a, Wq, rt.E4M3, gb, s_w, y, flags=flags)
    torch.cuda.synchronize()
    assert same_f32(host(s_a), sa) and same_f32(host(s_w), sw)
    assert_codes(Aq, aq, "A codes")
    assert_codes(Wq, wq, "W codes")
    del Aq, Wq
    gemm_sampled(orc, y, aq, orc.E4M3, sa, ga, wq, orc.E4M3, sw, gb, True, 5)
