"""Full-size parity of the widened rows, in the launch configuration the
benchmark times:

- cast-transpose of the delayed workload's G (8192 x 8192 bf16, E5M2, the
  history-derived per-tensor scale; and per-column DYNAMIC): both code
  copies, scales, amax and counters bit-exact on the whole tensor;
- weight-only FP8 GEMM at the decode shape (16 x 8192 x 8192, per-channel
  E4M3 weight, bf16 bias and output): every output at the GEMM tolerance;
- the ledger's error statistics of the decode weight with the 16 activation
  rows: weight sums within the binary64 summation bound 2 N K 2^-53, max |e|
  exact, output sums within the bound derived from the FP32 summation;
- the FP8-output prefill GEMM (4096 x 29568 x 8192, E4M3 output, output scale
  0.05): on whole rows and columns through whole tiles and through the split
  last wave, plus random points, each code between the oracle's codes of
  y_ref -+ T; the amax of Y is at least the sampled lower bound and agrees
  with the bf16-output GEMM of the same operands.

Codes and scales fed to the GEMMs are the oracle's, which the full-size
quantize tests show equal to the HIP path's."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import check_gemm, dev, host, same_f32
from test_gpu_ledger import bounds, sum_rtol

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
    assert bad.size == 0, "%s: %d codes differ, first at flat index %d" % (what, bad.size, bad[0] if bad.size else -1)


def test_cast_transpose_delayed_g(rt, orc):
    c = wl.C4Delayed()
    g = c.make_g(1)
    M, K = g.shape
    # the benchmark's scale: step 0 current scaling, pushed into the history
    _, _, _, am0, _ = orc.quantize(g, orc.E5M2, (0, 0))
    hist = np.zeros(c.history, np.float32)
    _, s_ref, r_ref = orc.history_update(hist, 0, float(am0.ravel()[0]), orc.E5M2)
    sg = np.array([[s_ref]], np.float32)
    rg = np.array([[r_ref]], np.float32)
    q, qt, _, _, am, cnt = orc.quantize_transpose(g, orc.E5M2, (0, 0), mode=orc.GIVEN, scale=sg, inv_scale=rg)
    G = dev(g)
    Q, QT = u8(M, K), u8(K, M)
    A = f32(1, 1)
    C = torch.zeros(2, dtype=torch.int64, device="cuda")
    rt.fp8_quantize_transpose(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, dev(sg), dev(rg), Q, QT, A, C)
    torch.cuda.synchronize()
    assert_codes(Q, q, "row-major codes")
    assert_codes(QT, qt, "K-major codes")
    assert same_f32(host(A), am) and host(C).tolist() == cnt.astype(np.int64).tolist()
    del q, qt
    # per-column DYNAMIC
    q2, qt2, s2, r2, _, _ = orc.quantize_transpose(g, orc.E5M2, (0, 1))
    S2, R2 = f32(1, K), f32(1, K)
    rt.fp8_quantize_transpose(G, (0, 1), rt.E5M2, rt.DYNAMIC, 1e-12, False, S2, R2, Q, QT)
    torch.cuda.synchronize()
    assert same_f32(host(S2), s2) and same_f32(host(R2), r2)
    assert_codes(Q, q2, "per-column row-major codes")
    assert_codes(QT, qt2, "per-column K-major codes")


def decode_operands(orc):
    c = wl.C2Decode()
    d = c.make()
    wq, sw, _, _, _ = orc.quantize(d["w"], orc.E4M3, (1, 0))
    return c, d, wq, sw


def test_weight_only_decode(rt, orc):
    c, d, wq, sw = decode_operands(orc)
    M, N, K = c.M, c.N, c.K
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_weight_only_gemm(dev(d["a"]), dev(wq), rt.E4M3, (1, 0), dev(sw), y, bias=dev(d["bias"]))
    torch.cuda.synchronize()
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    m, n = mm.ravel(), nn.ravel()
    yref, S = orc.wonly_gemm_points(d["a"], wq, orc.E4M3, sw, (1, 0), m, n, bias=d["bias"])
    ok, st = check_gemm(host(y).ravel(), yref, S, True, orc, bias=orc.bf16_bits_to_f32(d["bias"])[n])
    print("weight-only decode", st, flush=True)
    assert ok, st
    assert st["n_over_rel"] == 0, st


def test_ledger_decode(rt, orc):
    c, d, wq, sw = decode_operands(orc)
    stats = torch.full((7,), float("nan"), dtype=torch.float64, device="cuda")
    rt.fp8_quant_error(dev(d["w"]), dev(wq), rt.E4M3, (1, 0), dev(sw), stats, x=dev(d["a"]))
    torch.cuda.synchronize()
    got = host(stats)
    ref = orc.quant_error(d["w"], wq, orc.E4M3, sw, (1, 0), d["a"])
    print("ledger decode", got, ref, flush=True)
    assert np.allclose(got[:2], ref[:2], rtol=sum_rtol(c.N, c.K), atol=0)
    assert got[2] == ref[2]
    tol = bounds(orc, d["w"], wq, sw, orc.E4M3, (1, 0), d["a"]) + 1e-12 * np.abs(ref[3:])
    assert np.all(np.abs(got[3:] - ref[3:]) <= tol), (got[3:] - ref[3:], tol)


def order(cd):
    cd = np.asarray(cd).astype(np.int64)
    return np.where(cd & 0x80, -(cd & 0x7F), cd & 0x7F)


def test_fp8_output_prefill(rt, orc):
    c = wl.C3Prefill()
    M, N, K = c.M, c.N, c.K
    xq, sx, _, _, _ = orc.quantize(c.make_x(), orc.E4M3, (0, 0))
    w_bits = c.make_w()
    amw = orc.amax(w_bits)
    sw, rw = orc.compute_scale(amw, orc.E4M3)
    wq, _, _, _, _ = orc.quantize(w_bits, orc.E4M3, (0, 0), mode=orc.GIVEN, scale=sw, inv_scale=rw)
    del w_bits
    print("oracle codes done", flush=True)
    Xq, Wq = dev(xq), dev(wq)
    s_x, s_w = dev(np.asarray(sx, np.float32).reshape(1, 1)), dev(np.asarray(sw, np.float32).reshape(1, 1))
    s_y = np.array([[0.05]], np.float32)
    yq = u8(M, N)
    am_y = f32(1, 1)
    cnt_y = torch.zeros(2, dtype=torch.int64, device="cuda")
    rt.fp8_scaled_gemm_fp8out(Xq, rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (0, 0), s_w, yq, rt.E4M3, dev(s_y), None,
                              am_y, cnt_y)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    rt.fp8_scaled_gemm(Xq, rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (0, 0), s_w, yb)
    torch.cuda.synchronize()
    q = host(yq)
    # whole rows and columns through the split last wave (rows 3072-4095,
    # columns 25600-29567) and through whole tiles, plus random points
    rows = np.array([17, 3072, 3583, 4095])
    cols = np.array([5, 25600, 27111, 29567])
    g = np.random.default_rng(8)
    m = np.concatenate([np.repeat(rows, N), np.repeat(np.arange(M), len(cols)), g.integers(0, M, 16384)])
    n = np.concatenate([np.tile(np.arange(N), len(rows)), np.tile(cols, M), g.integers(0, N, 16384)])
    yref, S = orc.gemm_points(xq, orc.E4M3, sx, (0, 0), wq, orc.E4M3, sw, (0, 0), m, n)
    thw = orc.dot_truncation_bound(xq, orc.E4M3, sx, (0, 0), wq, orc.E4M3, sw, (0, 0), m, n)
    T = 1e-5 * S + thw
    lo = np.nextafter((yref - T).astype(np.float32), np.float32(-np.inf))
    hi = np.nextafter((yref + T).astype(np.float32), np.float32(np.inf))
    qlo = orc.quantize(lo.reshape(1, -1), orc.E4M3, (0, 0), mode=orc.GIVEN, scale=s_y)[0].ravel()
    qhi = orc.quantize(hi.reshape(1, -1), orc.E4M3, (0, 0), mode=orc.GIVEN, scale=s_y)[0].ravel()
    qs = q[m, n]
    ok = (order(qlo) <= order(qs)) & (order(qs) <= order(qhi))
    print("fp8out prefill: bad", int((~ok).sum()), "of", ok.size, flush=True)
    assert ok.all(), np.argwhere(~ok)[:5]
    am = float(host(am_y).ravel()[0])
    assert am >= float(np.max(np.abs(yref) - T)), (am, float(np.max(np.abs(yref))))
    # the same operands through the bf16-output GEMM: |y| <= amax, and the
    # largest bf16 output is within one bf16 rounding of amax
    ybm = float(np.abs(orc.bf16_bits_to_f32(host(yb))).max())
    assert abs(am - ybm) <= 2.0 ** -8 * am, (am, ybm)
    cnt = host(cnt_y).tolist()
    assert 0 <= cnt[0] <= M * N and 0 <= cnt[1] <= M * N
