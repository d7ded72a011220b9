"""Parity of the HIP weight-only FP8 GEMM (fp8_weight_only_gemm: FP8 weights
with tensor / channel / K-group / 2-D block scales, bf16 activations) with
the CPU oracle, every element, at the GEMM tolerance: fp32 output within
1e-5 S (+ 2^-24 |bias|), bf16 output within 1 bf16 ulp of RNE(y_ref) or the
cancellation fallback.  Shapes cover the decode shape, ragged M / N / K,
M above 16 (several workgroup rows), fewer K steps than waves, strided
operands, both weight formats and both output types; the identity weight is
checked bit for bit and a NaN activation row must propagate."""
import numpy as np
import pytest
import torch

from gpu_helpers import check_gemm, dev, host
from workloads import case_seed, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def n_groups(n, g):
    return 1 if (g <= 0 or g >= n) else -(-n // g)


def operands(orc, seed, M, N, K, fw, gw):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * np.exp(g.uniform(-2, 2, (M, 1)))).astype(np.float32)
    wf = (g.standard_normal((N, K)) * 0.02 * np.exp(g.uniform(-2, 2, (N, 1)))).astype(np.float32)
    w, sw, _, _, _ = orc.quantize(wf, fw, gw)
    return to_bf16_bits(x), w, sw


def run(rt, x, w, fw, gw, sw, out, bias=None, pad_x=0, pad_w=0, pad_y=0):
    M, K = x.shape
    N = w.shape[0]
    if pad_x:
        xs = np.zeros((M, K + pad_x), np.uint16)
        xs[:, :K] = x
        X = dev(xs)[:, :K]
    else:
        X = dev(x)
    if pad_w:
        ws = np.zeros((N, K + pad_w), np.uint8)
        ws[:, :K] = w
        Wt = dev(ws)[:, :K]
    else:
        Wt = dev(w)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    Y = torch.full((M, N + pad_y), float("nan"), dtype=dt, device="cuda")[:, :N]
    rt.fp8_weight_only_gemm(X, Wt, fw, gw, dev(sw), Y, bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    return host(Y)


CASES = [  # (M, N, K, fw, gw, out, bias)
    ((16, 8192, 1024), 0, (1, 0), "bf16", "bf16"),     # decode rows, per-channel, bias
    ((5, 300, 1040), 0, (0, 0), "f32", "f32"),         # ragged M, N and K tail, per-tensor
    ((40, 264, 2048), 1, (1, 128), "bf16", None),      # M > 16, K groups of 128, E5M2
    ((16, 256, 4096), 0, (1, 512), "f32", "bf16"),     # K groups of 512
    ((24, 384, 1024), 0, (128, 128), "f32", None),     # 2-D 128 x 128 weight blocks
    ((3, 96, 256), 0, (1, 0), "f32", None),            # 2 K steps: 14 of 16 waves idle
    ((16, 512, 8192), 1, (1, 0), "bf16", "f32"),       # long K
]


@pytest.mark.parametrize("case", CASES)
def test_wonly_within_tolerance(rt, orc, case):
    (M, N, K), fw, gw, out, bt = case
    x, w, sw = operands(orc, case_seed(case), M, N, K, fw, gw)
    bias = None
    if bt is not None:
        b = (np.random.default_rng(5).standard_normal(N) * 0.1).astype(np.float32)
        bias = to_bf16_bits(b) if bt == "bf16" else b
    y = run(rt, x, w, fw, gw, sw, out, bias)
    yref, S = orc.wonly_gemm_full(x, w, fw, sw, gw, bias=bias)
    bias_f = None
    if bias is not None:
        bias_f = orc.bf16_bits_to_f32(bias) if bt == "bf16" else bias
        bias_f = np.broadcast_to(np.asarray(bias_f, np.float64)[None, :], (M, N))
    ok, st = check_gemm(y, yref, S, out == "bf16", orc, bias=bias_f)
    print("wonly", case, st)
    assert ok, st
    assert st["n_over_rel"] == 0, st


def test_wonly_strided(rt, orc):
    M, N, K = 16, 160, 640
    x, w, sw = operands(orc, 21, M, N, K, 0, (1, 128))
    y = run(rt, x, w, 0, (1, 128), sw, "f32", pad_x=24, pad_w=48, pad_y=8)
    yref, S = orc.wonly_gemm_full(x, w, 0, sw, (1, 128))
    ok, st = check_gemm(y, yref, S, False, orc)
    assert ok, st


@pytest.mark.parametrize("fw", [0, 1])
def test_wonly_identity_weight_exact(rt, orc, fw):
    M, K = 16, 512
    g = np.random.default_rng(9)
    x = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    one = 0x38 if fw == 0 else 0x3C
    w = np.where(np.eye(K, dtype=bool), one, 0).astype(np.uint8)
    y = run(rt, x, w, fw, (0, 0), np.ones((1, 1), np.float32), "bf16")
    assert np.array_equal(y, x)


def test_wonly_nan_row_propagates(rt, orc):
    M, N, K = 8, 64, 256
    x, w, sw = operands(orc, 31, M, N, K, 0, (1, 0))
    x[3, 17] = 0x7FC0  # bf16 NaN
    y = run(rt, x, w, 0, (1, 0), sw, "f32")
    yref, S = orc.wonly_gemm_full(x, w, 0, sw, (1, 0))
    assert np.isnan(y[3]).all() and np.isnan(yref[3]).all()
    rows = [i for i in range(M) if i != 3]
    ok, st = check_gemm(y[rows], yref[rows], S[rows], False, orc)
    assert ok, st
