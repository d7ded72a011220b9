"""Parity of the fragment-ordered weight image (fp8_pack_weights16) and of the
decode GEMMs that read it (FP8RT_B_PACKED16).

- The HIP pack against the oracle's pack_weights16, every byte: ragged N (the
  last 16-row group zero-filled over a poisoned buffer), strided rows, one and
  many 128-byte K steps.
- fp8_scaled_gemm on the packed image at decode shapes: bit-identical to the
  row-major call (the matrix cores receive the same bytes in the same order)
  and within the GEMM tolerance of the oracle on every element.
- fp8_weight_only_gemm on the packed image: bit-identical to the row-major
  call and within tolerance of the oracle, including a last 32-column
  workgroup whose second 16-row tile lies past N, and M above 16.
- The decode workload (16 x 8192 x 8192, per-token / per-channel E4M3 and
  the bf16-activation weight-only layer): both GEMMs bit-identical to their
  row-major results on the whole output.

Codes and scales come from the oracle's quantizer; the packed image fed to the
GEMMs is the HIP pack, which the first test shows equal to the oracle's."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import check_gemm, dev, host
from workloads import case_seed, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def bits(y):
    """Raw bit patterns of a host array (NaNs compared by payload)."""
    y = np.ascontiguousarray(y)
    return y.view(np.uint32) if y.dtype == np.float32 else y.view(np.uint16)


def pack(rt, Q):
    N, K = Q.shape
    out = torch.full((rt.packed16_bytes(N, K),), 0xAB, dtype=torch.uint8, device="cuda")
    return rt.fp8_pack_weights16(Q, out=out)


PACK_CASES = [  # (N, K, pad)
    (16, 128, 0),      # one tile
    (17, 256, 0),      # a second group with one live row
    (200, 1024, 16),   # strided rows, ragged N
    (1, 384, 0),       # a single row
    (64, 4096, 32),    # many steps
]


@pytest.mark.parametrize("case", PACK_CASES)
def test_pack_matches_oracle(rt, orc, case):
    N, K, pad = case
    g = np.random.default_rng(N * 7 + K)
    full = g.integers(0, 256, (N, K + pad), dtype=np.uint8)
    q = np.ascontiguousarray(full[:, :K])
    Q = dev(full)[:, :K]
    p = pack(rt, Q)
    torch.cuda.synchronize()
    assert (p.N, p.K) == (N, K)
    got = host(p.data)
    ref = orc.pack_weights16(q)
    assert got.shape == ref.shape
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "%d bytes differ, first at %d" % (bad.size, bad[0])


def gemm_operands(orc, seed, M, N, K, fa, ga, gb):
    g = np.random.default_rng(seed)
    xa = (g.standard_normal((M, K)) * np.exp(g.uniform(-1, 1, (M, 1)))).astype(np.float32)
    xb = (g.standard_normal((N, K)) * 0.02 * np.exp(g.uniform(-1, 1, (N, 1)))).astype(np.float32)
    a, sa, _, _, _ = orc.quantize(xa, fa, ga)
    b, sb, _, _, _ = orc.quantize(xb, 0, gb)
    return a, sa, b, sb


GEMM_CASES = [  # (M, N, K, fa, ga, gb, out, bias)
    (1, 64, 128, 0, (0, 0), (0, 0), "f32", None),
    (5, 200, 1024, 1, (1, 0), (1, 0), "bf16", "bf16"),
    (16, 300, 2048, 0, (1, 0), (1, 0), "bf16", "f32"),
    (16, 8, 256, 0, (0, 0), (1, 0), "f32", "f32"),      # N below one group
    (3, 1000, 4096, 0, (1, 0), (0, 0), "bf16", None),
    (16, 512, 384, 1, (0, 0), (1, 0), "f32", None),     # 3 K steps for 16 waves
]


@pytest.mark.parametrize("case", GEMM_CASES)
def test_scaled_gemm_packed(rt, orc, case):
    M, N, K, fa, ga, gb, out, bt = case
    a, sa, b, sb = gemm_operands(orc, case_seed(case), M, N, K, fa, ga, gb)
    bias = None
    if bt is not None:
        bv = (np.random.default_rng(3).standard_normal(N) * 0.1).astype(np.float32)
        bias = to_bf16_bits(bv) if bt == "bf16" else bv
    A, B, SA, SB = dev(a), dev(b), dev(sa), dev(sb)
    Bias = None if bias is None else dev(bias)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y0 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    y1 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    rt.fp8_scaled_gemm(A, fa, ga, SA, B, 0, gb, SB, y0, bias=Bias)
    P = pack(rt, B)
    rt.fp8_scaled_gemm(A, fa, ga, SA, P, 0, gb, SB, y1, bias=Bias)
    torch.cuda.synchronize()
    h0, h1 = host(y0), host(y1)
    assert np.array_equal(bits(h0), bits(h1)), "packed and row-major results differ"
    yref, S = orc.gemm_full(a, fa, sa, ga, b, 0, sb, gb, bias=bias)
    thw = orc.dot_truncation_bound_full(a, fa, sa, ga, b, 0, sb, gb)
    bias_f = None
    if bias is not None:
        bias_f = orc.bf16_bits_to_f32(bias) if bt == "bf16" else bias
        bias_f = np.broadcast_to(np.asarray(bias_f, np.float64)[None, :], (M, N))
    ok, st = check_gemm(h1, yref, S, out == "bf16", orc, t_hw=thw, bias=bias_f)
    print("packed gemm", case, st)
    assert ok, st


WONLY_CASES = [  # (M, N, K, fw, gw, out, bias)
    (16, 8192, 1024, 0, (1, 0), "bf16", "bf16"),
    (5, 40, 1024, 0, (0, 0), "f32", None),          # 3 groups: the last workgroup's second tile is past N
    (20, 50, 2048, 1, (1, 128), "bf16", None),      # M > 16, K groups of 128, E5M2
    (16, 264, 4096, 0, (1, 512), "f32", "bf16"),    # K groups of 512
    (24, 384, 1024, 0, (128, 128), "f32", None),    # 2-D blocks
    (16, 16, 128, 0, (1, 0), "bf16", None),         # one group, one step
    (3, 96, 256, 0, (1, 0), "f32", None),           # 2 steps: most waves idle
]


@pytest.mark.parametrize("case", WONLY_CASES)
def test_weight_only_packed(rt, orc, case):
    M, N, K, fw, gw, out, bt = case
    g = np.random.default_rng(case_seed(case))
    x = to_bf16_bits((g.standard_normal((M, K)) * np.exp(g.uniform(-2, 2, (M, 1)))).astype(np.float32))
    wf = (g.standard_normal((N, K)) * 0.02 * np.exp(g.uniform(-2, 2, (N, 1)))).astype(np.float32)
    w, sw, _, _, _ = orc.quantize(wf, fw, gw)
    bias = None
    if bt is not None:
        bv = (g.standard_normal(N) * 0.1).astype(np.float32)
        bias = to_bf16_bits(bv) if bt == "bf16" else bv
    X, W, SW = dev(x), dev(w), dev(sw)
    Bias = None if bias is None else dev(bias)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y0 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    y1 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    rt.fp8_weight_only_gemm(X, W, fw, gw, SW, y0, bias=Bias)
    P = pack(rt, W)
    rt.fp8_weight_only_gemm(X, P, fw, gw, SW, y1, bias=Bias)
    torch.cuda.synchronize()
    h0, h1 = host(y0), host(y1)
    assert np.array_equal(bits(h0), bits(h1)), "packed and row-major results differ"
    yref, S = orc.wonly_gemm_full(x, w, fw, sw, gw, bias=bias)
    bias_f = None
    if bias is not None:
        bias_f = orc.bf16_bits_to_f32(bias) if bt == "bf16" else bias
        bias_f = np.broadcast_to(np.asarray(bias_f, np.float64)[None, :], (M, N))
    ok, st = check_gemm(h1, yref, S, out == "bf16", orc, bias=bias_f)
    print("packed wonly", case, st)
    assert ok, st
    assert st["n_over_rel"] == 0, st


@pytest.mark.slow
def test_decode_workload_packed(rt, orc):
    c = wl.C2Decode()
    d = c.make()
    M, N, K = c.M, c.N, c.K
    aq, sa, _, _, _ = orc.quantize(d["a"], orc.E4M3, (1, 0))
    wq, sw, _, _, _ = orc.quantize(d["w"], orc.E4M3, (1, 0))
    A, Aq, Wq, SA, SW, Bias = dev(d["a"]), dev(aq), dev(wq), dev(sa), dev(sw), dev(d["bias"])
    P = pack(rt, Wq)
    y = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), SA, Wq, rt.E4M3, (1, 0), SW, y[0], bias=Bias)
    rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), SA, P, rt.E4M3, (1, 0), SW, y[1], bias=Bias)
    rt.fp8_weight_only_gemm(A, Wq, rt.E4M3, (1, 0), SW, y[2], bias=Bias)
    rt.fp8_weight_only_gemm(A, P, rt.E4M3, (1, 0), SW, y[3], bias=Bias)
    torch.cuda.synchronize()
    assert np.array_equal(host(P.data), orc.pack_weights16(wq))
    h = [host(t) for t in y]
    assert np.array_equal(h[0], h[1]), "decode GEMM: packed and row-major differ"
    assert np.array_equal(h[2], h[3]), "weight-only decode: packed and row-major differ"


@pytest.mark.parametrize("grans", [((1, 128), (128, 128)), ((1, 0), (128, 128)), ((1, 128), (1, 0))],
                         ids=["tokgroup-block", "token-block", "tokgroup-channel"])
def test_decode_workload_block_scaled(rt, orc, grans):
    """The decode workload's operands under 1x128 token-group and 128x128
    weight-block scales (each 128-deep step's partial promoted by its two
    scales in the decode kernel): the weight image bit-identical to the
    row-major call on the whole output, and every row of 640 sampled output
    columns within the acceptance rule of the binary64 reference."""
    ga, gb = grans
    c = wl.C2Decode()
    d = c.make()
    M, N, K = c.M, c.N, c.K
    aq, sa, _, _, _ = orc.quantize(d["a"], orc.E4M3, ga)
    wq, sw, _, _, _ = orc.quantize(d["w"], orc.E4M3, gb)
    Aq, Wq, SA, SW, Bias = dev(aq), dev(wq), dev(sa), dev(sw), dev(d["bias"])
    P = pack(rt, Wq)
    y = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    rt.fp8_scaled_gemm(Aq, rt.E4M3, ga, SA, Wq, rt.E4M3, gb, SW, y[0], bias=Bias)
    rt.fp8_scaled_gemm(Aq, rt.E4M3, ga, SA, P, rt.E4M3, gb, SW, y[1], bias=Bias)
    torch.cuda.synchronize()
    h = [host(t) for t in y]
    assert np.array_equal(h[0], h[1]), "block-scaled decode GEMM: packed and row-major differ"
    g = np.random.default_rng(case_seed("decode-block", ga, gb))
    cols = np.unique(np.concatenate([np.arange(128), np.arange(N - 128, N), g.integers(0, N, 384)]))
    m = np.repeat(np.arange(M), len(cols))
    n = np.tile(cols, M)
    yref, S = orc.gemm_points(aq, orc.E4M3, sa, ga, wq, orc.E4M3, sw, gb, m, n, bias=d["bias"])
    thw = orc.dot_truncation_bound(aq, orc.E4M3, sa, ga, wq, orc.E4M3, sw, gb, m, n)
    ok, st = check_gemm(h[0][m, n], yref, S, True, orc, bias=orc.bf16_bits_to_f32(d["bias"])[n], t_hw=thw)
    print(grans, st)
    assert ok, st
