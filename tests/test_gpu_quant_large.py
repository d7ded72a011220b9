"""Parity of per-tensor DYNAMIC quantization on bf16 tensors of 8.4M-33.5M
elements (the two-pass path at the activation sizes of the prefill workload):
codes, scale, inverse scale, amax and counters bit-exact with the oracle, with
a ragged last segment, E4M3 and E5M2, the power-of-two round-up, optional
outputs absent, NaN / Inf / all-zero inputs, and back-to-back calls that
reuse the per-stream partial arrays."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, same_f32
from workloads import case_seed, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def make(seed, rows, cols, special=None):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((rows, cols)) * np.exp(g.uniform(-3, 3, (rows, 1)))).astype(np.float32)
    x[g.integers(0, rows), g.integers(0, cols)] = 700.0  # an outlier that sets the scale
    if special == "nan":
        x[g.integers(0, rows), g.integers(0, cols)] = np.nan
    elif special == "inf":
        x[g.integers(0, rows), g.integers(0, cols)] = -np.inf
    elif special == "zero":
        x[:] = 0.0
    return to_bf16_bits(x)


CASES = [  # (rows, cols, fmt, pow2, counts, inv, special)
    (2000, 8192, 0, False, True, True, None),    # ragged last stripe
    (4096, 8192, 1, True, False, False, None),   # the full capacity on 256 CUs
    (1200, 8192, 0, False, True, True, "nan"),
    (1100, 8192, 1, False, True, True, "inf"),
    (1030, 8192, 0, False, True, True, "zero"),
]


@pytest.mark.parametrize("case", CASES)
def test_large_per_tensor_bit_exact(rt, orc, case):
    rows, cols, fmt, pow2, counts, inv, special = case
    x = make(case_seed(case), rows, cols, special)
    q, s, r, am, cnt = orc.quantize(x, fmt, (0, 0), pow2=pow2)
    X = dev(x)
    Q = torch.full((rows, cols), 0xAA, dtype=torch.uint8, device="cuda")
    S = torch.full((1, 1), float("nan"), device="cuda")
    R = torch.full((1, 1), float("nan"), device="cuda") if inv else None
    A = torch.full((1, 1), float("nan"), device="cuda")
    C = torch.full((2,), -1, dtype=torch.int64, device="cuda") if counts else None
    rt.fp8_quantize(X, (0, 0), fmt, rt.DYNAMIC, 1e-12, pow2, S, R, Q, A, C)
    torch.cuda.synchronize()
    qg = host(Q)
    bad = np.flatnonzero(qg.ravel() != q.ravel())
    assert bad.size == 0, (bad.size, bad[:5])
    assert same_f32(host(S), s) and same_f32(host(A), am)
    if inv:
        assert same_f32(host(R), r)
    if counts:
        assert host(C).tolist() == cnt.astype(np.int64).tolist()


def test_large_repeated_calls(rt, orc):
    """Back-to-back calls on the same stream reuse the partial arrays: the
    second call must not see the first call's partials."""
    a = make(1, 2048, 8192)
    # |a| / 4: a different amax, so stale partials would change the scale
    b = to_bf16_bits(((a & np.uint16(0x7FFF)).astype(np.uint32) << 16).view(np.float32) * np.float32(0.25))
    outs = []
    for x in (a, b, a):
        Q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        S = torch.empty((1, 1), device="cuda")
        R = torch.empty((1, 1), device="cuda")
        C = torch.zeros(2, dtype=torch.int64, device="cuda")
        rt.fp8_quantize(dev(x), (0, 0), 0, rt.DYNAMIC, 1e-12, False, S, R, Q, None, C)
        outs.append((Q, S, R, C))
    torch.cuda.synchronize()
    for x, (Q, S, R, C) in zip((a, b, a), outs):
        q, s, r, _, cnt = orc.quantize(x, 0, (0, 0))
        assert np.array_equal(host(Q), q) and same_f32(host(S), s) and same_f32(host(R), r)
        assert host(C).tolist() == cnt.astype(np.int64).tolist()
