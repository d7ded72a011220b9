"""Parity of the HIP quantization-error statistics (fp8_quant_error) and the
granularity ledger (fp8_granularity_ledger) with the CPU oracle.

The weight sums (sum e^2, sum w^2) are binary64 sums of N K nonnegative
terms, added in different orders on the two sides: each within (n - 1) 2^-53
of the exact sum, so they agree within 2 N K 2^-53 relative; max |e| is
bit-exact.  The output sums use FP32 dot products of exact products (the
binary32 error split exactly into three bf16 parts, bf16 activations, on the
matrix cores), so each d and y_ref is within gamma * sum_k |x e| (resp.
|x w|) of the exact value, plus 2^-24 |x e| per term for rounding e to
binary32; gamma (dot_gamma) follows the kernel's summation: a product passes
through at most 32 additions inside one matrix-core instruction, the chain of
its wave's instructions and the 4 wave partials, each addition losing at most
one ulp.  The test propagates those bounds to each sum of squares.  Codes and
scales come from the oracle's quantization; the ledger's counters and scale
counts must equal the oracle's exactly."""
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
    assert torch.cuda.is_available()
    return rt


def bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make(seed, N, K, M, dtype):
    g = np.random.default_rng(seed)
    wf = (g.standard_normal((N, K)) * 0.02 * np.exp(g.uniform(-2, 2, (N, 1)))).astype(np.float32)
    wf[g.integers(0, N), g.integers(0, K)] = 3.0  # an outlier
    w = to_bf16_bits(wf) if dtype == "bf16" else wf
    x = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32)) if M else None
    return w, x


def wdouble(w):
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


def dot_gamma(K):
    """Relative bound of one kernel dot product: 128-deep K steps, 4 waves
    each taking a contiguous share, 4 eight-element runs per step and at most
    3 instructions per run (the three parts of the split), so a chain of at
    most 12 ceil(steps / 4) instructions per wave; at most 32 additions inside
    one instruction; 4 wave partials added in order; one ulp (2^-23) each."""
    steps = -(-K // 128)
    chain = 12 * -(-steps // 4)
    return (32 + chain + 4) * 2.0 ** -23


def bounds(orc, w, q, s, fmt, gran, x):
    """Per-sum tolerances for stats[3..6] from the FP32 summation bound."""
    K = w.shape[1]
    wh = orc.dequantize(q, fmt, s, gran).astype(np.float64)
    wd = wdouble(w)
    e = wh - wd
    xd = np.abs(bf16_to_f64(x))
    gamma = dot_gamma(K) * 1.01
    # the FP32 error e32 = fl32(w_hat - w) adds at most 2^-24 |e| per term
    Bd = (gamma + 2.0 ** -24) * (xd @ np.abs(e).T)
    By = gamma * (xd @ np.abs(wd).T)
    xs = bf16_to_f64(x)
    d = xs @ e.T
    yr = xs @ wd.T
    yq = yr + d
    Bq = Bd + By
    tol = [((2 * np.abs(d) + Bd) * Bd).sum(), ((2 * np.abs(yr) + By) * By).sum(),
           ((2 * np.abs(yq) + Bq) * Bq).sum(), (np.abs(yr) * Bq + np.abs(yq) * By + By * Bq).sum()]
    return np.array(tol)


def sum_rtol(N, K):
    """Two binary64 sums of N K nonnegative terms in different orders."""
    return 2.0 * N * K * 2.0 ** -53


def run_quant_error(rt, w, q, s, fmt, gran, x):
    st = torch.full((7,), float("nan"), dtype=torch.float64, device="cuda")
    rt.fp8_quant_error(dev(w), dev(q), fmt, gran, dev(s), st, x=None if x is None else dev(x))
    torch.cuda.synchronize()
    return host(st)


CASES = [  # (N, K, M, fmt, gran, dtype)
    (200, 1040, 5, 0, (1, 0), "bf16"),      # K tail inside the ninth step, a ragged last 16-row tile
    (64, 512, 0, 1, (0, 0), "f32"),         # no inputs: weight sums only
    (128, 2048, 20, 0, (1, 128), "bf16"),   # two activation tiles (16 + 4 rows)
    (256, 1024, 8, 0, (128, 128), "f32"),   # 2-D blocks
    (96, 768, 3, 0, (1, 32), "bf16"),       # 1x32 groups
    (40, 384, 40, 1, (1, 0), "f32"),        # three activation tiles, fp32 weight split too, 3 K steps for 4 waves
    (70000, 128, 2, 0, (1, 0), "bf16"),     # 4375 row tiles: more than the 4096 blocks of the grid
]


@pytest.mark.parametrize("case", CASES)
def test_quant_error_matches_oracle(rt, orc, case):
    N, K, M, fmt, gran, dtype = case
    w, x = make(case_seed(case), N, K, M, dtype)
    q, s, _, _, _ = orc.quantize(w, fmt, gran)
    ref = orc.quant_error(w, q, fmt, s, gran, x)
    got = run_quant_error(rt, w, q, s, fmt, gran, x)
    print("quant_error", case, got, ref)
    assert np.allclose(got[:2], ref[:2], rtol=sum_rtol(N, K), atol=0)
    assert got[2] == ref[2]
    if x is None:
        assert not got[3:].any()
    else:
        tol = bounds(orc, w, q, s, fmt, gran, x) + 1e-12 * np.abs(ref[3:])
        print("error / bound", np.abs(got[3:] - ref[3:]) / tol)
        assert np.all(np.abs(got[3:] - ref[3:]) <= tol), (got[3:] - ref[3:], tol)


def test_quant_error_nan(rt, orc):
    w, x = make(4, 32, 256, 2, "f32")
    q, s, _, _, _ = orc.quantize(w, 0, (1, 0))
    w = w.copy()
    w[7, 9] = np.nan
    got = run_quant_error(rt, w, q, s, 0, (1, 0), x)
    assert np.isnan(got[0]) and np.isnan(got[2]) and np.isnan(got[3])


@pytest.mark.parametrize("inf", [np.inf, -np.inf])
def test_quant_error_inf_weight(rt, orc, inf):
    """An infinite weight under finite codes: e = -+Inf; the sums become Inf
    or NaN exactly where the oracle's do."""
    w, x = make(6, 48, 256, 3, "f32")
    q, s, _, _, _ = orc.quantize(w, 0, (1, 0))
    w = w.copy()
    w[7, 9] = inf
    got = run_quant_error(rt, w, q, s, 0, (1, 0), x)
    ref = orc.quant_error(w, q, 0, s, (1, 0), x)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(np.isinf(got), np.isinf(ref)), (got, ref)
    fin = np.isfinite(ref)
    assert np.array_equal(got[~fin & ~np.isnan(ref)], ref[~fin & ~np.isnan(ref)])


SPECS = [((0, 0), 0), ((1, 0), 0), ((1, 128), 0), ((128, 128), 0), ((1, 32), 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ledger_rows(rt, orc, dtype):
    N, K, M, fmt = 256, 1024, 8, 0
    w, x = make(17, N, K, M, dtype)
    rows = rt.fp8_granularity_ledger(dev(w), fmt, SPECS, x=dev(x))
    assert len(rows) == len(SPECS)
    for (gran, pow2), r in zip(SPECS, rows):
        q, s, _, _, cnt = orc.quantize(w, fmt, gran, pow2=bool(pow2))
        st = orc.quant_error(w, q, fmt, s, gran, x)
        assert r["gran"] == gran and r["pow2_round_up"] == pow2
        assert r["qparam_count"] == s.size and r["qparam_bytes"] == 4 * s.size
        assert r["quantized_weight_bytes"] == N * K and r["total_state_bytes"] == N * K + 4 * s.size
        assert (r["saturated"], r["underflowed"]) == (int(cnt[0]), int(cnt[1]))
        assert np.isclose(r["weight_mse"], st[0] / (N * K), rtol=sum_rtol(N, K), atol=0)
        assert r["weight_max_abs_err"] == st[2]
        tol = bounds(orc, w, q, s, fmt, gran, x) + 1e-12 * np.abs(st[3:])
        assert abs(r["output_mse"] - st[3] / (M * N)) <= tol[0] / (M * N)
        cos_ref = st[6] / max(np.sqrt(st[4]) * np.sqrt(st[5]), 1e-8)
        dcos = tol[3] / np.sqrt(st[4] * st[5]) + abs(cos_ref) * (tol[1] / st[4] + tol[2] / st[5])
        assert abs(r["output_cosine"] - cos_ref) <= dcos + 1e-12, (r["output_cosine"], cos_ref, dcos)
        print("ledger", gran, pow2, r["qparam_bytes"], r["weight_mse"], r["output_mse"], r["output_cosine"])
    # with rows of very different spread, one scale per row beats one per tensor
    assert rows[1]["weight_mse"] < rows[0]["weight_mse"]


def test_ledger_stops_at_a_rejected_spec(rt, orc):
    w, x = make(23, 64, 512, 0, "bf16")
    specs = (rt.LedgerSpec * 2)(rt.LedgerSpec(rt.Gran(1, 0), 0), rt.LedgerSpec(rt.Gran(1, 24), 0))
    rows = (rt.LedgerRow * 2)()
    W = dev(w)
    stv = rt.lib().fp8_granularity_ledger(W.data_ptr(), rt.BF16, 64, 512, 512, None, 0, 0, 0, 1e-12, specs, 2,
                                          rows, None)
    torch.cuda.synchronize()
    assert stv == rt.EALIGN
    q, s, _, _, _ = orc.quantize(w, 0, (1, 0))
    assert rows[0].qparam_count == s.size and np.isnan(rows[0].output_cosine)
