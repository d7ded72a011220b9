"""Pins for the oracle's amax, scale, quantize, dequantize and delayed-scaling
history.  Expected values come from the pages' worked cases (golden fixture),
hand-computed exact sequences, brute force with numpy, and exact rational
arithmetic (fractions) for the correctly rounded quotients."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def f32_of_fraction(q: Fraction) -> np.float32:
    """Correctly rounded binary32 of an exact rational (via round-half-even on
    the exact value; checked against the neighbours)."""
    cand = np.float32(float(q))  # float() of a Fraction is correctly rounded to binary64
    best = cand
    for c in (np.nextafter(cand, np.float32(-np.inf)), cand, np.nextafter(cand, np.float32(np.inf))):
        if abs(Fraction(float(c)) - q) < abs(Fraction(float(best)) - q):
            best = c
    ties = [c for c in (np.nextafter(best, np.float32(-np.inf)), np.nextafter(best, np.float32(np.inf)))
            if abs(Fraction(float(c)) - q) == abs(Fraction(float(best)) - q)]
    if ties:  # exact tie: pick the even significand
        for c in [best] + ties:
            if int(np.array(c, np.float32).view(np.uint32)) % 2 == 0:
                return c
    return best


def test_amax_bruteforce(orc):
    g = np.random.default_rng(2)
    x = (g.standard_normal((37, 160)) * 3).astype(np.float32)
    for gran in [(0, 0), (1, 0), (1, 32), (16, 48), (37, 160), (5, 7)]:
        a = orc.amax(x, gran)
        er = x.shape[0] if gran[0] <= 0 else gran[0]
        ec = x.shape[1] if gran[1] <= 0 else gran[1]
        for i in range(a.shape[0]):
            for j in range(a.shape[1]):
                blk = x[i * er:(i + 1) * er, j * ec:(j + 1) * ec]
                assert a[i, j] == np.abs(blk).max()


def test_amax_nan_propagates_and_bf16_widening(orc):
    x = np.ones((4, 16), np.float32)
    x[2, 5] = np.nan
    a = orc.amax(x, (1, 0))
    assert math.isnan(a[2, 0]) and a[0, 0] == 1.0
    # bf16 bits widen exactly: 0x4300 = 128.0, 0xC3E0 = -448.0
    h = np.full((2, 16), 0x4300, np.uint16)
    h[1, 3] = 0xC3E0
    assert orc.amax(h, (1, 0)).ravel().tolist() == [128.0, 448.0]


def test_granularity_shapes_and_tail_group(orc):
    for case in GOLD["granularity_shapes"]["cases"]:
        x = np.arange(np.prod(case["shape"]), dtype=np.float32).reshape(case["shape"]) - 3
        assert list(orc.amax(x, tuple(case["gran"])).shape) == case["scale_shape"]
    # the 5-column, group-3 case keeps the 2-column tail group
    x = np.array([[1, 2, 3, 40, 5], [6, 7, 8, 9, -100]], np.float32)
    assert orc.amax(x, (1, 3)).tolist() == [[3.0, 40.0], [8.0, 100.0]]


def test_scale_contract_from_pages(orc):
    sc = GOLD["scale_contract"]
    for f in (0, 1):
        s, r = orc.compute_scale(orc.amax(np.array([sc["positive_for"]], np.float32)), f)
        assert s[0, 0] > 0 and np.isfinite(s[0, 0])
        s, r = orc.compute_scale(orc.amax(np.zeros((1, sc["finite_for_zeros"]), np.float32)), f)
        assert s[0, 0] > 0 and np.isfinite(s[0, 0]) and np.isfinite(r[0, 0])


def test_scale_is_correctly_rounded_quotient(orc):
    g = np.random.default_rng(4)
    a = np.exp(g.uniform(-40, 40, 3000)).astype(np.float32)
    for f, F in ((0, 448), (1, 57344)):
        s, r = orc.compute_scale(a, f)
        for ai, si, ri in zip(a, s, r):
            ac = max(ai, np.float32(1e-12))     # default eps clamp
            assert si == f32_of_fraction(Fraction(float(ac)) / F)
            assert ri == f32_of_fraction(F / Fraction(float(ac)))


def test_scale_eps_clamp_and_nonfinite(orc):
    s, r = orc.compute_scale(np.array([0.0, 1e-30, np.inf, np.nan], np.float32), 0, eps=1e-12)
    e = np.float32(1e-12)
    assert s[0] == f32_of_fraction(Fraction(float(e)) / 448) == s[1]
    assert math.isnan(s[2]) and math.isnan(r[2]) and math.isnan(s[3]) and math.isnan(r[3])


def test_pow2_round_up_is_exact_ceil_log2(orc):
    """s = 2^ceil(log2(a/F)) for the exact quotient, over random amax values and
    every binary32 value of three binades (exhaustive) per format."""
    g = np.random.default_rng(6)
    a = np.exp(g.uniform(-30, 30, 3000)).astype(np.float32)
    for f, F in ((0, 448), (1, 57344)):
        s, r = orc.compute_scale(a, f, pow2=True)
        for ai, si, ri in zip(a, s, r):
            q = Fraction(float(max(ai, np.float32(1e-12)))) / F
            k = math.ceil(math.log2(q))
            while Fraction(2) ** k < q:
                k += 1
            while Fraction(2) ** (k - 1) >= q:
                k -= 1
            assert si == np.float32(2.0 ** k) and ri == np.float32(2.0 ** -k)
    # exhaustive binades just above F * 2^j: the rounded quotient never crosses 2^j downward
    for f, F in ((0, 448.0), (1, 57344.0)):
        for j in (-3, 0, 5):
            lo = np.float32(F * 2.0 ** j)
            bits = np.arange(lo.view(np.uint32), lo.view(np.uint32) + (1 << 16), dtype=np.uint32)
            av = bits.view(np.float32)
            s, _ = orc.compute_scale(av, f, pow2=True)
            expect = np.where(av == lo, np.float32(2.0 ** j), np.float32(2.0 ** (j + 1)))
            assert np.array_equal(s, expect)


def test_outlier_case_from_page(orc):
    oc = GOLD["outlier_case"]
    x = np.full((8, 16), oc["body_value"], np.float32)
    x[3, 7] = oc["outlier"]
    q, s, r, am, cnt = orc.quantize(x, 0, (0, 0))
    assert s[0, 0] == f32_of_fraction(Fraction(int(oc["expected_scale_num"]), int(oc["expected_scale_den"])))
    assert am[0, 0] == 400.0
    assert orc.decode(q[3, 7], 0) == 448.0              # the outlier lands on the format edge
    body = orc.decode(q[0, 0], 0)
    assert body == 1.125                                # body x 448/400 = 1.12 -> nearest code 1.125
    assert abs(body * s[0, 0] - 1.0) < 0.01             # dequantized body stays near 1
    assert cnt.tolist() == [0, 0]


def test_dequant_example_from_page(orc):
    ex = GOLD["dequant_example"]
    for f in (0, 1):
        codes = np.array([[orc.encode(np.float32(v), f) for v in ex["fp8_values"]] +
                          [0] * 13], np.uint8)
        assert [orc.decode(c, f) for c in codes[0, :3]] == ex["fp8_values"]
        y = orc.dequantize(codes, f, np.array([[ex["scale"]]], np.float32))
        for got, want in zip(y[0, :3], ex["expected"]):
            assert abs(float(got) - want) <= 2 * abs(np.spacing(np.float32(want)))


def test_quantize_counts_and_given_mode(orc):
    # GIVEN scale that is too small: values beyond F_max * s saturate
    x = np.array([[0.5, 1.0, 2.0, -3.0, 1e-9, -1e-9, 0.0, -0.0] * 2], np.float32)
    s = np.array([[1.0 / 448.0]], np.float32)
    q, _, r, am, cnt = orc.quantize(x, 0, (0, 0), mode=orc.GIVEN, scale=s)
    assert r[0, 0] == np.float32(1.0 / np.float64(s[0, 0]))
    assert am[0, 0] == 3.0
    sat = sum(abs(np.float32(v * np.float64(r[0, 0]))) > 448 for v in x[0])
    assert cnt[0] == sat and sat in (4, 6)  # 2.0, -3.0 (x2), and 1.0 only if fl32(1/s) > 448
    assert cnt[1] == 4                 # +-1e-9 underflow to +-0 (x2)
    assert q[0, 4] == 0x00 and q[0, 5] == 0x80 and q[0, 7] == 0x80
    # explicit inverse scale overrides fl32(1/s)
    q2, _, _, _, _ = orc.quantize(x, 0, (0, 0), mode=orc.GIVEN, scale=s,
                                  inv_scale=np.array([[1.0]], np.float32))
    assert orc.decode(q2[0, 2], 0) == 2.0


def test_quantize_dynamic_matches_library_pipeline(orc):
    """Dynamic per-row quantize equals: amax -> r -> x*r in binary32 -> clamp ->
    torch float8 cast (a black-box library cast)."""
    g = np.random.default_rng(8)
    x = (g.standard_normal((12, 96)) * np.exp(g.uniform(-5, 5, (12, 1)))).astype(np.float32)
    for f, F, dt in ((0, 448.0, torch.float8_e4m3fn), (1, 57344.0, torch.float8_e5m2)):
        q, s, r, am, _ = orc.quantize(x, f, (1, 0))
        v = torch.from_numpy(x) * torch.from_numpy(r)   # binary32 multiply
        lib = v.clamp(-F, F).to(dt).view(torch.uint8).numpy()
        assert np.array_equal(q, lib)


def test_history_hand_computed_sequence(orc):
    d = GOLD["delayed_scaling"]
    hist = np.zeros(d["h"], np.float32)
    head = 0
    for a, es, er, eh in zip(d["amax"], d["expected_scale"], d["expected_inv_scale"],
                             d["expected_head"]):
        head, s, r = orc.history_update(hist, head, a, 0, eps=d["eps"])
        assert (s, r, head) == (np.float32(es), np.float32(er), eh)


def test_history_nan_and_pow2(orc):
    hist = np.zeros(4, np.float32)
    head, s, r = orc.history_update(hist, 0, 300.0, 0, pow2=True)
    assert s == 1.0 and r == 1.0            # 300/448 rounds up to 2^0
    head, s, r = orc.history_update(hist, head, float("nan"), 0)
    assert math.isnan(s) and math.isnan(r)
