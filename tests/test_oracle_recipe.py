"""Pins for the oracle's delayed-scaling recipe variants (history function =
window maximum or latest amax, and a margin m: the scale is derived from
f * 2^m), each against something other than the function itself:

- window maximum with m = 0 reproduces the page's hand-computed sequence
  (golden fixture) bit for bit;
- "latest" is current scaling of the newest amax: it equals the pinned scale
  rule applied to a_t alone, on random sequences;
- a one-entry window makes the two history functions agree;
- the margin multiplies s by exactly 2^m and r by 2^-m (both are correctly
  rounded quotients of a power-of-two multiple), with and without the
  power-of-two round-up;
- an old spike leaves the window exactly h steps after it entered (an
  off-by-one in the ring fails), while "latest" drops it at once;
- NaN propagates; a non-positive a_t counts as zero (eps takes over).
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_window_max_margin0_is_page_sequence(orc):
    d = GOLD["delayed_scaling"]
    hist = np.zeros(d["h"], np.float32)
    head = 0
    for a, es, er, eh in zip(d["amax"], d["expected_scale"], d["expected_inv_scale"], d["expected_head"]):
        head, s, r = orc.history_update_recipe(hist, head, a, 0, orc.HIST_MAX, 0, eps=d["eps"])
        assert (s, r, head) == (np.float32(es), np.float32(er), eh)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("pow2", [False, True])
def test_latest_is_current_scaling(orc, fmt, pow2):
    g = np.random.default_rng(fmt + 2 * pow2)
    hist = np.zeros(8, np.float32)
    head = 0
    for a in np.exp(g.uniform(-20, 12, 40)).astype(np.float32):
        head, s, r = orc.history_update_recipe(hist, head, a, fmt, orc.HIST_LATEST, 0, pow2=pow2)
        sc, rc = orc.compute_scale(np.array([a], np.float32), fmt, pow2=pow2)
        assert s == sc[0] and r == rc[0]


def test_one_entry_window_equals_latest(orc):
    g = np.random.default_rng(3)
    h1 = np.zeros(1, np.float32)
    h2 = np.zeros(5, np.float32)
    k1 = k2 = 0
    for a in np.exp(g.uniform(-5, 5, 30)).astype(np.float32):
        k1, s1, r1 = orc.history_update_recipe(h1, k1, a, 0, orc.HIST_MAX, 0)
        k2, s2, r2 = orc.history_update_recipe(h2, k2, a, 0, orc.HIST_LATEST, 0)
        assert (s1, r1) == (s2, r2)


@pytest.mark.parametrize("fn", [0, 1])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("fmt", [0, 1])
def test_margin_is_an_exact_power_of_two(orc, fn, pow2, fmt):
    g = np.random.default_rng(10 + fn + 2 * pow2 + 4 * fmt)
    seq = np.exp(g.uniform(-10, 10, 24)).astype(np.float32)
    base = []
    hist = np.zeros(6, np.float32)
    head = 0
    for a in seq:
        head, s, r = orc.history_update_recipe(hist, head, a, fmt, fn, 0, pow2=pow2)
        base.append((s, r))
    for m in (1, 3, 16):
        hist = np.zeros(6, np.float32)
        head = 0
        for a, (s0, r0) in zip(seq, base):
            head, s, r = orc.history_update_recipe(hist, head, a, fmt, fn, m, pow2=pow2)
            assert s == np.float32(math.ldexp(float(s0), m))
            assert r == np.float32(math.ldexp(float(r0), -m))


def test_spike_leaves_window_after_h_steps(orc):
    h = 4
    seq = [1.0, 1.0, 100.0] + [1.0] * 8
    hw = np.zeros(h, np.float32)
    hl = np.zeros(h, np.float32)
    kw = kl = 0
    s_max, s_lat = [], []
    for a in seq:
        kw, s, _ = orc.history_update_recipe(hw, kw, a, 0, orc.HIST_MAX, 0)
        s_max.append(s)
        kl, s, _ = orc.history_update_recipe(hl, kl, a, 0, orc.HIST_LATEST, 0)
        s_lat.append(s)
    big, small = np.float32(100.0 / 448.0), np.float32(1.0 / 448.0)
    # the spike enters at step 2 and stays for steps 2..5 (h = 4 entries)
    assert s_max == [small, small] + [big] * h + [small] * (len(seq) - 2 - h)
    assert s_lat == [small, small, big] + [small] * (len(seq) - 3)


def test_nan_and_nonpositive(orc):
    hist = np.zeros(3, np.float32)
    head, s, r = orc.history_update_recipe(hist, 0, float("nan"), 0, orc.HIST_LATEST, 2)
    assert math.isnan(s) and math.isnan(r)
    head, s, r = orc.history_update_recipe(hist, head, -5.0, 0, orc.HIST_LATEST, 0, eps=448.0 * 2 ** -20)
    assert s == np.float32(2 ** -20) and r == np.float32(2 ** 20)
    head, s, r = orc.history_update_recipe(hist, head, 7.0, 0, orc.HIST_MAX, 0)
    assert math.isnan(s)  # the NaN is still in the 3-entry window


def test_rejects_bad_recipe(orc):
    hist = np.zeros(3, np.float32)
    with pytest.raises(ValueError):
        orc.history_update_recipe(hist, 0, 1.0, 0, 2, 0)
    with pytest.raises(ValueError):
        orc.history_update_recipe(hist, 0, 1.0, 0, 0, 17)
