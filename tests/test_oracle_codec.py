"""Pins for the oracle's FP8 codec (decode, encode, bf16 rounding).

Each pin comes from outside the oracle: the pages' format facts (golden
fixture), exhaustive closed-form properties, brute force over all codes, and
torch's own float8 / bfloat16 casts used as a black-box library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))
FMTS = {"e4m3": 0, "e5m2": 1}
TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def test_format_constants_match_pages(orc):
    for name, f in FMTS.items():
        g = GOLD["formats"][name]
        assert g["sign_bits"] + g["exponent_bits"] + g["mantissa_bits"] == 8
        assert orc.fmax(f) == g["max_finite"]
        finite = [orc.decode(c, f) for c in range(256)]
        finite = [v for v in finite if math.isfinite(v)]
        assert max(finite) == g["max_finite"]
        assert min(finite) == -g["max_finite"]
        # 1.0 is the code with exponent field == bias and zero mantissa
        assert orc.decode(g["bias"] << g["mantissa_bits"], f) == 1.0
        # smallest normal 2^(1-bias), smallest subnormal 2^(1-bias-m)
        assert orc.decode(1 << g["mantissa_bits"], f) == 2.0 ** (1 - g["bias"])
        assert orc.decode(1, f) == 2.0 ** (1 - g["bias"] - g["mantissa_bits"])


def test_decode_table_special_codes(orc):
    assert orc.decode(0x7E, 0) == 448.0
    assert math.isnan(orc.decode(0x7F, 0)) and math.isnan(orc.decode(0xFF, 0))
    assert orc.decode(0x7B, 1) == 57344.0
    assert orc.decode(0x7C, 1) == math.inf and orc.decode(0xFC, 1) == -math.inf
    for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert math.isnan(orc.decode(c, 1))
    # E4M3 (fn) has no infinities and exactly two NaN codes
    assert sum(math.isnan(orc.decode(c, 0)) for c in range(256)) == 2
    assert not any(math.isinf(orc.decode(c, 0)) for c in range(256))
    assert math.copysign(1.0, orc.decode(0x80, 0)) == -1.0


@pytest.mark.parametrize("f", [0, 1])
def test_decode_table_exhaustive_vs_library(orc, f):
    lib = torch.arange(256, dtype=torch.uint8).view(TORCH[f]).to(torch.float64).numpy()
    mine = orc.decode_table(f)
    both_nan = np.isnan(lib) & np.isnan(mine)
    assert np.all(both_nan | (lib == mine))
    # sign bit symmetric, positive codes strictly increasing over the finite range
    pos = mine[:0x7F if f == 0 else 0x7C]
    assert np.all(np.diff(pos) > 0)
    assert np.all((mine[0x80:] == -mine[:0x80]) | np.isnan(mine[:0x80]))


@pytest.mark.parametrize("f", [0, 1])
def test_roundtrip_every_finite_code(orc, f):
    for c in range(256):
        v = orc.decode(c, f)
        if math.isfinite(v):
            assert orc.encode(np.float32(v), f) == c, hex(c)


@pytest.mark.parametrize("f", [0, 1])
def test_encode_matches_bruteforce_nearest(orc, f):
    g = np.random.default_rng(5)
    fm = orc.fmax(f)
    vals = list((g.standard_normal(4000) * np.exp(g.uniform(-14, 12, 4000))).astype(np.float32))
    table = sorted({abs(orc.decode(c, f)) for c in range(256) if math.isfinite(orc.decode(c, f))})
    mids = [(a + b) / 2 for a, b in zip(table[:-1], table[1:])]
    vals += [np.float32(m) for m in mids] + [np.float32(-m) for m in mids]
    vals += [np.nextafter(np.float32(m), np.float32(0)) for m in mids]
    vals += [np.nextafter(np.float32(m), np.float32(1e9)) for m in mids]
    vals += [np.float32(fm * 1.01), np.float32(-fm * 3), np.float32(np.inf), np.float32(-np.inf)]
    for v in vals:
        assert orc.encode(v, f) == orc.encode_bruteforce(v, f), (v, f)


@pytest.mark.parametrize("f", [0, 1])
def test_encode_matches_library_cast_after_clamp(orc, f):
    """torch's CPU float8 cast (round to nearest even) on clamped inputs."""
    g = np.random.default_rng(11)
    fm = orc.fmax(f)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-20, 14, 20000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0625, 1.1875, 2 ** -10, 1.5 * 2 ** -9, fm,
                                     -fm, 1e30, -1e30], np.float32)])
    lib = torch.from_numpy(x).clamp(-fm, fm).to(TORCH[f]).view(torch.uint8).numpy()
    mine = np.array([orc.encode(v, f) for v in x], np.uint8)
    assert np.array_equal(lib, mine)


def test_encode_special_values(orc):
    assert orc.encode(np.float32(np.nan), 0) == 0x7F
    assert orc.encode(np.float32(np.nan), 1) == 0x7F
    assert orc.encode(np.float32(-0.0), 0) == 0x80
    assert orc.encode(np.float32(np.inf), 0) == 0x7E
    assert orc.encode(np.float32(-np.inf), 1) == 0xFB
    assert orc.encode(np.float32(470.0), 0) == 0x7E      # saturates, never NaN
    assert orc.encode(np.float32(61440.0), 1) == 0x7B    # saturates, never Inf
    assert orc.encode(np.float32(-2.0 ** -11), 0) == 0x80  # negative underflow keeps sign


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_teaching_grid_equivalence_in_normal_range(orc, name):
    """The pages' teaching grid, step = 2^(floor(log2|v|) - m), round half even,
    equals the encoder on the normal range (it has no subnormal floor)."""
    f = FMTS[name]
    lo, hi = GOLD["teaching_grid"]["normal_range"][name]
    mb = GOLD["formats"][name]["mantissa_bits"]
    g = np.random.default_rng(17)
    mag = np.exp(g.uniform(np.log(lo), np.log(hi), 20000)).astype(np.float32)
    v = mag * np.where(g.integers(0, 2, mag.size) == 0, -1, 1).astype(np.float32)
    step = np.exp2(np.floor(np.log2(np.abs(v.astype(np.float64)))) - mb)
    grid = np.round(v / step) * step
    grid = np.clip(grid, -hi, hi)
    mine = np.array([orc.decode(orc.encode(t, f), f) for t in v])
    assert np.array_equal(grid, mine)


def test_bf16_rounding_matches_library(orc):
    g = np.random.default_rng(3)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-90, 88, 20000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 3.3e38, 1e-40, -1e-42],
                                    np.float32)])
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([orc.lib().orc_round_bf16_from_f32(float(v)) for v in x], np.uint16)
    assert np.array_equal(lib, mine)
