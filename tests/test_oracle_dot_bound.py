"""Pins of the GEMM tolerance term T_hw (oracle.dot_truncation_bound) against
an independent emulation of the model it bounds (tests/dot_model.py): within
each 8-product group of consecutive K, products aligned to the group's
largest exponent sum E_g and truncated toward zero to 2^(E_g - 13).

- hand cases whose emulated value and bound are worked out here by hand:
  the 2^13 / 2^14 boundary, a group of subnormal codes (E_g taken at the
  smallest normal exponent), mixed signs, K tails, scale-block edges;
- the bound holds for every element of random operands of both format
  pairs and all scale granularities, and is reached within a small factor
  on operands built to lose almost a unit per product;
- the vectorised emulation agrees with a scalar, product-by-product
  emulation in exact rationals."""
from fractions import Fraction

import numpy as np
import pytest

import dot_model as dm
from workloads import case_seed

E4M3, E5M2 = 0, 1
ONE = 0x38                              # E4M3 code of 1.0


def enc(orc, vals, fmt=E4M3):
    return np.array([[orc.encode(float(v), fmt) for v in row] for row in vals], np.uint8)


def bound_and_model(orc, a, fa, sa, ga, b, fb, sb, gb):
    M, N = a.shape[0], b.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    m, n = mm.ravel(), nn.ravel()
    bnd = orc.dot_truncation_bound(a, fa, sa, ga, b, fb, sb, gb, m, n)
    emu, exa = dm.emulate_points(a, fa, sa, ga, b, fb, sb, gb, m, n)
    return bnd.reshape(M, N), emu.reshape(M, N), exa.reshape(M, N)


def one_scale():
    return np.ones((1, 1), np.float32)


def test_boundary_2p13_kept_2p14_dropped(orc):
    """X = 256 (E_g = 8, unit 2^-5) with d in the same group: d = 2^-5 (ratio 2^13)
    survives, d = 2^-6 (ratio 2^14) is dropped; in the next group d survives.
    Bound = (nonzero products in the group) * 2^(E_g - 13)."""
    rows = [[256, 2 ** -5] + [0] * 14,
            [256, 2 ** -6] + [0] * 14,
            [256] + [0] * 7 + [2 ** -6] + [0] * 7]
    a = enc(orc, rows)
    b = np.full((1, 16), ONE, np.uint8)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert emu[:, 0].tolist() == [256 + 2 ** -5, 256.0, 256 + 2 ** -6]
    assert exa[:, 0].tolist() == [256 + 2 ** -5, 256 + 2 ** -6, 256 + 2 ** -6]
    # second group of row 2: one product 2^-6, E_g = -6, unit 2^-19
    assert bnd[:, 0].tolist() == [2 ** -4, 2 ** -4, 2 ** -5 + 2 ** -19]


def test_subnormal_group_uses_smallest_normal_exponent(orc):
    """A group of E4M3 subnormals (0x01 = 2^-9, 0x03 = 3 * 2^-9) times 1.0:
    E_g = -6 + 0, not -9 or -8, so the bound is 2 * 2^-19; nothing is lost.
    With 256 in the group, E_g = 8 and both subnormals are dropped."""
    a = np.zeros((2, 8), np.uint8)
    a[0, :2] = [0x01, 0x03]
    a[1, :3] = [0x01, 0x03, orc.encode(256.0, E4M3)]
    b = np.full((1, 8), ONE, np.uint8)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert bnd[0, 0] == 2 * 2.0 ** -19
    assert emu[0, 0] == exa[0, 0] == 4 * 2.0 ** -9
    assert bnd[1, 0] == 3 * 2.0 ** -5
    assert emu[1, 0] == 256.0 and exa[1, 0] == 256 + 4 * 2.0 ** -9
    # E5M2 subnormal 0x01 = 2^-16 counts at -14
    a5 = np.zeros((1, 8), np.uint8)
    a5[0, 0] = 0x01
    bnd5, emu5, _ = bound_and_model(orc, a5, E5M2, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert bnd5[0, 0] == 2.0 ** (-14 - 13) and emu5[0, 0] == 2.0 ** -16


def test_mixed_signs_truncate_toward_zero(orc):
    """-256 and +256 with small terms of both signs: each small term is
    truncated toward zero on its own magnitude, so 2^-6 and -2^-6 both vanish
    while 2^-5 and -2^-4 survive; the bound counts all five products."""
    row = [-256, 2 ** -6, -(2 ** -6), 2 ** -5, -(2 ** -4), 0, 0, 0]
    a = enc(orc, [row])
    b = np.full((1, 8), ONE, np.uint8)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert emu[0, 0] == -256 + 2 ** -5 - 2 ** -4
    assert exa[0, 0] == -256 + 2 ** -5 - 2 ** -4
    assert bnd[0, 0] == 5 * 2.0 ** -5
    # signs on the B side flip the products, not the magnitudes
    b2 = b.copy()
    b2[0, 1] = 0xB8                       # -1.0
    _, emu2, _ = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b2, E4M3, one_scale(), (0, 0))
    assert emu2[0, 0] == emu[0, 0]


def test_k_tail_group(orc):
    """K = 12: groups {0..7} and {8..11}.  Group 0 is eight 1.0s (E_g = 0,
    nothing lost); the tail group [256, 2^-5, 2^-6, 1] has E_g = 8, unit 2^-5:
    2^-6 is dropped, 2^-5 and 1 kept."""
    row = [1] * 8 + [256, 2 ** -5, 2 ** -6, 1]
    a = enc(orc, [row])
    b = np.full((1, 12), ONE, np.uint8)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert bnd[0, 0] == 8 * 2.0 ** -13 + 4 * 2.0 ** -5
    assert emu[0, 0] == 8 + 256 + 2 ** -5 + 1
    assert exa[0, 0] == emu[0, 0] + 2 ** -6


@pytest.mark.parametrize("blk", [32, 128])
def test_scale_block_edges(orc, blk):
    """K-blocked scales: the group ending at k = blk - 1 takes the first
    block's scale and the group starting at k = blk the second's; each group's
    bound term is multiplied by |s_a s_b| of its own block."""
    K = 2 * blk
    row = [0.0] * K
    row[blk - 8], row[blk - 7] = 256, 2 ** -6          # last group of block 0
    row[blk], row[blk + 1] = 256, 2 ** -6              # first group of block 1
    a = enc(orc, [row])
    b = np.full((1, K), ONE, np.uint8)
    sa = np.array([[2.0, -0.5]], np.float32)
    sb = np.array([[3.0, 4.0]], np.float32)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, sa, (1, blk), b, E4M3, sb, (1, blk))
    assert bnd[0, 0] == 6.0 * 2 * 2.0 ** -5 + 2.0 * 2 * 2.0 ** -5
    assert emu[0, 0] == 6.0 * 256 - 2.0 * 256
    assert exa[0, 0] == 6.0 * (256 + 2 ** -6) - 2.0 * (256 + 2 ** -6)


def random_operands(g, M, N, K, fa, spread):
    """Codes of values N(0,1) * 2^U(-spread, spread): wide exponent ranges
    inside a group, so truncation happens."""
    import oracle

    xa = g.standard_normal((M, K)) * np.exp2(g.uniform(-spread, spread, (M, K)))
    xb = g.standard_normal((N, K)) * np.exp2(g.uniform(-spread, spread, (N, K)))
    fm_a = oracle.fmax(fa)
    xa = np.clip(xa, -fm_a, fm_a).astype(np.float32)
    xb = np.clip(xb, -448, 448).astype(np.float32)
    a = np.vectorize(lambda v: oracle.encode(float(v), fa), otypes=[np.uint8])(xa)
    b = np.vectorize(lambda v: oracle.encode(float(v), E4M3), otypes=[np.uint8])(xb)
    return a, b


GRANS = [((0, 0), (0, 0)), ((1, 0), (1, 0)), ((1, 128), (128, 128)), ((1, 32), (1, 32)), ((1, 128), (1, 0))]


@pytest.mark.parametrize("fa", [E4M3, E5M2])
@pytest.mark.parametrize("grans", GRANS)
@pytest.mark.parametrize("spread", [3, 10])
def test_bound_holds_on_random_operands(orc, fa, grans, spread):
    g = np.random.default_rng(case_seed("dotbound", fa, grans, spread))
    M, N, K = 9, 11, 300 if grans[0][1] == 0 else 256
    a, b = random_operands(g, M, N, K, fa, spread)
    ga, gb = grans

    def scales(rows, cols, gr, gc):
        er = rows if gr <= 0 else gr
        ec = K if gc <= 0 or gc > K else gc
        return (g.uniform(0.25, 4, ((rows + er - 1) // er, (K + ec - 1) // ec)) *
                g.choice([-1, 1], ((rows + er - 1) // er, (K + ec - 1) // ec))).astype(np.float32)

    sa, sb = scales(M, K, *ga), scales(N, K, *gb)
    bnd, emu, exa = bound_and_model(orc, a, fa, sa, ga, b, E4M3, sb, gb)
    lost = np.abs(exa - emu)
    assert np.all(lost <= bnd * (1 + 1e-12)), float((lost / bnd).max())
    if spread == 10:
        assert np.count_nonzero(lost) > 0          # the model does truncate here
    # the oracle's exact reference agrees with the emulation's exact sums
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    yref, S = orc.gemm_points(a, fa, sa, ga, b, E4M3, sb, gb, mm.ravel(), nn.ravel())
    assert np.all(np.abs(yref.reshape(M, N) - exa) <= 1e-13 * S.reshape(M, N))


@pytest.mark.parametrize("fa", [E4M3, E5M2])
def test_no_loss_when_group_exponents_are_close(orc, fa):
    """Products whose exponent sums lie within 7 of the group maximum are
    multiples of 2^(E_g - 13) already: the emulation equals the exact sum."""
    g = np.random.default_rng(case_seed("close", fa))
    a, b = random_operands(g, 6, 7, 128, fa, 0)
    sgA, sigA, uA, eA, lA = dm.code_fields(fa)
    sgB, sigB, uB, eB, lB = dm.code_fields(E4M3)
    # keep only codes with exponents in [-2, 1] on both sides (sums within 6)
    a = np.where((eA[a] >= -2) & (eA[a] <= 1), a, 0).astype(np.uint8)
    b = np.where((eB[b] >= -2) & (eB[b] <= 1), b, 0).astype(np.uint8)
    _, emu, exa = bound_and_model(orc, a, fa, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    assert np.array_equal(emu, exa)


def test_bound_is_nearly_reached(orc):
    """Each group: 256 (E_g = 8, unit 2^-5) and seven products just under one
    unit (1.875 * 2^-3 times 1.875 * 2^-4 = 0.879 * 2^-5 each).  The loss is
    7 * 0.879 = 6.15 units against a bound of 8 units."""
    K = 64
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    big, small = orc.encode(256.0, E4M3), orc.encode(1.875 * 2 ** -3, E4M3)
    for k0 in range(0, K, 8):
        a[0, k0], b[0, k0] = big, ONE
        a[0, k0 + 1:k0 + 8] = small
        b[0, k0 + 1:k0 + 8] = orc.encode(1.875 * 2 ** -4, E4M3)
    bnd, emu, exa = bound_and_model(orc, a, E4M3, one_scale(), (0, 0), b, E4M3, one_scale(), (0, 0))
    ratio = (exa - emu)[0, 0] / bnd[0, 0]
    assert abs(ratio - 7 * 0.87890625 / 8) < 1e-12


@pytest.mark.parametrize("fa", [E4M3, E5M2])
def test_vectorised_emulation_matches_scalar_rationals(orc, fa):
    g = np.random.default_rng(case_seed("scalar", fa))
    M, N, K = 3, 4, 40
    a, b = random_operands(g, M, N, K, fa, 9)
    sa = np.array([[1.0, 2.0, -0.5, 4.0, 1.0]], np.float32).repeat(M, 0)
    sb = np.ones((1, 1), np.float32)
    bnd, emu, exa = bound_and_model(orc, a, fa, sa, (1, 8), b, E4M3, sb, (0, 0))
    for m in range(M):
        for n in range(N):
            e_s, x_s = dm.emulate_dot_scalar(a[m], fa, b[n], E4M3, lambda k0: sa[m, k0 // 8])
            assert emu[m, n] == float(e_s) and exa[m, n] == float(x_s)
            assert Fraction(float(bnd[m, n])) >= abs(x_s - e_s)
