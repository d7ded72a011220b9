"""fp8_quantize_packed16: the quantize with its codes written straight into
the fragment-ordered weight image.

- Against the oracle (its quantize, then its pack_weights16): every byte of
  the image over a poisoned buffer (the rows past N of a short last 16-row
  group must come back zero), and scales, inverse scales, amax and counters
  bit for bit.  One case or more per quantize kernel: per tensor (DYNAMIC and
  GIVEN), per row, 1 x 32 and 1 x 128 groups, 128 x 128 blocks and a 16 x 48
  grid of groups, fp32 and bf16 inputs, E4M3 and E5M2.
- Per-row and per-tensor scales take a kernel of their own when a row fits
  its registers (up to 4 steps of 128 per wave for bf16; 2 for fp32, 1
  with counters), the row-wise kernels otherwise: cases on both sides of
  each limit.
- At the weights' own sizes (8192 x 8192 per channel, 18432 x 7168 in
  128 x 128 blocks, 29568 x 8192 per tensor GIVEN, 4096 x 8192 per tensor
  DYNAMIC): the image equals the library's row-major quantize followed by
  its pack, byte for byte, with the same scales and counters."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from workloads import case_seed, to_bf16_bits

pytestmark = pytest.mark.gpu

DYN, GIVEN = 0, 1


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def make_input(seed, rows, cols, dtype, special=False):
    """Normal values with a per-row magnitude spread, an all-zero row, a few
    outliers and values that underflow; with `special`, a NaN in one row and
    an Inf in another (codes bit for bit; NaN scales and amax by position)."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(g.uniform(-4, 4, (rows, 1))).astype(np.float32)
    x[g.integers(0, rows), :] = 0.0
    x.reshape(-1)[g.integers(0, rows * cols, 5)] *= 300.0
    x.reshape(-1)[g.integers(0, rows * cols, 7)] = 1e-30
    if special:
        x[1, g.integers(0, cols)] = np.nan
        x[rows - 2, g.integers(0, cols)] = -np.inf
    return to_bf16_bits(x) if dtype == "bf16" else x


def same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def same_nan(a, b):
    """Bit for bit except NaN payloads: the oracle writes the canonical quiet
    NaN, the kernels carry the input's payload through the integer max of
    |x| (a bf16 0xFFFF gives amax bits 0x7FFF0000); NaN in the same places."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and same_f32(a[~na], b[~nb])



CASES = [  # (N, K, gran, dtype, fmt, mode, counters)
    (16, 128, (0, 0), "bf16", 0, DYN, True),       # one tile, per tensor
    (17, 256, (1, 32), "f32", 1, DYN, True),       # a second group with one live row
    (130, 512, (1, 128), "bf16", 1, DYN, True),
    (200, 1024, (1, 0), "f32", 0, DYN, True),      # per row, ragged N
    (300, 768, (128, 128), "bf16", 0, DYN, True),  # ragged blocks on both sides
    (96, 384, (16, 48), "f32", 0, DYN, True),
    (1000, 2048, (0, 0), "f32", 0, GIVEN, True),   # saturating given scale
    (64, 4096, (1, 0), "bf16", 1, GIVEN, True),
    (40, 6144, (1, 0), "bf16", 0, DYN, True),      # three steps per wave
    (40, 8192, (1, 0), "bf16", 0, DYN, False),     # four steps per wave (no counters)
    (40, 8192, (1, 0), "bf16", 0, DYN, True),      # four steps per wave, with counters
    (24, 8320, (1, 0), "bf16", 0, DYN, True),      # 65 steps: past the image kernel, the row kernel
    (33, 4096, (0, 0), "f32", 0, DYN, True),       # fp32 with counters past one step: the tensor kernel
    (33, 8192, (0, 0), "bf16", 1, DYN, False),     # per tensor: amax pass, then the image kernel
    (48, 4096, (1, 0), "f32", 0, GIVEN, False),
    (48, 8192, (1, 0), "f32", 0, DYN, False),      # fp32 past the register budget
    (40, 8192, (1, 0), "bf16", 0, DYN, False, True),   # NaN and Inf rows, the image kernel
    (40, 8192, (1, 0), "bf16", 1, DYN, True, True),    # the same, the general kernel
    (64, 2048, (0, 0), "bf16", 0, GIVEN, True, True),  # per tensor, given scale
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_quantize_into_image_matches_oracle(rt, orc, case):
    N, K, gran, dtype, fmt, mode, counters = case[:7]
    special = len(case) > 7 and case[7]
    x = make_input(case_seed("image", case), N, K, dtype, special)
    G = rt.scale_shape((N, K), gran)
    if mode == DYN:
        oq, os_, or_, oam, ocnt = orc.quantize(x, fmt, gran)
        S = torch.full(G, -1.0, device="cuda")
        R = torch.full(G, -1.0, device="cuda")
    else:
        # half the dynamic scale of the finite values: some codes saturate
        _, s0, _, _, _ = orc.quantize(make_input(case_seed("image", case), N, K, dtype), fmt, gran)
        s_given = (s0 * 0.5).astype(np.float32)
        oq, os_, or_, oam, ocnt = orc.quantize(x, fmt, gran, mode=GIVEN, scale=s_given)
        S = dev(s_given)
        R = None
    am = torch.full(G, -1.0, device="cuda")
    cnt = torch.full((2,), -1, dtype=torch.int64, device="cuda") if counters else None
    out = torch.full((rt.packed16_bytes(N, K),), 0xAB, dtype=torch.uint8, device="cuda")
    p = rt.fp8_quantize_packed16(dev(x), gran, fmt, mode, 1e-12, False, S, R, out=out, amax_out=am,
                                 sat_underflow=cnt)
    torch.cuda.synchronize()
    assert (p.N, p.K) == (N, K)
    got = host(p.data)
    ref = orc.pack_weights16(oq)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "%d image bytes differ, first at %d" % (bad.size, bad[0])
    same = same_nan if special else same_f32
    assert same(host(am), oam)
    if mode == DYN:
        assert same(host(S), os_) and same(host(R), or_)
    if counters:
        assert host(cnt).view(np.uint64).tolist() == ocnt.tolist()
    if mode == GIVEN:
        assert ocnt[0] > 0                               # the case does saturate


FULL = [  # (N, K, gran, fmt, mode, counters)
    (8192, 8192, (1, 0), 0, DYN, False),
    (8192, 8192, (1, 0), 0, DYN, True),
    (18432, 7168, (128, 128), 0, DYN, True),
    (29568, 8192, (0, 0), 0, GIVEN, False),
    (29568, 8192, (0, 0), 0, GIVEN, True),
    (4096, 8192, (0, 0), 1, DYN, False),
]


@pytest.mark.parametrize("case", FULL, ids=[str(c) for c in FULL])
def test_quantize_into_image_full_size(rt, case):
    """The image against quantize + pack of the same weight on the device."""
    N, K, gran, fmt, mode, counters = case
    print("quantize into image, full size", case, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(case_seed("image-full", case))
    w = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    G = rt.scale_shape((N, K), gran)
    if mode == DYN:
        s0, s1 = torch.empty(G, device="cuda"), torch.empty(G, device="cuda")
    else:
        s0 = torch.full(G, float(w.float().abs().max()) / 448.0 * 0.25, device="cuda")  # saturates the tails
        s1 = s0.clone()
    c0 = torch.zeros(2, dtype=torch.int64, device="cuda")
    c1 = torch.zeros(2, dtype=torch.int64, device="cuda")
    q = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    rt.fp8_quantize(w, gran, fmt, mode, 1e-12, False, s0, None, q, None, c0)
    ref = rt.fp8_pack_weights16(q)
    out = torch.full((rt.packed16_bytes(N, K),), 0xAB, dtype=torch.uint8, device="cuda")
    p = rt.fp8_quantize_packed16(w, gran, fmt, mode, 1e-12, False, s1, None, out=out,
                                 sat_underflow=c1 if counters else None)
    torch.cuda.synchronize()
    assert torch.equal(p.data, ref.data)
    assert torch.equal(s0, s1)
    if counters:
        assert c0.tolist() == c1.tolist()
        if mode == GIVEN:
            assert c1[0].item() > 0
