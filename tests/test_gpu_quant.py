"""Parity of the HIP amax / scale / quantize / dequantize / history path with
the CPU oracle: bit-exact codes, scales, inverse scales, amax and counters,
on seeded inputs spanning several workgroups, ragged tails and special
values.  Calls go through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, same_f32
from workloads import case_seed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def make_input(seed, rows, cols, dtype):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(g.uniform(-6, 6, (rows, 1))).astype(np.float32)   # per-row magnitude spread
    x[g.integers(0, rows), :] = 0.0                                 # an all-zero row
    idx = g.integers(0, rows * cols, 5)
    x.reshape(-1)[idx] *= 300.0                                     # outliers
    x.reshape(-1)[g.integers(0, rows * cols, 7)] = 1e-30            # underflow candidates
    if dtype == "bf16":
        from workloads import to_bf16_bits
        return to_bf16_bits(x)
    return x


def run_quant(rt, x_np, gran, fmt, mode=0, eps=1e-12, pow2=False, scale=None, inv=None,
              want_inv=True, ldx_pad=0, ldq_pad=0):
    rows, cols = x_np.shape
    xd = dev(x_np)
    if ldx_pad:
        big = torch.zeros((rows, cols + ldx_pad), dtype=xd.dtype, device="cuda")
        big[:, :cols] = xd
        xd = big[:, :cols]
    G = rt.scale_shape((rows, cols), gran)
    qd = torch.full((rows, cols + ldq_pad), 0xAA, dtype=torch.uint8, device="cuda")[:, :cols]
    if mode == rt.DYNAMIC:
        s = torch.full(G, -1.0, device="cuda")
        r = torch.full(G, -1.0, device="cuda") if want_inv else None
    else:
        s = dev(np.ascontiguousarray(scale, np.float32).reshape(G))
        r = None if inv is None else dev(np.ascontiguousarray(inv, np.float32).reshape(G))
    am = torch.full(G, -1.0, device="cuda")
    cnt = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    rt.fp8_quantize(xd, gran, fmt, mode, eps, pow2, s, r, qd, am, cnt)
    torch.cuda.synchronize()
    return (host(qd), host(s), None if r is None else host(r), host(am),
            host(cnt).view(np.uint64))


GRANS = [(0, 0), (1, 0), (1, 128), (1, 32), (1, 64), (128, 128), (16, 48), (3, 0), (0, 80)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", GRANS)
def test_dynamic_quantize_bit_exact(rt, orc, dtype, fmt, gran):
    rows, cols = (300, 400) if gran[0] > 1 else (37, 400)
    x = make_input(case_seed(dtype, fmt, gran), rows, cols, dtype)
    q, s, r, am, cnt = run_quant(rt, x, gran, fmt)
    oq, os_, or_, oam, ocnt = orc.quantize(x, fmt, gran)
    assert same_f32(am, oam)
    assert same_f32(s, os_) and same_f32(r, or_)
    assert np.array_equal(q, oq), np.argwhere(q != oq)[:5]
    assert cnt.tolist() == ocnt.tolist()


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", [(0, 0), (1, 32), (1, 128), (128, 128)])
def test_dynamic_pow2_scales(rt, orc, fmt, gran):
    x = make_input(77 + fmt, 260, 512, "bf16")
    q, s, r, am, cnt = run_quant(rt, x, gran, fmt, pow2=True)
    oq, os_, or_, oam, ocnt = orc.quantize(x, fmt, gran, pow2=True)
    assert same_f32(s, os_) and same_f32(r, or_)
    assert np.array_equal(q, oq)
    assert cnt.tolist() == ocnt.tolist()
    ex = (s.view(np.uint32) & 0x7FFFFF)
    assert np.all(ex == 0)                      # every scale is a power of two


@pytest.mark.parametrize("fmt", [0, 1])
def test_every_tie_and_edge_value(rt, orc, fmt):
    """GIVEN s = 1: the cast alone, over every code, every midpoint between
    neighbouring codes and their +-1,2 ulp neighbours, subnormals, values past
    F_max, +-0, +-Inf, NaN and a million wide-range random values."""
    pts = set()
    for f in (0, 1):
        finite = sorted({abs(orc.decode(c, f)) for c in range(256) if np.isfinite(orc.decode(c, f))})
        pts.update(finite)
        pts.update((a + b) / 2 for a, b in zip(finite[:-1], finite[1:]))
        pts.update([finite[-1] * k for k in (1.03, 1.0625, 1.125, 2.0, 1e6)])
    base = np.array(sorted(pts), np.float32).view(np.uint32).astype(np.int64)
    nb = np.concatenate([base + d for d in (-2, -1, 0, 1, 2)])
    nb = nb[(nb >= 0) & (nb < 0x7F800000)].astype(np.uint32).view(np.float32)
    g = np.random.default_rng(5)
    rnd = (g.standard_normal(1 << 20) * np.exp(g.uniform(-30, 14, 1 << 20))).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 1e-45, -1e-45, 3e38], np.float32)
    x = np.concatenate([nb, -nb, special, rnd])
    x = np.concatenate([x, np.zeros((-len(x)) % 1024, np.float32)]).reshape(-1, 1024)
    one = np.ones((1, 1), np.float32)
    q, s, r, am, cnt = run_quant(rt, x, (0, 0), fmt, mode=rt.GIVEN, scale=one)
    oq, _, _, oam, ocnt = orc.quantize(x, fmt, (0, 0), mode=orc.GIVEN, scale=one)
    assert np.array_equal(q, oq), [(x.ravel()[i], q.ravel()[i], oq.ravel()[i])
                                   for i in np.flatnonzero(q.ravel() != oq.ravel())[:5]]
    assert same_f32(am, oam)
    assert cnt.tolist() == ocnt.tolist()


@pytest.mark.parametrize("gran", [(0, 0), (1, 0), (1, 128), (128, 128)])
def test_given_mode_with_and_without_inverse(rt, orc, gran):
    x = make_input(91, 200, 256, "bf16")
    _, s0, r0, _, _ = orc.quantize(x, 1, gran)
    s = (s0 * np.float32(0.75)).astype(np.float32)          # a stale, too-small scale: saturates
    for inv in (None, (r0 * np.float32(1.5)).astype(np.float32)):
        q, _, _, am, cnt = run_quant(rt, x, gran, 1, mode=rt.GIVEN, scale=s, inv=inv)
        oq, _, _, oam, ocnt = orc.quantize(x, 1, gran, mode=orc.GIVEN, scale=s, inv_scale=inv)
        assert np.array_equal(q, oq)
        assert same_f32(am, oam)
        assert cnt.tolist() == ocnt.tolist() and ocnt[0] > 0


@pytest.mark.parametrize("gran", [(0, 0), (1, 0), (1, 128), (64, 64)])
def test_nan_and_inf_groups(rt, orc, gran):
    x = make_input(5, 130, 256, "f32")
    x[3, 17] = np.nan
    x[70, 200] = np.inf
    x[129, 5] = -np.inf
    for mode in (0, 1):
        kw = {}
        if mode == 1:
            kw = dict(scale=np.full(rt.scale_shape(x.shape, gran), 0.01, np.float32))
        q, s, r, am, cnt = run_quant(rt, x, gran, 0, mode=mode, **kw)
        oq, os_, or_, oam, ocnt = orc.quantize(x, 0, gran, mode=mode, **({} if mode == 0 else
                                                                          {"scale": kw["scale"]}))
        assert np.array_equal(q, oq)
        assert same_f32(am, oam)
        if mode == 0:
            assert same_f32(s, os_) and same_f32(r, or_)
        assert cnt.tolist() == ocnt.tolist()


def test_strided_operands_and_null_outputs(rt, orc):
    x = make_input(12, 40, 256, "bf16")
    for gran in ((0, 0), (1, 128), (8, 64)):
        q, s, r, am, cnt = run_quant(rt, x, gran, 0, ldx_pad=48, ldq_pad=16, want_inv=False)
        oq, os_, _, oam, _ = orc.quantize(x, 0, gran)
        assert np.array_equal(q, oq) and same_f32(s, os_)


def test_all_zero_tensor_gives_finite_positive_scale(rt, orc):
    x = np.zeros((16, 64), np.float32)
    q, s, r, am, cnt = run_quant(rt, x, (0, 0), 0)
    assert s[0, 0] > 0 and np.isfinite(s[0, 0]) and np.isfinite(r[0, 0])
    _, os_, or_, _, ocnt = orc.quantize(x, 0, (0, 0))
    assert same_f32(s, os_) and same_f32(r, or_)
    assert np.all(q == 0) and cnt.tolist() == [0, 0]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gran", GRANS)
def test_amax_entry_point(rt, orc, dtype, gran):
    rows, cols = (300, 400) if gran[0] > 1 else (37, 400)
    x = make_input(3, rows, cols, dtype)
    x_d = dev(x)
    am = torch.full(rt.scale_shape(x.shape, gran), -1.0, device="cuda")
    rt.fp8_amax(x_d, gran, am)
    torch.cuda.synchronize()
    assert same_f32(host(am), orc.amax(x, gran))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("pow2", [False, True])
def test_compute_scale(rt, orc, fmt, pow2):
    g = np.random.default_rng(8)
    a = np.exp(g.uniform(-80, 85, 5000)).astype(np.float32)
    a[:6] = [0.0, np.nan, np.inf, 1e-13, 448.0, 57344.0]
    s = torch.empty(a.size, device="cuda")
    r = torch.empty(a.size, device="cuda")
    rt.fp8_compute_scale(dev(a), fmt, 1e-12, pow2, s, r)
    torch.cuda.synchronize()
    os_, or_ = orc.compute_scale(a, fmt, pow2=pow2)
    assert same_f32(host(s), os_) and same_f32(host(r), or_)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("gran", [(0, 0), (1, 0), (1, 128), (128, 128), (1, 32)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize(rt, orc, fmt, gran, out):
    g = np.random.default_rng(4)
    rows, cols = 150, 384
    codes = g.integers(0, 256, (rows, cols)).astype(np.uint8)
    sc = np.exp(g.uniform(-8, 8, rt.scale_shape((rows, cols), gran))).astype(np.float32)
    y = torch.empty((rows, cols), dtype=torch.float32 if out == "f32" else torch.bfloat16, device="cuda")
    rt.fp8_dequantize(dev(codes), fmt, gran, dev(sc), y)
    torch.cuda.synchronize()
    oy = orc.dequantize(codes, fmt, sc, gran, out_dtype=0 if out == "f32" else 1)
    yh = host(y)
    if out == "f32":
        assert same_f32(yh, oy)
    else:
        assert same_f32(orc.bf16_bits_to_f32(yh), orc.bf16_bits_to_f32(oy))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("length", [1, 16, 100])
def test_history_update_sequence(rt, orc, fmt, length):
    g = np.random.default_rng(length)
    steps = 60
    a_seq = np.exp(g.normal(0, 1.5, steps)).astype(np.float32)
    a_seq[13] *= 100.0
    a_seq[20] = 0.0
    hist_d = torch.zeros(length, device="cuda")
    head_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    s_d = torch.empty(1, device="cuda")
    r_d = torch.empty(1, device="cuda")
    hist_o = np.zeros(length, np.float32)
    head_o = 0
    for t in range(steps):
        rt.fp8_amax_history_update(hist_d, head_d, dev(a_seq[t:t + 1]), fmt, 1e-12, t % 2 == 1, s_d, r_d)
        head_o, so, ro = orc.history_update(hist_o, head_o, a_seq[t], fmt, pow2=t % 2 == 1)
        torch.cuda.synchronize()
        assert int(host(head_d)[0]) == head_o
        assert same_f32(host(hist_d), hist_o)
        assert same_f32(host(s_d), [so]) and same_f32(host(r_d), [ro])
