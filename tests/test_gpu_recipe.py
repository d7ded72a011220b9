"""Parity of the HIP delayed-scaling recipe step (fp8_delayed_scale_update:
window-max or latest history function, power-of-two margin) with the CPU
oracle: history ring, head, scale and inverse scale bit-exact after every
step of a sequence with a spike, zeros, a negative value, a subnormal amax
and a NaN, for both formats, with and without the power-of-two round-up."""
import numpy as np
import pytest
import torch

from gpu_helpers import host, same_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    rt.lib()
    assert torch.cuda.is_available()
    return rt


def sequence(seed):
    g = np.random.default_rng(seed)
    a = np.exp(g.uniform(-8, 8, 40)).astype(np.float32)
    a[7] *= np.float32(1e4)          # spike
    a[11] = 0.0
    a[12] = -3.0                     # never a real amax; counts as zero
    a[20] = np.float32(1e-41)        # subnormal
    a[33] = np.nan
    return a


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("fn", [0, 1])
@pytest.mark.parametrize("margin", [0, 2, 16])
@pytest.mark.parametrize("pow2", [False, True])
def test_recipe_sequence_bit_exact(rt, orc, fmt, fn, margin, pow2):
    length = 5
    seq = sequence(100 + fmt + 2 * fn + 4 * margin + 64 * pow2)
    hist_ref = np.zeros(length, np.float32)
    head_ref = 0
    H = torch.zeros(length, dtype=torch.float32, device="cuda")
    head = torch.zeros(1, dtype=torch.int32, device="cuda")
    an = torch.empty(1, dtype=torch.float32, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    r = torch.empty(1, dtype=torch.float32, device="cuda")
    eps = 1e-12
    for t, a in enumerate(seq):
        an.fill_(float(a))
        rt.fp8_delayed_scale_update(H, head, an, fmt, fn, margin, eps, pow2, s, r)
        head_ref, s_ref, r_ref = orc.history_update_recipe(hist_ref, head_ref, float(a), fmt, fn, margin,
                                                           eps=eps, pow2=pow2)
        torch.cuda.synchronize()
        assert same_f32(host(H), hist_ref), t
        assert int(host(head)[0]) == head_ref, t
        assert same_f32(host(s), [s_ref]) and same_f32(host(r), [r_ref]), (t, host(s), s_ref, host(r), r_ref)


def test_window_max_margin0_matches_history_update(rt):
    """The recipe entry point with the window maximum and no margin is the
    plain history update: same ring, head and scales on one sequence."""
    seq = sequence(7)
    out = []
    for use_recipe in (False, True):
        H = torch.zeros(6, dtype=torch.float32, device="cuda")
        head = torch.zeros(1, dtype=torch.int32, device="cuda")
        an = torch.empty(1, dtype=torch.float32, device="cuda")
        s = torch.empty(1, dtype=torch.float32, device="cuda")
        r = torch.empty(1, dtype=torch.float32, device="cuda")
        trace = []
        for a in seq:
            an.fill_(float(a))
            if use_recipe:
                rt.fp8_delayed_scale_update(H, head, an, 0, rt.HIST_MAX, 0, 1e-12, False, s, r)
            else:
                rt.fp8_amax_history_update(H, head, an, 0, 1e-12, False, s, r)
            trace.append(np.concatenate([host(s), host(r), host(H)]))
        out.append(np.stack(trace))
    assert same_f32(out[0], out[1])
