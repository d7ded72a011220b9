"""Test-side helpers: move numpy arrays (float32, bf16 bits as uint16, uint8)
to and from the GPU, and the GEMM acceptance rule."""
import os

import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def same_f32(a, b) -> bool:
    """Bitwise equality of binary32 arrays, any NaN equal to any NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    if a.shape != b.shape:
        return False
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 at |v| (8 significant bits, binary32 exponent range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


# Statistics of every GEMM acceptance check in this process, written out at
# the end of the session when FP8RT_PARITY_LOG names a file (tests/conftest.py).
GEMM_STATS = []


def check_gemm(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray, out_bf16: bool, orc, bias=None,
               rel=1e-5, t_hw=None):
    """The one GEMM acceptance rule, applied per element whatever the number of
    elements.  fp32: |y - y_ref| <= rel * S + T_hw (+ 2^-24 |bias|).  bf16: within
    1 bf16 ulp of RNE_bf16(y_ref), or |y - y_ref| <= rel * S + T_hw + ulp_bf16(y_ref)
    where cancellation makes |y_ref| << S.  T_hw bounds the truncation inside the
    matrix cores' FP8 dot product (oracle.dot_truncation_bound); kernels whose
    products are exact pass none.  Besides pass / fail the stats record how many
    elements exceed rel * S alone (n_over_rel) and the largest |y - y_ref| / S;
    they are recorded, never a pass condition.  Returns (ok, stats)."""
    y_ref = np.asarray(y_ref, np.float64)
    S = np.asarray(S, np.float64)
    t_hw = np.zeros_like(S) if t_hw is None else np.asarray(t_hw, np.float64)
    slack = np.zeros_like(S) if bias is None else 2.0 ** -24 * np.abs(np.asarray(bias, np.float64))
    if not out_bf16:
        err = np.abs(y_gpu.astype(np.float64) - y_ref)
        ok = err <= rel * S + t_hw + slack
        ratio = err / np.maximum(S, 1e-300)
        st = {"max_err_over_S": float(ratio.max()) if ratio.size else 0.0, "n_bad": int((~ok).sum()),
              "n_over_rel": int((err > rel * S + slack).sum()), "n": int(ok.size)}
    else:
        yb = orc.bf16_bits_to_f32(y_gpu).astype(np.float64)
        rb = orc.bf16_bits_to_f32(orc.round_bf16(y_ref)).astype(np.float64)
        ulp = bf16_ulp(rb)
        strict = np.abs(yb - rb) <= ulp
        err = np.abs(yb - y_ref)
        fallback_rel = err <= rel * S + bf16_ulp(y_ref) + slack
        fallback = err <= rel * S + t_hw + bf16_ulp(y_ref) + slack
        ok = strict | fallback
        ratio = err / np.maximum(S, 1e-300)
        st = {"n_fallback": int((~strict & fallback).sum()), "n_bad": int((~ok).sum()),
              "n_over_rel": int((~strict & ~fallback_rel).sum()), "n": int(ok.size),
              "max_err_over_S": float(ratio.max()) if ratio.size else 0.0}
    st["frac_over_rel"] = st["n_over_rel"] / max(st["n"], 1)
    GEMM_STATS.append(dict(st, out="bf16" if out_bf16 else "f32",
                           test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]))
    return bool(ok.all()), st
