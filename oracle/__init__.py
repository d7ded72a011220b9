"""CPU oracle for the FP8 runtime chain -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``liboracle.so`` (built from ``fp8_oracle.c`` with
gcc).  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this package; the HIP library never does, and the two share
no code.  Arrays are numpy arrays on the host; bfloat16 tensors travel as
``uint16`` bit patterns.

The arithmetic lives in ``fp8_oracle.c``; each C function cites the passage
of the pages it follows (page title and section).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "fp8_oracle.c"), os.path.join(_HERE, "fp8_dot_bound.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A build with AddressSanitizer and UndefinedBehaviorSanitizer, loaded instead
# when FP8RT_ORACLE_SANITIZED=1 (the process must preload gcc's libasan).
_ASAN_PATH = os.path.join(_HERE, "liboracle_asan.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
DYNAMIC, GIVEN = 0, 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-Wall", "-fPIC", "-shared",
                               "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """Compile the same sources with ASan + UBSan (every UB report fatal)."""
    tmp = _ASAN_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-Wall", "-fPIC", "-shared", *SANITIZE_FLAGS,
                           "-o", tmp, *_SRCS, "-lm"])
    os.replace(tmp, _ASAN_PATH)
    return _ASAN_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB_PATH
        if os.environ.get("FP8RT_ORACLE_SANITIZED") == "1":
            path = _ASAN_PATH
            if not os.path.exists(path):
                raise ImportError("liboracle_asan.so is not built (oracle.build_sanitized())")
        elif not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(path)
        P, I64, I, F, D = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_double
        L.orc_fmax.restype = D
        L.orc_fmax.argtypes = [I]
        L.orc_decode.restype = D
        L.orc_decode.argtypes = [C.c_uint, I]
        L.orc_encode.restype = C.c_uint
        L.orc_encode.argtypes = [F, I]
        L.orc_encode_bruteforce.restype = C.c_uint
        L.orc_encode_bruteforce.argtypes = [F, I]
        L.orc_amax.restype = I
        L.orc_amax.argtypes = [P, I, I64, I64, I64, I64, I64, P]
        L.orc_compute_scale.restype = I
        L.orc_compute_scale.argtypes = [P, I64, I, F, I, P, P]
        L.orc_quantize.restype = I
        L.orc_quantize.argtypes = [P, I, I64, I64, I64, I64, I64, I, I, F, I, P, P, P, I64, P, P]
        L.orc_quantize_transpose.restype = I
        L.orc_quantize_transpose.argtypes = [P, I, I64, I64, I64, I64, I64, I, I, F, I, P, P, P, I64, P,
                                             I64, P, P]
        L.orc_dequantize.restype = I
        L.orc_dequantize.argtypes = [P, I, I64, I64, I64, I64, I64, P, P, I, I64]
        L.orc_history_update.restype = I
        L.orc_history_update.argtypes = [P, I, P, F, I, F, I, P, P]
        gemm_args = [P, I, I64, I64, I64, P, P, I, I64, I64, I64, P, I64, I64, I64, P, I, P, P,
                     I64, P]
        L.orc_gemm_points.restype = I
        L.orc_gemm_points.argtypes = gemm_args + [P]
        L.orc_gemm_points_exact.restype = I
        L.orc_gemm_points_exact.argtypes = gemm_args
        L.orc_pack_weights16.restype = I
        L.orc_pack_weights16.argtypes = [P, I64, I64, I64, P]
        L.orc_quant_error.restype = I
        L.orc_quant_error.argtypes = [P, I, I64, I64, I64, P, I, I64, I64, I64, P, P, I64, I64, P]
        L.orc_history_update_recipe.restype = I
        L.orc_history_update_recipe.argtypes = [P, I, P, F, I, I, I, F, I, P, P]
        L.orc_wonly_gemm_points.restype = I
        L.orc_wonly_gemm_points.argtypes = [P, I, I64, P, I, I64, I64, I64, P, I64, I64, I64, P, I,
                                            P, P, I64, P, P]
        L.orc_dot_truncation_bound.restype = I
        L.orc_dot_truncation_bound.argtypes = [P, I, I64, I64, I64, P, P, I, I64, I64, I64, P, I64,
                                               I64, I64, P, P, I64, P]
        L.orc_round_bf16.restype = C.c_uint16
        L.orc_round_bf16.argtypes = [D]
        L.orc_round_bf16_from_f32.restype = C.c_uint16
        L.orc_round_bf16_from_f32.argtypes = [F]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bf16 bits as uint16, got %s" % x.dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def ngroups(n: int, g: int) -> int:
    if g <= 0 or g >= n:
        return 1
    return -(-n // g)


def fmax(fmt: int) -> float:
    return lib().orc_fmax(fmt)


def decode(code: int, fmt: int) -> float:
    return lib().orc_decode(int(code), fmt)


def decode_table(fmt: int) -> np.ndarray:
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(v: float, fmt: int) -> int:
    return int(lib().orc_encode(float(v), fmt))


def encode_bruteforce(v: float, fmt: int) -> int:
    return int(lib().orc_encode_bruteforce(float(v), fmt))


def amax(x: np.ndarray, gran=(0, 0)) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = np.empty(ngroups(rows, gran[0]) * ngroups(cols, gran[1]), np.float32)
    _check(lib().orc_amax(_ptr(x), _dtype_code(x), rows, cols, cols, gran[0], gran[1],
                          _ptr(out)), "amax")
    return out.reshape(ngroups(rows, gran[0]), ngroups(cols, gran[1]))


def compute_scale(amax_arr: np.ndarray, fmt: int, eps: float = 1e-12, pow2: bool = False):
    a = np.ascontiguousarray(amax_arr, dtype=np.float32).ravel()
    s = np.empty_like(a)
    r = np.empty_like(a)
    _check(lib().orc_compute_scale(_ptr(a), a.size, fmt, eps, int(pow2), _ptr(s), _ptr(r)),
           "compute_scale")
    return s.reshape(np.shape(amax_arr)), r.reshape(np.shape(amax_arr))


def quantize(x: np.ndarray, fmt: int, gran=(0, 0), mode: int = DYNAMIC, eps: float = 1e-12,
             pow2: bool = False, scale: np.ndarray | None = None,
             inv_scale: np.ndarray | None = None):
    """Returns (codes uint8, scale, inv_scale, amax, counts[sat, under])."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    G = (ngroups(rows, gran[0]), ngroups(cols, gran[1]))
    q = np.empty((rows, cols), np.uint8)
    am = np.empty(G, np.float32)
    cnt = np.zeros(2, np.uint64)
    if mode == DYNAMIC:
        s = np.empty(G, np.float32)
        r = np.empty(G, np.float32)
    else:
        s = np.ascontiguousarray(scale, dtype=np.float32).reshape(G)
        r = None if inv_scale is None else np.ascontiguousarray(inv_scale, np.float32).reshape(G)
    _check(lib().orc_quantize(_ptr(x), _dtype_code(x), rows, cols, cols, gran[0], gran[1], fmt,
                              mode, eps, int(pow2), _ptr(s), _ptr(r), _ptr(q), cols, _ptr(am),
                              _ptr(cnt)), "quantize")
    if r is None:
        r = (1.0 / s.astype(np.float64)).astype(np.float32)
    return q, s, r, am, cnt


def quantize_transpose(x: np.ndarray, fmt: int, gran=(0, 0), mode: int = DYNAMIC,
                       eps: float = 1e-12, pow2: bool = False, scale: np.ndarray | None = None,
                       inv_scale: np.ndarray | None = None):
    """Cast-transpose: returns (codes [rows x cols], codes transposed [cols x rows],
    scale, inv_scale, amax, counts[sat, under])."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    G = (ngroups(rows, gran[0]), ngroups(cols, gran[1]))
    q = np.empty((rows, cols), np.uint8)
    qt = np.empty((cols, rows), np.uint8)
    am = np.empty(G, np.float32)
    cnt = np.zeros(2, np.uint64)
    if mode == DYNAMIC:
        s = np.empty(G, np.float32)
        r = np.empty(G, np.float32)
    else:
        s = np.ascontiguousarray(scale, dtype=np.float32).reshape(G)
        r = None if inv_scale is None else np.ascontiguousarray(inv_scale, np.float32).reshape(G)
    _check(lib().orc_quantize_transpose(_ptr(x), _dtype_code(x), rows, cols, cols, gran[0], gran[1],
                                        fmt, mode, eps, int(pow2), _ptr(s), _ptr(r), _ptr(q), cols,
                                        _ptr(qt), rows, _ptr(am), _ptr(cnt)), "quantize_transpose")
    if r is None:
        r = (1.0 / s.astype(np.float64)).astype(np.float32)
    return q, qt, s, r, am, cnt


def dequantize(q: np.ndarray, fmt: int, scale: np.ndarray, gran=(0, 0), out_dtype: int = F32):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, cols = q.shape
    s = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.empty((rows, cols), np.float32 if out_dtype == F32 else np.uint16)
    _check(lib().orc_dequantize(_ptr(q), fmt, rows, cols, cols, gran[0], gran[1], _ptr(s),
                                _ptr(y), out_dtype, cols), "dequantize")
    return y


def history_update(hist: np.ndarray, head: int, amax_new: float, fmt: int, eps: float = 1e-12,
                   pow2: bool = False):
    """Updates ``hist`` in place; returns (new_head, s_next, r_next)."""
    assert hist.dtype == np.float32 and hist.flags.c_contiguous
    h = C.c_int(head)
    s = np.empty(1, np.float32)
    r = np.empty(1, np.float32)
    _check(lib().orc_history_update(_ptr(hist), hist.size, C.byref(h), float(amax_new), fmt,
                                    eps, int(pow2), _ptr(s), _ptr(r)), "history_update")
    return h.value, s[0], r[0]


def quant_error(w, q, fmt, scale, gran, x=None):
    """Ledger statistics of a quantized weight (binary64): sum e^2, sum w^2,
    max |e|, sum d^2, sum y_ref^2, sum y_q^2, sum y_ref y_q (see the C
    header); x is bf16 bits [M, K] or None."""
    w = np.ascontiguousarray(w)
    q = np.ascontiguousarray(q, np.uint8)
    N, K = w.shape
    assert q.shape == (N, K)
    s = np.ascontiguousarray(scale, np.float32)
    M = 0
    if x is not None:
        x = np.ascontiguousarray(x, np.uint16)
        M = x.shape[0]
        assert x.shape[1] == K
    st = np.empty(7, np.float64)
    _check(lib().orc_quant_error(_ptr(w), _dtype_code(w), N, K, K, _ptr(q), fmt, K, gran[0], gran[1],
                                 _ptr(s), _ptr(x), M, K, _ptr(st)), "quant_error")
    return st


def pack_weights16(q):
    """Fragment-ordered layout of codes q [N, K] (K % 128 == 0): a flat uint8
    array of ceil(N/16) * 16 * K bytes."""
    q = np.ascontiguousarray(q, np.uint8)
    N, K = q.shape
    out = np.empty(((N + 15) // 16) * 16 * K, np.uint8)
    _check(lib().orc_pack_weights16(_ptr(q), N, K, K, _ptr(out)), "pack_weights16")
    return out


HIST_MAX, HIST_LATEST = 0, 1


def history_update_recipe(hist: np.ndarray, head: int, amax_new: float, fmt: int, fn: int = HIST_MAX,
                          margin: int = 0, eps: float = 1e-12, pow2: bool = False):
    """Recipe variant of history_update (history function fn, margin m: the
    scale is derived from f * 2^m).  Updates ``hist`` in place; returns
    (new_head, s_next, r_next)."""
    assert hist.dtype == np.float32 and hist.flags.c_contiguous
    h = C.c_int(head)
    s = np.empty(1, np.float32)
    r = np.empty(1, np.float32)
    _check(lib().orc_history_update_recipe(_ptr(hist), hist.size, C.byref(h), float(amax_new), fmt, fn,
                                           margin, eps, int(pow2), _ptr(s), _ptr(r)),
           "history_update_recipe")
    return h.value, s[0], r[0]


def _gemm_common(a, fa, sa, ga, b, fb, sb, gb, bias):
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    sa = np.ascontiguousarray(sa, np.float32)
    sb = np.ascontiguousarray(sb, np.float32)
    bt = F32
    if bias is not None:
        bias = np.ascontiguousarray(bias)
        bt = _dtype_code(bias)
    return a, b, M, N, K, sa, sb, bias, bt


def gemm_points(a, fa, sa, ga, b, fb, sb, gb, m_idx, n_idx, bias=None):
    """Reference y and S = sum |terms| at points (m_idx[i], n_idx[i]); binary64."""
    a, b, M, N, K, sa, sb, bias, bt = _gemm_common(a, fa, sa, ga, b, fb, sb, gb, bias)
    m_idx = np.ascontiguousarray(m_idx, np.int64)
    n_idx = np.ascontiguousarray(n_idx, np.int64)
    y = np.empty(m_idx.size, np.float64)
    S = np.empty(m_idx.size, np.float64)
    _check(lib().orc_gemm_points(_ptr(a), fa, K, ga[0], ga[1], _ptr(sa), _ptr(b), fb, K, gb[0],
                                 gb[1], _ptr(sb), M, N, K, _ptr(bias), bt, _ptr(m_idx),
                                 _ptr(n_idx), m_idx.size, _ptr(y), _ptr(S)), "gemm_points")
    return y, S


def gemm_points_exact(a, fa, sa, ga, b, fb, sb, gb, m_idx, n_idx, bias=None):
    a, b, M, N, K, sa, sb, bias, bt = _gemm_common(a, fa, sa, ga, b, fb, sb, gb, bias)
    m_idx = np.ascontiguousarray(m_idx, np.int64)
    n_idx = np.ascontiguousarray(n_idx, np.int64)
    y = np.empty(m_idx.size, np.float64)
    _check(lib().orc_gemm_points_exact(_ptr(a), fa, K, ga[0], ga[1], _ptr(sa), _ptr(b), fb, K,
                                       gb[0], gb[1], _ptr(sb), M, N, K, _ptr(bias), bt,
                                       _ptr(m_idx), _ptr(n_idx), m_idx.size, _ptr(y)),
           "gemm_points_exact")
    return y


def wonly_gemm_points(x, w, fw, sw, gw, m_idx, n_idx, bias=None):
    """Weight-only FP8 reference at points (m_idx[i], n_idx[i]):
    y = sum_k x[m,k] s_w(n,k) dec(W[n,k]) + bias[n] and S = sum_k |term|, in
    binary64.  x: [M, K] float32 or bf16 bits (uint16); w: [N, K] codes."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w, np.uint8)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    sw = np.ascontiguousarray(sw, np.float32)
    bt = F32
    if bias is not None:
        bias = np.ascontiguousarray(bias)
        bt = _dtype_code(bias)
    m_idx = np.ascontiguousarray(m_idx, np.int64)
    n_idx = np.ascontiguousarray(n_idx, np.int64)
    y = np.empty(m_idx.size, np.float64)
    S = np.empty(m_idx.size, np.float64)
    _check(lib().orc_wonly_gemm_points(_ptr(x), _dtype_code(x), K, _ptr(w), fw, K, gw[0], gw[1],
                                       _ptr(sw), M, N, K, _ptr(bias), bt, _ptr(m_idx), _ptr(n_idx),
                                       m_idx.size, _ptr(y), _ptr(S)), "wonly_gemm_points")
    return y, S


def wonly_gemm_full(x, w, fw, sw, gw, bias=None):
    """Every output point of the weight-only GEMM; (y [M,N], S [M,N])."""
    M, N = x.shape[0], w.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, S = wonly_gemm_points(x, w, fw, sw, gw, mm.ravel(), nn.ravel(), bias)
    return y.reshape(M, N), S.reshape(M, N)


def gemm_full(a, fa, sa, ga, b, fb, sb, gb, bias=None):
    """Every output point; returns (y [M,N], S [M,N]) in binary64."""
    M, N = a.shape[0], b.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, S = gemm_points(a, fa, sa, ga, b, fb, sb, gb, mm.ravel(), nn.ravel(), bias)
    return y.reshape(M, N), S.reshape(M, N)


def dot_truncation_bound(a, fa, sa, ga, b, fb, sb, gb, m_idx, n_idx):
    """Tolerance term for the matrix-core FP8 dot product (see fp8_dot_bound.c)."""
    a, b, M, N, K, sa, sb, _, _ = _gemm_common(a, fa, sa, ga, b, fb, sb, gb, None)
    m_idx = np.ascontiguousarray(m_idx, np.int64)
    n_idx = np.ascontiguousarray(n_idx, np.int64)
    out = np.empty(m_idx.size, np.float64)
    _check(lib().orc_dot_truncation_bound(_ptr(a), fa, K, ga[0], ga[1], _ptr(sa), _ptr(b), fb, K,
                                          gb[0], gb[1], _ptr(sb), M, N, K, _ptr(m_idx),
                                          _ptr(n_idx), m_idx.size, _ptr(out)),
           "dot_truncation_bound")
    return out


def dot_truncation_bound_full(a, fa, sa, ga, b, fb, sb, gb):
    M, N = a.shape[0], b.shape[0]
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return dot_truncation_bound(a, fa, sa, ga, b, fb, sb, gb, mm.ravel(), nn.ravel()).reshape(M, N)


def round_bf16(v) -> np.ndarray:
    """binary64 -> bf16 bits (nearest even), elementwise."""
    f = np.vectorize(lambda t: lib().orc_round_bf16(float(t)), otypes=[np.uint16])
    return f(np.asarray(v, np.float64))


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)
