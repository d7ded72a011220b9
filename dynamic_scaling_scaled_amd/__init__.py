"""Python binding of the gfx950 FP8 runtime chain (``libfp8rt.so``).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI of ``include/fp8rt.h`` and raises on a
non-OK status.  All arithmetic runs in the library's HIP kernels; there is no
CPU fallback: calling any function without the built library raises.

Tensors are torch tensors on the GPU: inputs ``float32`` or ``bfloat16``,
FP8 codes ``uint8``, scales ``float32``, counters ``int64`` (read as uint64).
Granularities are ``(rows, cols)`` group extents, 0 meaning the whole
dimension: per-tensor (0, 0), per-row (1, 0), per-group (1, 128),
per-block (128, 128), MX-style (1, 32).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8rt.so")
# FP8RT_LIB names another build of this library to load instead (the
# host-sanitized build of the CPU checks); there is no fallback either way.
if os.environ.get("FP8RT_LIB"):
    LIB_PATH = os.environ["FP8RT_LIB"]

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
DYNAMIC, GIVEN = 0, 1
POW2_SCALES = 1
B_PACKED16 = 2
EXACT_PRODUCTS = 4
EXACT_AUTO_BYTES = 1 << 20
FMAX = {E4M3: 448.0, E5M2: 57344.0}

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP, ESCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 16 << 20


class Fp8rtError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


class Gran(C.Structure):
    _fields_ = [("rows", C.c_int32), ("cols", C.c_int32)]


class LedgerSpec(C.Structure):
    _fields_ = [("gran", Gran), ("pow2_round_up", C.c_int32)]


class LedgerRow(C.Structure):
    _fields_ = [("gran", Gran), ("pow2_round_up", C.c_int32), ("qparam_count", C.c_int64),
                ("qparam_bytes", C.c_int64), ("quantized_weight_bytes", C.c_int64),
                ("total_state_bytes", C.c_int64), ("weight_mse", C.c_double),
                ("weight_max_abs_err", C.c_double), ("output_mse", C.c_double),
                ("output_cosine", C.c_double), ("saturated", C.c_uint64), ("underflowed", C.c_uint64)]


_lib = None


def lib():
    """Load the built library; raises if it is missing (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libfp8rt.so is not built: run __graft_entry__.build() "
                              "or python dynamic_scaling_scaled_amd/_build.py")
        L = C.CDLL(LIB_PATH)
        P, I64, I32, F, U32 = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_uint32
        L.fp8rt_status_string.restype = C.c_char_p
        L.fp8rt_status_string.argtypes = [C.c_int]
        L.fp8_amax.restype = C.c_int
        L.fp8_amax.argtypes = [P, C.c_int, I64, I64, I64, Gran, P, P]
        L.fp8_compute_scale.restype = C.c_int
        L.fp8_compute_scale.argtypes = [P, I64, C.c_int, F, I32, P, P, P]
        L.fp8_quantize.restype = C.c_int
        L.fp8_quantize.argtypes = [P, C.c_int, I64, I64, I64, Gran, C.c_int, C.c_int, F, I32, P, P,
                                   P, I64, P, P, P]
        L.fp8_quantize_transpose.restype = C.c_int
        L.fp8_quantize_transpose.argtypes = [P, C.c_int, I64, I64, I64, Gran, C.c_int, C.c_int, F, I32,
                                             P, P, P, I64, P, I64, P, P, P]
        L.fp8_dequantize.restype = C.c_int
        L.fp8_dequantize.argtypes = [P, C.c_int, I64, I64, I64, Gran, P, P, C.c_int, I64, P]
        L.fp8_amax_history_update.restype = C.c_int
        L.fp8_amax_history_update.argtypes = [P, I32, P, P, C.c_int, F, I32, P, P, P]
        L.fp8_scaled_gemm.restype = C.c_int
        L.fp8_scaled_gemm.argtypes = [P, C.c_int, I64, Gran, P, P, C.c_int, I64, Gran, P, I64, I64,
                                      I64, P, C.c_int, P, C.c_int, I64, U32, P]
        L.fp8_scaled_gemm_noalloc.restype = C.c_int
        L.fp8_scaled_gemm_noalloc.argtypes = L.fp8_scaled_gemm.argtypes
        L.fp8_quant_error.restype = C.c_int
        L.fp8_quant_error.argtypes = [P, C.c_int, I64, I64, I64, P, C.c_int, I64, Gran, P, P, I64, I64, P, P]
        L.fp8_granularity_ledger.restype = C.c_int
        L.fp8_granularity_ledger.argtypes = [P, C.c_int, I64, I64, I64, P, I64, I64, C.c_int, F,
                                             C.POINTER(LedgerSpec), I32, C.POINTER(LedgerRow), P]
        L.fp8_delayed_scale_update.restype = C.c_int
        L.fp8_delayed_scale_update.argtypes = [P, I32, P, P, C.c_int, C.c_int, I32, F, I32, P, P, P]
        L.fp8_weight_only_gemm.restype = C.c_int
        L.fp8_weight_only_gemm.argtypes = [P, C.c_int, I64, P, C.c_int, I64, Gran, P, I64, I64, I64, P,
                                           C.c_int, P, C.c_int, I64, U32, P]
        L.fp8_pack_weights16.restype = C.c_int
        L.fp8_pack_weights16.argtypes = [P, I64, I64, I64, P, P]
        L.fp8_quantize_packed16.restype = C.c_int
        L.fp8_quantize_packed16.argtypes = [P, C.c_int, I64, I64, I64, Gran, C.c_int, C.c_int, F, I32, P, P,
                                            P, P, P, P]
        L.fp8_scaled_gemm_fp8out.restype = C.c_int
        L.fp8_scaled_gemm_fp8out.argtypes = [P, C.c_int, I64, Gran, P, P, C.c_int, I64, Gran, P, I64, I64,
                                             I64, P, C.c_int, C.c_int, P, P, P, I64, P, P, U32, P]
        _lib = L
    return _lib


def _check(fn, status):
    if status != OK:
        raise Fp8rtError(fn, status, lib().fp8rt_status_string(status).decode())


def _ptr(t):
    # a plain int: the c_void_p argtypes convert it, no object per argument
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:  # the current stream's handle, without a Stream object
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _mat(t: torch.Tensor):
    st = t.stride()
    if len(st) != 2 or st[1] != 1:
        raise ValueError("expected a 2-D row-major tensor with unit column stride")
    rows, cols = t.shape
    return rows, cols, st[0]


def ngroups(n: int, g: int) -> int:
    return 1 if (g <= 0 or g >= n) else -(-n // g)


def scale_shape(shape, gran):
    return (ngroups(shape[0], gran[0]), ngroups(shape[1], gran[1]))


def fp8_amax(x, gran, amax, stream=None):
    rows, cols, ld = _mat(x)
    _check("fp8_amax", lib().fp8_amax(_ptr(x), _dtype(x), rows, cols, ld, Gran(*gran), _ptr(amax),
                                      _stream(stream)))


def fp8_compute_scale(amax, fmt, eps, pow2_round_up, scale, inv_scale=None, stream=None):
    _check("fp8_compute_scale", lib().fp8_compute_scale(_ptr(amax), amax.numel(), fmt, eps,
                                                        int(pow2_round_up), _ptr(scale),
                                                        _ptr(inv_scale), _stream(stream)))


def fp8_quantize(x, gran, fmt, mode, eps, pow2_round_up, scale, inv_scale, q, amax_out=None,
                 sat_underflow=None, stream=None):
    rows, cols, ld = _mat(x)
    _, _, ldq = _mat(q)
    _check("fp8_quantize", lib().fp8_quantize(_ptr(x), _dtype(x), rows, cols, ld, Gran(*gran), fmt,
                                              mode, eps, int(pow2_round_up), _ptr(scale),
                                              _ptr(inv_scale), _ptr(q), ldq, _ptr(amax_out),
                                              _ptr(sat_underflow), _stream(stream)))


def fp8_quantize_transpose(x, gran, fmt, mode, eps, pow2_round_up, scale, inv_scale, q, qt,
                           amax_out=None, sat_underflow=None, stream=None):
    rows, cols, ld = _mat(x)
    _, _, ldq = _mat(q)
    qr, qc, ldqt = _mat(qt)
    if (qr, qc) != (cols, rows):
        raise ValueError("qt must be [cols x rows]")
    _check("fp8_quantize_transpose",
           lib().fp8_quantize_transpose(_ptr(x), _dtype(x), rows, cols, ld, Gran(*gran), fmt, mode, eps,
                                        int(pow2_round_up), _ptr(scale), _ptr(inv_scale), _ptr(q), ldq,
                                        _ptr(qt), ldqt, _ptr(amax_out), _ptr(sat_underflow),
                                        _stream(stream)))


def fp8_dequantize(q, fmt, gran, scale, y, stream=None):
    rows, cols, ldq = _mat(q)
    _, _, ldy = _mat(y)
    _check("fp8_dequantize", lib().fp8_dequantize(_ptr(q), fmt, rows, cols, ldq, Gran(*gran),
                                                  _ptr(scale), _ptr(y), _dtype(y), ldy,
                                                  _stream(stream)))


def fp8_amax_history_update(history, head, amax_new, fmt, eps, pow2_round_up, scale_next,
                            inv_scale_next=None, stream=None):
    _check("fp8_amax_history_update",
           lib().fp8_amax_history_update(_ptr(history), history.numel(), _ptr(head), _ptr(amax_new),
                                         fmt, eps, int(pow2_round_up), _ptr(scale_next),
                                         _ptr(inv_scale_next), _stream(stream)))


class PackedWeights:
    """A fragment-ordered weight image (fp8_pack_weights16): the uint8 device
    tensor `data` and the logical shape [N x K] of the codes it holds."""

    def __init__(self, data, N, K):
        self.data, self.N, self.K = data, int(N), int(K)

    def data_ptr(self):
        return self.data.data_ptr()


def packed16_bytes(N, K):
    return (N + 15) // 16 * 16 * K


def fp8_pack_weights16(q, out=None, stream=None):
    """Fragment-ordered image of row-major codes q [N x K] (K % 128 == 0)."""
    if q.dtype != torch.uint8:
        raise ValueError("q must be uint8 codes")
    N, K, ldq = _mat(q)
    if out is None:
        out = torch.empty(packed16_bytes(N, K), dtype=torch.uint8, device=q.device)
    if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < packed16_bytes(N, K):
        raise ValueError("out must be contiguous uint8 with packed16_bytes(N, K) bytes")
    _check("fp8_pack_weights16", lib().fp8_pack_weights16(_ptr(q), N, K, ldq, _ptr(out), _stream(stream)))
    return PackedWeights(out, N, K)


def fp8_quantize_packed16(x, gran, fmt, mode, eps, pow2_round_up, scale, inv_scale, out=None, amax_out=None,
                          sat_underflow=None, stream=None):
    """fp8_quantize of x [N x K] with the codes written straight into the
    fragment-ordered weight image (K % 128 == 0); returns PackedWeights."""
    rows, cols, ld = _mat(x)
    if out is None:
        out = torch.empty(packed16_bytes(rows, cols), dtype=torch.uint8, device=x.device)
    if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < packed16_bytes(rows, cols):
        raise ValueError("out must be contiguous uint8 with packed16_bytes(N, K) bytes")
    _check("fp8_quantize_packed16",
           lib().fp8_quantize_packed16(_ptr(x), _dtype(x), rows, cols, ld, Gran(*gran), fmt, mode, eps,
                                       int(pow2_round_up), _ptr(scale), _ptr(inv_scale), _ptr(out),
                                       _ptr(amax_out), _ptr(sat_underflow), _stream(stream)))
    return PackedWeights(out, rows, cols)


def _weight(b, flags):
    """(N, K, ld, flags) of a row-major code matrix or a PackedWeights."""
    if isinstance(b, PackedWeights):
        return b.N, b.K, b.K, flags | B_PACKED16
    N, K, ld = _mat(b)
    return N, K, ld, flags


def fp8_scaled_gemm(a, fa, ga, scale_a, b, fb, gb, scale_b, y, bias=None, flags=0, stream=None):
    M, K, lda = _mat(a)
    N, K2, ldb, flags = _weight(b, flags)
    if K2 != K:
        raise ValueError("A and B disagree on K")
    _, _, ldy = _mat(y)
    bias_t = _dtype(bias) if bias is not None else F32
    _check("fp8_scaled_gemm",
           lib().fp8_scaled_gemm(_ptr(a), fa, lda, Gran(*ga), _ptr(scale_a), _ptr(b), fb, ldb,
                                 Gran(*gb), _ptr(scale_b), M, N, K, _ptr(bias), bias_t, _ptr(y),
                                 _dtype(y), ldy, flags, _stream(stream)))


def fp8_scaled_gemm_noalloc(a, fa, ga, scale_a, b, fb, gb, scale_b, y, bias=None, flags=0, stream=None):
    """fp8_scaled_gemm on the library's fixed device scratch: allocates nothing."""
    M, K, lda = _mat(a)
    N, K2, ldb, flags = _weight(b, flags)
    if K2 != K:
        raise ValueError("A and B disagree on K")
    _, _, ldy = _mat(y)
    bias_t = _dtype(bias) if bias is not None else F32
    _check("fp8_scaled_gemm_noalloc",
           lib().fp8_scaled_gemm_noalloc(_ptr(a), fa, lda, Gran(*ga), _ptr(scale_a), _ptr(b), fb, ldb,
                                         Gran(*gb), _ptr(scale_b), M, N, K, _ptr(bias), bias_t, _ptr(y),
                                         _dtype(y), ldy, flags, _stream(stream)))


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments; returns the status."""
    return getattr(lib(), name)(*args)


def fp8_scaled_gemm_fp8out(a, fa, ga, scale_a, b, fb, gb, scale_b, yq, fy, scale_y, inv_scale_y=None,
                           amax_y=None, sat_underflow=None, bias=None, flags=0, stream=None):
    M, K, lda = _mat(a)
    N, K2, ldb, flags = _weight(b, flags)
    if K2 != K:
        raise ValueError("A and B disagree on K")
    My, Ny, ldy = _mat(yq)
    if (My, Ny) != (M, N) or yq.dtype != torch.uint8:
        raise ValueError("yq must be uint8 [M x N]")
    bt = F32 if bias is None else _dtype(bias)
    _check("fp8_scaled_gemm_fp8out",
           lib().fp8_scaled_gemm_fp8out(_ptr(a), fa, lda, Gran(*ga), _ptr(scale_a), _ptr(b), fb, ldb, Gran(*gb),
                                        _ptr(scale_b), M, N, K, _ptr(bias), bt, fy, _ptr(scale_y),
                                        _ptr(inv_scale_y), _ptr(yq), ldy, _ptr(amax_y), _ptr(sat_underflow),
                                        flags, _stream(stream)))


HIST_MAX, HIST_LATEST = 0, 1


def fp8_quant_error(w, q, fmt, gran, scale, stats, x=None, stream=None):
    """stats (float64[7] on the device) <- the quantization error sums of w
    restored from (q, scale); x: optional bf16 inputs [M, K]."""
    N, K, ldw = _mat(w)
    Nq, Kq, ldq = _mat(q)
    if (Nq, Kq) != (N, K) or q.dtype != torch.uint8:
        raise ValueError("q must be uint8 [N x K]")
    if stats.dtype != torch.float64 or stats.numel() < 7:
        raise ValueError("stats must be float64 with 7 entries")
    M, ldx = 0, 0
    if x is not None:
        M, Kx, ldx = _mat(x)
        if Kx != K:
            raise ValueError("x and w disagree on K")
    _check("fp8_quant_error",
           lib().fp8_quant_error(_ptr(w), _dtype(w), N, K, ldw, _ptr(q), fmt, ldq, Gran(*gran), _ptr(scale),
                                 _ptr(x), M, ldx, _ptr(stats), _stream(stream)))


def fp8_granularity_ledger(w, fmt, specs, x=None, eps=1e-12, stream=None):
    """Quantizes w at each (gran, pow2) spec and returns the ledger rows as
    dicts (scale count and bytes, weight / output error, counters)."""
    N, K, ldw = _mat(w)
    M, ldx = 0, 0
    if x is not None:
        M, Kx, ldx = _mat(x)
        if Kx != K:
            raise ValueError("x and w disagree on K")
    sp = (LedgerSpec * len(specs))(*[LedgerSpec(Gran(*g), int(p)) for g, p in specs])
    rows = (LedgerRow * len(specs))()
    _check("fp8_granularity_ledger",
           lib().fp8_granularity_ledger(_ptr(w), _dtype(w), N, K, ldw, _ptr(x), M, ldx, fmt, eps, sp, len(specs),
                                        rows, _stream(stream)))
    out = []
    for r in rows:
        d = {k: getattr(r, k) for k, _ in LedgerRow._fields_ if k != "gran"}
        d["gran"] = (r.gran.rows, r.gran.cols)
        out.append(d)
    return out


def fp8_delayed_scale_update(history, head, amax_new, fmt, fn, margin, eps, pow2, scale_next,
                             inv_scale_next=None, stream=None):
    """Delayed-scaling recipe step: push amax_new into the ring, derive the
    next (s, r) from f * 2^margin (f = window max or latest amax)."""
    if history.dtype != torch.float32 or history.dim() != 1 or not history.is_contiguous():
        raise ValueError("history must be a contiguous float32 vector")
    _check("fp8_delayed_scale_update",
           lib().fp8_delayed_scale_update(_ptr(history), history.numel(), _ptr(head), _ptr(amax_new), fmt, fn,
                                          margin, eps, int(pow2), _ptr(scale_next), _ptr(inv_scale_next),
                                          _stream(stream)))


def fp8_weight_only_gemm(x, w, fw, gw, scale_w, y, bias=None, flags=0, stream=None):
    """y = x (s_w o dec(w))^T + bias: x [M, K] bf16, w [N, K] uint8 codes or
    their PackedWeights image."""
    M, K, ldx = _mat(x)
    N, K2, ldw, flags = _weight(w, flags)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    _, _, ldy = _mat(y)
    bt = F32 if bias is None else _dtype(bias)
    _check("fp8_weight_only_gemm",
           lib().fp8_weight_only_gemm(_ptr(x), _dtype(x), ldx, _ptr(w), fw, ldw, Gran(*gw), _ptr(scale_w),
                                      M, N, K, _ptr(bias), bt, _ptr(y), _dtype(y), ldy, flags,
                                      _stream(stream)))


__all__ = ["fp8_pack_weights16", "fp8_quantize_packed16", "PackedWeights", "packed16_bytes", "B_PACKED16", "fp8_quant_error", "fp8_granularity_ledger", "LedgerSpec", "LedgerRow", "fp8_delayed_scale_update", "HIST_MAX", "HIST_LATEST", "fp8_weight_only_gemm", "fp8_scaled_gemm_fp8out", "fp8_amax", "fp8_compute_scale", "fp8_quantize", "fp8_quantize_transpose", "fp8_dequantize",
           "fp8_amax_history_update", "fp8_scaled_gemm", "lib", "raw_call", "Gran", "Fp8rtError",
           "E4M3", "E5M2", "F32", "BF16", "DYNAMIC", "GIVEN", "POW2_SCALES", "EXACT_PRODUCTS", "EXACT_AUTO_BYTES", "FMAX", "ngroups",
           "scale_shape"]
