"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects bad arguments with the
documented status before anything is launched.  Every call here is invalid on
purpose, so none of them reaches a kernel."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8rt.h")


@pytest.fixture(scope="module")
def rt():
    import dynamic_scaling_scaled_amd as rt
    if not os.path.exists(rt.LIB_PATH):
        from dynamic_scaling_scaled_amd import _build
        _build.build()
    rt.lib()
    return rt


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:fp8rt_status|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for n in ("fp8_amax", "fp8_compute_scale", "fp8_quantize", "fp8_dequantize",
              "fp8_amax_history_update", "fp8_scaled_gemm", "fp8rt_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(rt):
    L = rt.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(rt):
    L = rt.lib()
    for s in range(5):
        assert len(L.fp8rt_status_string(s)) > 0


FAKE = 0x10000  # never dereferenced: every call below fails validation first
FAKE_ODD = 0x10004


def q(rt, **kw):
    a = dict(x=FAKE, xt=rt.BF16, rows=16, cols=64, ldx=64, gran=(0, 0), f=rt.E4M3, mode=rt.DYNAMIC,
             eps=1e-12, pow2=0, scale=FAKE, inv=None, qq=FAKE, ldq=64, amax=None, cnt=None)
    a.update(kw)
    return rt.lib().fp8_quantize(a["x"], a["xt"], a["rows"], a["cols"], a["ldx"], rt.Gran(*a["gran"]),
                                 a["f"], a["mode"], a["eps"], a["pow2"], a["scale"], a["inv"],
                                 a["qq"], a["ldq"], a["amax"], a["cnt"], None)


def test_quantize_validation(rt):
    assert q(rt, x=None) == rt.EINVAL
    assert q(rt, qq=None) == rt.EINVAL
    assert q(rt, scale=None) == rt.EINVAL
    assert q(rt, rows=0) == rt.EINVAL
    assert q(rt, cols=-16) == rt.EINVAL
    assert q(rt, ldx=48) == rt.EINVAL
    assert q(rt, ldq=32) == rt.EINVAL
    assert q(rt, eps=0.0) == rt.EINVAL
    assert q(rt, eps=float("nan")) == rt.EINVAL
    assert q(rt, eps=1e-35) == rt.EINVAL
    assert q(rt, f=2) == rt.EINVAL
    assert q(rt, xt=7) == rt.EINVAL
    assert q(rt, mode=5) == rt.EINVAL
    assert q(rt, gran=(-1, 0)) == rt.EINVAL
    assert q(rt, cols=40, ldx=48, ldq=48) == rt.EALIGN
    assert q(rt, ldx=72) == rt.EALIGN
    assert q(rt, ldq=72) == rt.EALIGN
    assert q(rt, gran=(1, 24)) == rt.EALIGN
    assert q(rt, x=FAKE + 8) == rt.EALIGN
    assert q(rt, qq=FAKE + 4) == rt.EALIGN
    assert q(rt, scale=FAKE + 2) == rt.EALIGN
    assert q(rt, cnt=FAKE_ODD) == rt.EALIGN


def test_amax_scale_dequant_history_validation(rt):
    L = rt.lib()
    G = rt.Gran
    assert L.fp8_amax(None, 1, 16, 64, 64, G(0, 0), FAKE, None) == rt.EINVAL
    assert L.fp8_amax(FAKE, 1, 16, 64, 64, G(0, 0), None, None) == rt.EINVAL
    assert L.fp8_amax(FAKE, 1, 16, 60, 64, G(0, 0), FAKE, None) == rt.EALIGN
    assert L.fp8_compute_scale(FAKE, 0, 0, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_compute_scale(FAKE, 4, 0, -1.0, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_compute_scale(FAKE, 4, 3, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_compute_scale(FAKE + 1, 4, 0, 1e-12, 0, FAKE, None, None) == rt.EALIGN
    assert L.fp8_dequantize(FAKE, 0, 16, 64, 64, G(0, 0), FAKE, None, 0, 64, None) == rt.EINVAL
    assert L.fp8_dequantize(FAKE, 0, 16, 64, 64, G(0, 0), FAKE, FAKE, 0, 32, None) == rt.EINVAL
    assert L.fp8_dequantize(FAKE, 0, 16, 64, 64, G(0, 0), FAKE, FAKE + 8, 0, 64, None) == rt.EALIGN
    assert L.fp8_amax_history_update(FAKE, 0, FAKE, FAKE, 0, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_amax_history_update(FAKE, 2000, FAKE, FAKE, 0, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_amax_history_update(None, 16, FAKE, FAKE, 0, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_amax_history_update(FAKE, 16, None, FAKE, 0, 1e-12, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_amax_history_update(FAKE, 16, FAKE, FAKE, 0, 0.0, 0, FAKE, None, None) == rt.EINVAL
    assert L.fp8_amax_history_update(FAKE + 2, 16, FAKE, FAKE, 0, 1e-12, 0, FAKE, None, None) == rt.EALIGN


def g(rt, fn="fp8_scaled_gemm", **kw):
    a = dict(a=FAKE, fa=rt.E4M3, lda=128, ga=(0, 0), sa=FAKE, b=FAKE, fb=rt.E4M3, ldb=128, gb=(0, 0),
             sb=FAKE, M=64, N=64, K=128, bias=None, bt=0, y=FAKE, yt=rt.BF16, ldy=64, flags=0)
    a.update(kw)
    return getattr(rt.lib(), fn)(a["a"], a["fa"], a["lda"], rt.Gran(*a["ga"]), a["sa"], a["b"],
                                    a["fb"], a["ldb"], rt.Gran(*a["gb"]), a["sb"], a["M"], a["N"],
                                    a["K"], a["bias"], a["bt"], a["y"], a["yt"], a["ldy"],
                                    a["flags"], None)


@pytest.mark.parametrize("fn", ["fp8_scaled_gemm", "fp8_scaled_gemm_noalloc"])
def test_gemm_validation(rt, fn):
    g = lambda rt, **kw: globals()["g"](rt, fn, **kw)
    assert g(rt, a=None) == rt.EINVAL
    assert g(rt, sb=None) == rt.EINVAL
    assert g(rt, y=None) == rt.EINVAL
    assert g(rt, M=0) == rt.EINVAL
    assert g(rt, lda=64) == rt.EINVAL
    assert g(rt, ldy=32) == rt.EINVAL
    assert g(rt, flags=8) == rt.EINVAL
    assert g(rt, flags=15) == rt.EINVAL
    assert g(rt, fa=9) == rt.EINVAL
    assert g(rt, K=120, lda=128, ldb=128) == rt.EALIGN
    assert g(rt, lda=136) == rt.EALIGN
    assert g(rt, a=FAKE + 8) == rt.EALIGN
    assert g(rt, fb=rt.E5M2) == rt.EUNSUPPORTED                       # E4M3 x E5M2 not built
    assert g(rt, fa=rt.E5M2, fb=rt.E5M2) == rt.EUNSUPPORTED
    assert g(rt, K=512, lda=512, ldb=512, ga=(1, 128), gb=(128, 256)) == rt.EUNSUPPORTED  # K-blocks differ
    assert g(rt, K=256, lda=256, ldb=256, ga=(1, 64), gb=(0, 0)) == rt.EUNSUPPORTED       # not a multiple of 128
    assert g(rt, K=256, lda=256, ldb=256, ga=(1, 32), gb=(1, 32)) == rt.EUNSUPPORTED      # 1x32 needs POW2 flag
    assert g(rt, K=256, lda=256, ldb=256, ga=(2, 128), gb=(0, 0)) == rt.EUNSUPPORTED      # A blocks span rows
    # the packed weight image: decode shapes only
    assert g(rt, flags=10) == rt.EINVAL
    assert g(rt, flags=rt.B_PACKED16, M=80, ldy=64) == rt.EUNSUPPORTED                    # M = 80 > 64
    assert g(rt, flags=rt.B_PACKED16, M=16, K=144, lda=144, ldb=144) == rt.EUNSUPPORTED  # K % 128
    assert g(rt, flags=rt.B_PACKED16 | rt.POW2_SCALES, K=256, lda=256, ldb=256, ga=(1, 32),
             gb=(1, 32)) == rt.EUNSUPPORTED                                               # 1x32 scales
    assert g(rt, flags=rt.B_PACKED16, M=8, lda=64) == rt.EINVAL                           # lda < K still checked
    # exact products: decode shapes only, row-major or packed
    X = rt.EXACT_PRODUCTS
    assert g(rt, flags=X, M=80, ldy=64) == rt.EUNSUPPORTED                                # M = 80 > 64
    assert g(rt, flags=X, M=16, K=144, lda=144, ldb=144) == rt.EUNSUPPORTED              # K % 128
    assert g(rt, flags=X | rt.B_PACKED16, M=65, ldy=64) == rt.EUNSUPPORTED
    assert g(rt, flags=X | rt.POW2_SCALES, K=256, lda=256, ldb=256, ga=(1, 32), gb=(1, 32)) == rt.EUNSUPPORTED


def qtr(rt, **kw):
    a = dict(x=FAKE, xt=rt.BF16, rows=32, cols=64, ldx=64, gran=(0, 0), f=rt.E4M3, mode=rt.DYNAMIC,
             eps=1e-12, pow2=0, scale=FAKE, inv=None, qq=FAKE, ldq=64, qt=FAKE, ldqt=32, amax=None,
             cnt=None)
    a.update(kw)
    return rt.lib().fp8_quantize_transpose(a["x"], a["xt"], a["rows"], a["cols"], a["ldx"],
                                           rt.Gran(*a["gran"]), a["f"], a["mode"], a["eps"], a["pow2"],
                                           a["scale"], a["inv"], a["qq"], a["ldq"], a["qt"], a["ldqt"],
                                           a["amax"], a["cnt"], None)


def test_quantize_transpose_validation(rt):
    assert qtr(rt, qt=None) == rt.EINVAL
    assert qtr(rt, x=None) == rt.EINVAL
    assert qtr(rt, ldqt=16) == rt.EINVAL          # ldqt < rows
    assert qtr(rt, rows=24, ldqt=32) == rt.EALIGN  # rows not a multiple of 16
    assert qtr(rt, ldqt=40) == rt.EALIGN
    assert qtr(rt, qt=FAKE_ODD) == rt.EALIGN
    assert qtr(rt, gran=(1, 32)) == rt.EUNSUPPORTED
    assert qtr(rt, gran=(16, 16)) == rt.EUNSUPPORTED
    assert qtr(rt, mode=rt.DYNAMIC, eps=float("nan")) == rt.EINVAL


def test_gemm_fp8out_validation(rt):
    L = rt.lib()
    G = rt.Gran

    def call(**kw):
        a = dict(a=FAKE, lda=64, sa=FAKE, b=FAKE, ldb=64, sb=FAKE, M=32, N=32, K=64, fy=rt.E4M3, sy=FAKE,
                 yq=FAKE, ldy=32, flags=0)
        a.update(kw)
        return L.fp8_scaled_gemm_fp8out(a["a"], rt.E4M3, a["lda"], G(0, 0), a["sa"], a["b"], rt.E4M3, a["ldb"],
                                        G(0, 0), a["sb"], a["M"], a["N"], a["K"], None, rt.F32, a["fy"], a["sy"],
                                        None, a["yq"], a["ldy"], None, None, a["flags"], None)
    assert call(yq=None) == rt.EINVAL
    assert call(sy=None) == rt.EINVAL
    assert call(fy=7) == rt.EINVAL
    assert call(ldy=16) == rt.EINVAL
    assert call(K=48, lda=48, ldb=48) == rt.EALIGN or call(K=40, lda=48, ldb=48) == rt.EALIGN
    assert call(sy=FAKE + 2) == rt.EALIGN
    assert call(M=128 * 8193, N=128, ldy=128) == rt.EUNSUPPORTED
    assert call(flags=rt.B_PACKED16) == rt.EUNSUPPORTED      # the image needs K a multiple of 128
    assert call(flags=rt.B_PACKED16, M=16, N=16 * 8193, K=128, lda=128, ldb=128, ldy=16 * 8193) == rt.EUNSUPPORTED
    assert call(flags=rt.EXACT_PRODUCTS) == rt.EUNSUPPORTED  # FP8 matrix cores only


def test_weight_only_gemm_validation(rt):
    L = rt.lib()
    G = rt.Gran

    def call(**kw):
        a = dict(x=FAKE, xt=rt.BF16, ldx=256, w=FAKE, fw=rt.E4M3, ldw=256, gw=(1, 0), sw=FAKE, M=16, N=64,
                 K=256, bias=None, bt=rt.F32, y=FAKE, yt=rt.BF16, ldy=64, flags=0)
        a.update(kw)
        return L.fp8_weight_only_gemm(a["x"], a["xt"], a["ldx"], a["w"], a["fw"], a["ldw"], G(*a["gw"]), a["sw"],
                                      a["M"], a["N"], a["K"], a["bias"], a["bt"], a["y"], a["yt"], a["ldy"],
                                      a["flags"], None)
    assert call(x=None) == rt.EINVAL
    assert call(w=None) == rt.EINVAL
    assert call(sw=None) == rt.EINVAL
    assert call(y=None) == rt.EINVAL
    assert call(fw=5) == rt.EINVAL
    assert call(yt=9) == rt.EINVAL
    assert call(M=0) == rt.EINVAL
    assert call(ldx=128) == rt.EINVAL            # ldx < K
    assert call(ldy=32) == rt.EINVAL             # ldy < N
    assert call(gw=(-1, 0)) == rt.EINVAL
    assert call(M=16 * 65536) == rt.EINVAL
    assert call(xt=rt.F32) == rt.EUNSUPPORTED    # activations stay bf16
    assert call(K=248, ldx=248, ldw=256) == rt.EALIGN
    assert call(ldx=260) == rt.EALIGN            # 520-byte rows
    assert call(ldw=264) == rt.EALIGN
    assert call(x=FAKE + 8) == rt.EALIGN
    assert call(sw=FAKE + 2) == rt.EALIGN
    assert call(gw=(1, 64)) == rt.EUNSUPPORTED   # K groups are whole 128-deep steps
    assert call(gw=(1, 192)) == rt.EUNSUPPORTED
    assert call(flags=1) == rt.EINVAL                                       # POW2 means nothing here
    assert call(flags=4) == rt.EINVAL                                       # products are exact already
    assert call(flags=rt.B_PACKED16, K=144, ldx=144, ldw=144) == rt.EALIGN  # packed: K % 128
    assert call(flags=rt.B_PACKED16, K=144, ldx=144, ldw=0) == rt.EALIGN    # ldw ignored, K still checked


def test_pack_weights16_validation(rt):
    L = rt.lib()

    def call(**kw):
        a = dict(q=FAKE, N=64, K=256, ldq=256, qp=FAKE)
        a.update(kw)
        return L.fp8_pack_weights16(a["q"], a["N"], a["K"], a["ldq"], a["qp"], None)
    assert call(q=None) == rt.EINVAL
    assert call(qp=None) == rt.EINVAL
    assert call(N=0) == rt.EINVAL
    assert call(K=0) == rt.EINVAL
    assert call(ldq=128) == rt.EINVAL
    assert call(N=2 ** 31 + 1) == rt.EINVAL
    assert call(K=144, ldq=144) == rt.EALIGN
    assert call(ldq=264) == rt.EALIGN
    assert call(q=FAKE + 8) == rt.EALIGN
    assert call(qp=FAKE + 8) == rt.EALIGN
    assert rt.packed16_bytes(17, 256) == 32 * 256 and rt.packed16_bytes(16, 128) == 2048


def test_quantize_packed16_validation(rt):
    """fp8_quantize's checks, plus K a multiple of 128 and the pack's size limits."""
    L = rt.lib()

    def call(**kw):
        a = dict(x=FAKE, xt=rt.BF16, rows=16, cols=256, ldx=256, gran=(1, 0), f=rt.E4M3, mode=rt.DYNAMIC,
                 eps=1e-12, pow2=0, scale=FAKE, inv=None, qp=FAKE, amax=None, cnt=None)
        a.update(kw)
        return L.fp8_quantize_packed16(a["x"], a["xt"], a["rows"], a["cols"], a["ldx"], rt.Gran(*a["gran"]),
                                       a["f"], a["mode"], a["eps"], a["pow2"], a["scale"], a["inv"], a["qp"],
                                       a["amax"], a["cnt"], None)
    assert call(x=None) == rt.EINVAL
    assert call(qp=None) == rt.EINVAL
    assert call(scale=None) == rt.EINVAL
    assert call(rows=0) == rt.EINVAL
    assert call(cols=0) == rt.EINVAL
    assert call(rows=2 ** 31 + 1) == rt.EINVAL
    assert call(ldx=128) == rt.EINVAL
    assert call(eps=0.0) == rt.EINVAL
    assert call(mode=5) == rt.EINVAL
    assert call(cols=64, ldx=64) == rt.EALIGN        # K not a multiple of 128
    assert call(cols=144, ldx=144) == rt.EALIGN
    assert call(qp=FAKE + 8) == rt.EALIGN
    assert call(x=FAKE + 8) == rt.EALIGN
    assert call(gran=(1, 24)) == rt.EALIGN
    assert call(cnt=FAKE_ODD) == rt.EALIGN


def test_delayed_scale_update_validation(rt):
    L = rt.lib()

    def call(**kw):
        a = dict(h=FAKE, n=16, head=FAKE, a=FAKE, f=rt.E4M3, fn=rt.HIST_MAX, m=0, eps=1e-12, s=FAKE)
        a.update(kw)
        return L.fp8_delayed_scale_update(a["h"], a["n"], a["head"], a["a"], a["f"], a["fn"], a["m"], a["eps"], 0,
                                          a["s"], None, None)
    assert call(h=None) == rt.EINVAL
    assert call(s=None) == rt.EINVAL
    assert call(n=0) == rt.EINVAL
    assert call(n=1025) == rt.EINVAL
    assert call(fn=2) == rt.EINVAL
    assert call(m=-1) == rt.EINVAL
    assert call(m=17) == rt.EINVAL
    assert call(eps=float("inf")) == rt.EINVAL
    assert call(head=FAKE + 2) == rt.EALIGN


def test_quant_error_and_ledger_validation(rt):
    L = rt.lib()
    G = rt.Gran

    def qe(**kw):
        a = dict(w=FAKE, wt=rt.BF16, N=32, K=64, ldw=64, q=FAKE, f=rt.E4M3, ldq=64, g=(1, 0), s=FAKE, x=None, M=0,
                 ldx=0, st=FAKE)
        a.update(kw)
        return L.fp8_quant_error(a["w"], a["wt"], a["N"], a["K"], a["ldw"], a["q"], a["f"], a["ldq"], G(*a["g"]),
                                 a["s"], a["x"], a["M"], a["ldx"], a["st"], None)
    assert qe(w=None) == rt.EINVAL
    assert qe(q=None) == rt.EINVAL
    assert qe(st=None) == rt.EINVAL
    assert qe(N=0) == rt.EINVAL
    assert qe(ldq=32) == rt.EINVAL
    assert qe(x=FAKE, M=0, ldx=64) == rt.EINVAL
    assert qe(x=FAKE, M=4, ldx=32) == rt.EINVAL
    assert qe(K=40, ldw=40, ldq=40) == rt.EALIGN
    assert qe(ldw=68) == rt.EALIGN
    assert qe(q=FAKE + 4) == rt.EALIGN
    assert qe(st=FAKE + 4) == rt.EALIGN
    assert qe(g=(1, 12)) == rt.EUNSUPPORTED

    spec = (rt.LedgerSpec * 1)(rt.LedgerSpec(G(1, 0), 0))
    rows = (rt.LedgerRow * 1)()

    def led(**kw):
        a = dict(w=FAKE, N=32, K=64, ldw=64, specs=spec, n=1, rows=rows, eps=1e-12)
        a.update(kw)
        return L.fp8_granularity_ledger(a["w"], rt.BF16, a["N"], a["K"], a["ldw"], None, 0, 0, rt.E4M3, a["eps"],
                                        a["specs"], a["n"], a["rows"], None)
    assert led(w=None) == rt.EINVAL
    assert led(n=0) == rt.EINVAL
    assert led(n=65) == rt.EINVAL
    assert led(specs=None) == rt.EINVAL
    assert led(rows=None) == rt.EINVAL
    assert led(eps=float("nan")) == rt.EINVAL
    assert led(K=40, ldw=40) == rt.EALIGN
    assert C.sizeof(rt.LedgerRow) == 96 and C.sizeof(rt.LedgerSpec) == 12


def test_gemm_noalloc_refuses_shapes_beyond_its_scratch(rt):
    """The allocation-free GEMM checks its fixed scratch (16 MiB) on the host:
    1x32 exponent tables of (ceil(M/256) + ceil(N/256)) * K/128 * 1024 bytes fit
    at M = 16384, N = 49152, K = 8192 (exactly 16 MiB) and not at N = 49408."""
    big = dict(M=16384, K=8192, lda=8192, ldb=8192, ga=(1, 32), gb=(1, 32), flags=rt.POW2_SCALES)
    assert g(rt, "fp8_scaled_gemm_noalloc", N=49408, ldy=49408, **big) == rt.ESCRATCH
    # 128 x 128 B blocks with 1x128 A groups on a large shape: ceil(M/256)*256 * K/128 * 4 bytes
    assert g(rt, "fp8_scaled_gemm_noalloc", M=65536 * 2, N=256, K=65536 // 2, lda=32768, ldb=32768,
             ldy=256, ga=(1, 128), gb=(128, 128)) == rt.ESCRATCH
    assert rt.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert b"16 MiB" in rt.lib().fp8rt_status_string(rt.ESCRATCH)
