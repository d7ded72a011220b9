"""Build the HIP library ``libfp8rt.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8rt.so")
# measurement aids beside the library (csrc/calib): the matrix cores' rate with
# register-held operands, used by bench.py --calibrate-mfma; never linked into
# libfp8rt.so
CALIB_LIB = os.path.join(PKG, "libfp8rt_calib.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


# Per-file code generation options.  The K-blocked GEMM promotes every MFMA
# result with a VALU FMA, so its MFMA results live in VGPRs.
FILE_FLAGS = {
    "gemm_kblock.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_calib(verbose)
    return LIB


def build_calib(verbose: bool = False) -> str:
    srcs = sorted(os.path.join(CSRC, "calib", f) for f in os.listdir(os.path.join(CSRC, "calib"))
                  if f.endswith(".hip"))
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the calibration library:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print("built", CALIB_LIB)
    return CALIB_LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build for CPU checks
# of the library's host code (argument validation and dispatch), loaded with
# clang's ASan runtime preloaded.  Device code is built without
# instrumentation; this library is never used on a GPU.
ASAN_BUILD = os.path.join(ROOT, "_build_asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libfp8rt_asan.so")
HOST_SANITIZE = ["-fno-gpu-sanitize", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """clang's shared ASan runtime (the one hipcc's host compiler links against)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob

        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        path = hits[-1] if hits else ""
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    os.makedirs(ASAN_BUILD, exist_ok=True)

    def comp(src):
        obj = os.path.join(ASAN_BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *HOST_SANITIZE, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE,
               "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
        return obj

    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *HOST_SANITIZE, "-o",
           ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
