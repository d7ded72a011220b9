"""CPU runs under AddressSanitizer + UndefinedBehaviorSanitizer (every report
fatal):
  - the oracle built with gcc's sanitizers, driven by all of its pin tests;
  - the library's host code (argument validation, dispatch, status strings)
    built with the host compiler's sanitizers, driven by the boundary tests,
    which call every entry point with invalid arguments (out-of-range enum
    values, null pointers, misaligned sizes) and never reach a kernel.
Each run is a subprocess with the matching sanitizer runtime preloaded into
the interpreter; pytest runs there without output capture, so a report is
printed before the process exits with its error status."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    import oracle

    oracle.build_sanitized()
    libs = [subprocess.run(["gcc", "-print-file-name=%s" % n], capture_output=True, text=True).stdout.strip()
            for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = run({"FP8RT_ORACLE_SANITIZED": "1", "LD_PRELOAD": " ".join(libs)}, tests)
    assert " passed" in out


def test_library_host_code_under_asan_ubsan():
    from dynamic_scaling_scaled_amd import _build

    lib = _build.build_host_sanitized()
    rt = _build.asan_runtime()
    if not rt:
        pytest.skip("the host compiler's ASan runtime is not installed")
    out = run({"FP8RT_LIB": lib, "LD_PRELOAD": rt}, [os.path.join(ROOT, "tests", "test_boundary.py")])
    assert " passed" in out
