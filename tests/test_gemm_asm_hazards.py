"""The large GEMM's inline MFMAs and the compiler's schedule around them (CPU
only: compiles the kernel file to gfx950 assembly).

k_gemm_big16 issues its 16x16x128 MFMAs as inline assembly with the
accumulator as one tied AGPR operand, so the hazard recognizer does not see
them; the kernel pads the two places where VALU code touches the
accumulators with 24 wait states (acc_fence).  This checks, for every
instantiation, that the compiler kept that padding effective (no accumulator
write between the zero fill's fence and the first MFMA, no accumulator read
between the last MFMA and the epilogue's fence) and that the main loop holds
no accumulator copy, spill or wait for all vector-memory loads."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "dynamic_scaling_scaled_amd", "csrc", "gemm_big.hip")


@pytest.fixture(scope="module")
def asm():
    from dynamic_scaling_scaled_amd import _build

    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm_big.s")
        cmd = [_build.hipcc(), *_build.HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", _build.INCLUDE,
               "-I", _build.CSRC, SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail("hipcc failed:\n" + r.stderr[-2000:])
        return open(out).read()


def kernels(s):
    for m in re.finditer(r"^(_ZN\S*k_gemm_big16\S*):", s, re.M):
        end = s.index("s_endpgm", m.start())
        yield m.group(1), s[m.start():end].split("\n")


def main_loop(lines):
    labels = {m.group(1): k for k, l in enumerate(lines) for m in [re.match(r"^(\.LBB\d+_\d+):", l)] if m}
    loops = []
    for k, l in enumerate(lines):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", l)
        if m and labels.get(m.group(1), len(lines)) < k:
            loops.append(lines[labels[m.group(1)]:k])
    return max(loops, key=len)


def test_every_instantiation_is_there(asm):
    names = [n for n, _ in kernels(asm)]
    assert len(names) == 16, names   # 2 A formats x 4 outputs x (per-tensor/row, 1x32)


def test_accumulator_fences_bracket_the_mfmas(asm):
    for name, lines in kernels(asm):
        nop = [k for k, l in enumerate(lines) if l.strip() == "s_nop 7"]
        fences = [k for k in nop if lines[k + 1].strip() == "s_nop 7" and lines[k + 2].strip() == "s_nop 7"]
        mf = [k for k, l in enumerate(lines) if "v_mfma" in l]
        init = [f for f in fences if f < mf[0]]
        done = [f for f in fences if f > mf[-1]]
        assert init and done, name
        between = lines[init[-1] + 3:mf[0]]
        assert not [l for l in between if re.search(r"v_accvgpr_(write|mov)", l)], name
        after = lines[mf[-1] + 1:done[0]]
        assert not [l for l in after if re.search(r"v_accvgpr_(read|mov)|global_store\S* \S+, a", l)], name


def test_main_loop_is_clean(asm):
    for name, lines in kernels(asm):
        loop = main_loop(lines)
        text = "\n".join(loop)
        assert text.count("v_mfma") == 128, name          # two stages of 8 x 8 MFMAs
        assert "v_accvgpr_mov" not in text and "scratch_" not in text, name
        assert "vmcnt(0)" not in text, name                  # only the barriers' vmcnt(16) waits
        assert text.count("s_barrier") == 4, name
