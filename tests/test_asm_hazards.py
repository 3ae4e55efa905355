"""Wait-state check of the MFMAs issued from inline assembly.

The bf16/fp16 16x16x32 and int8 16x16x64 K loops issue their MFMAs as inline
assembly (so each accumulator stays in its AGPRs), which the compiler's
hazard recognizer does not look into.  An MFMA needs a few wait states after
a VALU instruction writes one of its source registers.  The bf16 loops never
produce such a write (operands come from LDS reads, accumulators are first
written by the MFMAs themselves); the int8 loop's uint8 operands are flipped
to int8 in their registers at least three MFMAs ahead of their first use.
This test compiles the three kernel files for gfx950 and checks that no VALU
instruction writes a source register of such an MFMA within 4 wait states
before it.  Only MFMAs between the compiler's inline-assembly markers are
checked: those from MFMA builtins (the skinny kernels') are spaced out by the
compiler itself.  CPU only (hipcc cross-compiles); skipped without hipcc."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "onnx_matmul_family_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instructions(asm):
    """Instruction lines, and the indices of those that come from inline
    assembly (between the compiler's ;;#ASMSTART / ;;#ASMEND markers)."""
    out, in_asm, inside = [], set(), False
    for line in asm.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
        elif s.startswith(";;#ASMEND"):
            inside = False
        elif s and not s.startswith((";", ".", "_")) and not s.endswith(":"):
            if inside:
                in_asm.add(len(out))
            out.append(s)
    return out, in_asm


ASM_MFMA = ("v_mfma_f32_16x16x32", "v_mfma_i32_16x16x64_i8")


def _violations(ins, window=4, only=None):
    """MFMAs (of the forms this library issues from inline assembly; with
    `only`, just those at these indices) with a VALU write of one of their
    source registers within `window` wait states before them."""
    bad, n = [], 0
    for i, line in enumerate(ins):
        if not line.startswith(ASM_MFMA) or (only is not None and i not in only):
            continue
        n += 1
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        src = set().union(*[_regs(o) for o in ops[1:]])
        ws, j = 0, i - 1
        while j >= 0 and ws < window:
            p = ins[j]
            if p.startswith("s_nop"):
                ws += int(p.split()[1]) + 1
            else:
                if p.startswith("v_") and not p.startswith("v_mfma"):
                    if _regs(p.split(None, 1)[1].split(",")[0].strip()) & src:
                        bad.append((p, line, ws))
                ws += 1
            j -= 1
    return n, bad


def _compile(src, out):
    extra = ["-ffp-contract=off"] if src == "qlinear.hip" else []  # as the library build
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S"] + extra + [
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def test_checker_flags_a_planted_write():
    ins = ["v_mov_b32_e32 v5, v9", "v_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]"]
    assert len(_violations(ins)[1]) == 1
    assert len(_violations(["s_nop 3"] + ins[:1] + ["s_nop 3"] + ins[1:])[1]) == 0
    flip = ["v_bitop3_b32 v53, v57, s51, 0 bitop3:0x3c", "v_mfma_i32_16x16x32_i8 a[0:3], v[18:21], v[50:53], 0",
            "v_mfma_i32_16x16x64_i8 a[4:7], v[18:21], v[50:53], 0"]
    assert len(_violations(flip)[1]) == 1  # the 16x16x64 form at distance 1 (the 16x16x32 int8 form is not ours)
    # only MFMAs from inline assembly are checked: a builtin's MFMA is the compiler's to space out
    asm = "\n".join(["v_mov_b32_e32 v5, v9", ins[1], ";;#ASMSTART", ins[1], ";;#ASMEND"])
    code, in_asm = _instructions(asm)
    assert in_asm == {2}
    assert [b[2] for b in _violations(code, only=in_asm)[1]] == [1]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_no_valu_write_of_mfma16_operands():
    with tempfile.TemporaryDirectory() as d:
        srcs = ["dense16.hip", "grouped.hip", "qlinear.hip"]
        with ThreadPoolExecutor(3) as ex:
            asms = list(ex.map(lambda s: _compile(s, os.path.join(d, s + ".s")), srcs))
    total = 0
    for src, asm in zip(srcs, asms):
        ins, in_asm = _instructions(asm)
        n, bad = _violations(ins, only=in_asm)
        total += n
        assert not bad, "%s: %s" % (src, bad[:3])
        assert n > 1000, src  # the inline-assembly loops were found
