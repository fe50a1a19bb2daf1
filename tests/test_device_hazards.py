"""Static check of the gfx950 device code for a hazard the compiler cannot see.

On gfx9 parts a vector memory instruction that reads an SGPR (its scalar base
address, or a scalar offset) needs five wait states after a VALU instruction
that wrote that SGPR (v_readfirstlane, v_cmp into an SGPR pair, a carry out).
The compiler inserts them between its own instructions, but the kernels issue
their LDS-DMA and asynchronous loads from inline assembly, whose operands it
does not inspect: a scalar base computed by v_readfirstlane and consumed at
once by such a load reads a stale register and can fault.  The test compiles
every kernel source with the library's flags to gfx950 assembly and requires
at least five wait states (instructions, or s_nop N counting N + 1) between any
VALU write of an SGPR and a vector memory instruction that reads it.
"""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_fine_grained_amd import build

WAIT_STATES = 5


def _sgprs(text):
    regs = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", text):
        regs |= set(range(int(a), int(b) + 1))
    regs |= {int(a) for a in re.findall(r"(?<![\w\[:])s(\d+)\b", text)}
    return regs


def _valu_sgpr_writes(ins):
    op, _, rest = ins.partition(" ")
    if not op.startswith("v_") or "mfma" in op:
        return set()
    operands = [o.strip() for o in rest.split(",")]
    written = _sgprs(operands[0]) if operands else set()
    if "_co_" in op and len(operands) > 1:  # carry out into an SGPR pair
        written |= _sgprs(operands[1])
    return written


def _vmem_sgpr_reads(ins):
    op, _, rest = ins.partition(" ")
    if not op.startswith(("global_", "buffer_", "scratch_", "flat_")):
        return set()
    operands = [o.strip() for o in rest.split(",")]
    reads = set()
    for o in operands[1:]:
        reads |= _sgprs(o.split()[0] if o else "")
    return reads


def hazards(asm_text):
    """(function, gap, writer, reader) for every VMEM read of an SGPR written by
    a VALU instruction fewer than WAIT_STATES wait states before it."""
    found = []
    for func in re.split(r"\n(?=[A-Za-z_.$][\w.$]*:\s*; @)", asm_text):
        name = func.split(":", 1)[0]
        # instructions only: comments (the inline-assembly markers among them),
        # directives and labels are skipped, so a label is crossed along the
        # fall-through path
        code = []
        for line in func.splitlines():
            line = line.split(";")[0].strip()
            if line and not line.startswith(".") and not line.endswith(":"):
                code.append(line)
        for i, ins in enumerate(code):
            reads = _vmem_sgpr_reads(ins)
            if not reads:
                continue
            gap = 0
            for k in range(i - 1, -1, -1):
                prev = code[k]
                if prev.startswith("s_nop"):
                    gap += int(prev.split()[1]) + 1
                else:
                    if _valu_sgpr_writes(prev) & reads:
                        found.append((name, gap, prev, ins))
                        break
                    gap += 1
                if gap >= WAIT_STATES:
                    break
    return found


def test_scanner_catches_the_pattern():
    bad = "k:  ; @k\n\tv_readfirstlane_b32 s9, v5\n\t;;#ASMSTART\n\tglobal_load_dword v1, v2, s[8:9]\n\t;;#ASMEND\n"
    ok = "k:  ; @k\n\tv_readfirstlane_b32 s9, v5\n\ts_nop 4\n\tglobal_load_dword v1, v2, s[8:9]\n"
    carry = "k:  ; @k\n\tv_add_co_u32_e64 v3, s[8:9], v1, v2\n\tglobal_load_dword v1, v2, s[8:9]\n"
    assert len(hazards(bad)) == 1
    assert hazards(ok) == []
    assert len(hazards(carry)) == 1


def _compiler():
    for cand in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_kernels_have_no_valu_sgpr_to_vmem_hazard():
    cxx = _compiler()
    if cxx is None:
        pytest.skip("no HIP compiler")
    srcs = [s for s in build.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [cxx, *build.FLAGS, "--cuda-device-only", "-S", "-x", "hip", os.path.join(build.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as f:
                return src, hazards(f.read())
        with ThreadPoolExecutor(len(srcs)) as ex:
            results = list(ex.map(one, srcs))
    problems = [(src, h) for src, hs in results for h in hs]
    assert not problems, problems[:10]
