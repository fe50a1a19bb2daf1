"""Static check of the gfx950 device code for hazards the compiler cannot see.

The kernels issue their LDS-DMA and asynchronous loads from inline assembly,
whose operands and implicit registers the compiler does not inspect, so it
cannot insert the wait states the hardware needs around them.  Two rules of
the gfx9 family (gfx950 included) are checked here:

* VALU -> SGPR -> VMEM: a vector memory instruction that reads an SGPR (its
  scalar base address, or a scalar offset) needs five wait states after a
  VALU instruction that wrote that SGPR (v_readfirstlane, v_cmp into an SGPR
  pair, a carry out).  A scalar base computed by v_readfirstlane and
  consumed at once by such a load reads a stale register and can fault.
* SALU -> M0 -> LDS DMA: a load that writes LDS directly (``*_load_lds_*``)
  takes its LDS address from M0 and needs one wait state after a scalar ALU
  write of M0 (the compiler places ``s_nop 0`` there for its own
  ``global_load_lds`` builtin).  Without it the DMA can use the previous M0,
  which silently lands a tile in the wrong LDS slot.  A VALU write of M0
  (v_readfirstlane into m0) falls under the first rule.

The test compiles every kernel source with the library's flags to gfx950
assembly and walks back from each reading instruction over every control-flow
predecessor -- the fall-through path and every branch that targets the label
in front of it, loop back-edges included -- counting wait states
(instructions, or s_nop N counting N + 1) until the rule's distance is
covered or a hazardous writer is found.
"""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_fine_grained_amd import build

VALU_SGPR_VMEM_WAIT_STATES = 5
SALU_M0_LDS_DMA_WAIT_STATES = 1
M0 = "m0"


def _sgprs(text):
    regs = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", text):
        regs |= set(range(int(a), int(b) + 1))
    regs |= {int(a) for a in re.findall(r"(?<![\w\[:])s(\d+)\b", text)}
    if re.search(r"\bm0\b", text):
        regs.add(M0)
    return regs


def _operands(ins):
    _, _, rest = ins.partition(" ")
    return [o.strip() for o in rest.split(",")] if rest.strip() else []


def _is_lds_dma(ins):
    op = ins.split()[0]
    return op.startswith(("global_", "buffer_")) and "_lds" in op or (
        op.startswith("buffer_load") and re.search(r"\blds\b", ins) is not None)


def _valu_sgpr_writes(ins):
    op = ins.split()[0]
    if not op.startswith("v_") or "mfma" in op:
        return set()
    operands = _operands(ins)
    written = _sgprs(operands[0]) if operands else set()
    if "_co_" in op and len(operands) > 1:  # carry out into an SGPR pair
        written |= _sgprs(operands[1])
    return written


def _vmem_sgpr_reads(ins):
    op = ins.split()[0]
    if not op.startswith(("global_", "buffer_", "scratch_", "flat_")):
        return set()
    reads = set()
    for o in _operands(ins)[1:]:
        reads |= _sgprs(o.split()[0] if o else "")
    if _is_lds_dma(ins):
        reads.add(M0)  # the LDS destination address
    return reads


def _salu_m0_write(ins):
    op = ins.split()[0]
    if not op.startswith("s_") or op.startswith(("s_nop", "s_waitcnt", "s_barrier", "s_cbranch", "s_branch")):
        return False
    operands = _operands(ins)
    return bool(operands) and operands[0] == M0


_BRANCH = re.compile(r"^s_(?:branch|cbranch_\w+)\s+(\S+)")
_NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc_b64")


def _parse(func):
    """Instructions of one function and the predecessors of each: the
    previous instruction unless it ends the straight-line path, and every
    branch whose target label stands in front of the instruction."""
    code, labels_at = [], {}
    pending = []
    for line in func.splitlines():
        line = line.split(";")[0].strip()  # comments, inline-assembly markers among them
        if not line or line.startswith("."):
            if line.endswith(":"):  # .LBB labels
                pending.append(line[:-1])
            continue
        if line.endswith(":"):
            pending.append(line[:-1])
            continue
        for lab in pending:
            labels_at[lab] = len(code)
        pending = []
        code.append(line)
    preds = [[] for _ in code]
    for i, ins in enumerate(code):
        if i + 1 < len(code) and not ins.split()[0] in _NO_FALLTHROUGH:
            preds[i + 1].append(i)
        m = _BRANCH.match(ins)
        if m and m.group(1) in labels_at:
            preds[labels_at[m.group(1)]].append(i)
    return code, preds


def _walk_back(code, preds, i, need, is_writer):
    """(gap, writer) pairs: writers reached from instruction i along some path
    with fewer than `need` wait states between them and i."""
    found = []
    seen = set()
    stack = [(p, 0) for p in preds[i]]
    while stack:
        k, gap = stack.pop()
        if (k, gap) in seen:
            continue
        seen.add((k, gap))
        prev = code[k]
        if prev.startswith("s_nop"):
            step = int(prev.split()[1], 0) + 1
        else:
            if is_writer(prev):
                found.append((gap, prev))
                continue
            step = 1
        if gap + step >= need:
            continue
        stack.extend((p, gap + step) for p in preds[k])
    return found


def hazards(asm_text):
    """(function, rule, gap, writer, reader) for every hazard in the assembly."""
    found = []
    for func in re.split(r"\n(?=[A-Za-z_.$][\w.$]*:\s*; @)", asm_text):
        name = func.split(":", 1)[0]
        code, preds = _parse(func)
        for i, ins in enumerate(code):
            reads = _vmem_sgpr_reads(ins)
            if not reads:
                continue
            for gap, w in _walk_back(code, preds, i, VALU_SGPR_VMEM_WAIT_STATES,
                                     lambda p: bool(_valu_sgpr_writes(p) & reads)):
                found.append((name, "valu-sgpr-vmem", gap, w, ins))
            if _is_lds_dma(ins):
                for gap, w in _walk_back(code, preds, i, SALU_M0_LDS_DMA_WAIT_STATES, _salu_m0_write):
                    found.append((name, "salu-m0-lds-dma", gap, w, ins))
    return found


def _k(body):
    return "k:  ; @k\n" + body


def test_scanner_catches_the_patterns():
    # VALU-written SGPR read by an inline-assembly load
    bad = _k("\tv_readfirstlane_b32 s9, v5\n\t;;#ASMSTART\n\tglobal_load_dword v1, v2, s[8:9]\n\t;;#ASMEND\n")
    ok = _k("\tv_readfirstlane_b32 s9, v5\n\ts_nop 4\n\tglobal_load_dword v1, v2, s[8:9]\n")
    carry = _k("\tv_add_co_u32_e64 v3, s[8:9], v1, v2\n\tglobal_load_dword v1, v2, s[8:9]\n")
    assert [h[1] for h in hazards(bad)] == ["valu-sgpr-vmem"]
    assert hazards(ok) == []
    assert len(hazards(carry)) == 1
    # SALU write of M0 directly before an LDS DMA; one wait state is enough
    m0 = _k("\ts_mov_b32 m0, s14\n\tglobal_load_lds_dwordx4 v122, s[26:27]\n")
    m0_nop = _k("\ts_mov_b32 m0, s14\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v122, s[26:27]\n")
    m0_other = _k("\ts_mov_b32 m0, s14\n\tv_mov_b32 v1, 0\n\tglobal_load_lds_dword v1, off\n")
    m0_plain_load = _k("\ts_mov_b32 m0, s14\n\tglobal_load_dwordx4 v[0:3], v122, s[26:27]\n")
    assert [h[1] for h in hazards(m0)] == ["salu-m0-lds-dma"]
    assert hazards(m0_nop) == [] and hazards(m0_other) == [] and hazards(m0_plain_load) == []
    # VALU write of M0 before an LDS DMA: the five-wait-state rule
    vm0 = _k("\tv_readfirstlane_b32 m0, v3\n\ts_nop 1\n\tglobal_load_lds_dword v1, off\n")
    assert [h[1] for h in hazards(vm0)] == ["valu-sgpr-vmem"]
    # across a loop back-edge: the writer is the loop's last instruction before
    # the branch, the reader the first instruction after the label
    loop = _k("\ts_mov_b32 s9, 0\n.LBB0_1:\n\tglobal_load_dword v1, v2, s[8:9]\n\ts_add_u32 s4, s4, 1\n"
              "\tv_readfirstlane_b32 s9, v7\n\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    assert [h[1] for h in hazards(loop)] == ["valu-sgpr-vmem"]
    loop_m0 = _k(".LBB0_1:\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n\tv_add_u32_e32 v1, 16, v1\n"
                 "\tv_readfirstlane_b32 m0, v5\n\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    assert [h[1] for h in hazards(loop_m0)] == ["valu-sgpr-vmem"]
    # (the taken branch is itself one wait state, enough for an SALU write of M0)
    loop_salu_m0 = loop_m0.replace("v_readfirstlane_b32 m0, v5", "s_mov_b32 m0, s5")
    assert hazards(loop_salu_m0) == []
    # a forward branch that jumps over the writer: only the fall-through path is hazardous
    fwd = _k("\ts_cbranch_scc1 .LBB0_2\n\tv_readfirstlane_b32 s9, v5\n.LBB0_2:\n\tglobal_load_dword v1, v2, s[8:9]\n")
    assert len(hazards(fwd)) == 1
    # an unconditional branch ends the straight-line path
    jump = _k("\tv_readfirstlane_b32 s9, v5\n\ts_branch .LBB0_3\n.LBB0_2:\n\tglobal_load_dword v1, v2, s[8:9]\n"
              ".LBB0_3:\n\ts_endpgm\n")
    assert hazards(jump) == []


# Instructions that read M0 without naming it (gfx9 family).
_IMPLICIT_M0 = ("s_sendmsg", "s_movrel", "v_movrel", "ds_gws", "ds_append", "ds_consume", "ds_ordered_count",
                "v_interp", "s_ttracedata")


def m0_ownership_problems(asm_text):
    """The inline-assembly DMA helpers write M0 without saving it (the compiler
    reserves M0 and cannot take it as a clobber).  That is safe only if the
    compiled code names M0 nowhere else, nothing else reads it implicitly, and
    every LDS DMA is issued right after its own M0 write and one wait state
    (the three instructions of one asm statement, which the compiler cannot
    split).  Returns the instructions that break this."""
    bad = []
    for func in re.split(r"\n(?=[A-Za-z_.$][\w.$]*:\s*; @)", asm_text):
        code, _ = _parse(func)
        for i, ins in enumerate(code):
            op = ins.split()[0]
            if re.search(r"\bm0\b", ins) and not (op == "s_mov_b32" and _operands(ins)[0] == M0):
                bad.append(("names m0", ins))
            if op.startswith(_IMPLICIT_M0):
                bad.append(("reads m0", ins))
            if _is_lds_dma(ins):
                if i < 2 or code[i - 1] != "s_nop 0" or not code[i - 2].startswith("s_mov_b32 m0,"):
                    bad.append(("lds dma without its own m0 write", ins))
    return bad


def test_m0_ownership_check_catches_the_patterns():
    ok = _k("\ts_mov_b32 m0, s14\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v122, s[26:27]\n")
    assert m0_ownership_problems(ok) == []
    assert m0_ownership_problems(_k("\ts_mov_b32 m0, s14\n\ts_nop 0\n\tv_mov_b32 v1, 0\n"
                                    "\tglobal_load_lds_dword v1, off\n"))
    assert m0_ownership_problems(_k("\ts_add_u32 m0, m0, 4\n"))
    assert m0_ownership_problems(_k("\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)\n"))


def _compiler():
    for cand in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def compile_to_asm(src, out):
    cmd = [_compiler(), *build.FLAGS, "--cuda-device-only", "-S", "-x", "hip", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.timeout(600)
def test_kernels_have_no_inline_assembly_hazard():
    if _compiler() is None:
        pytest.skip("no HIP compiler")
    srcs = [s for s in build.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            text = compile_to_asm(src, os.path.join(tmp, src + ".s"))
            return src, hazards(text), len(re.findall(r"_load_lds_", text)), m0_ownership_problems(text)
        with ThreadPoolExecutor(len(srcs)) as ex:
            results = list(ex.map(one, srcs))
    # the scan has something to look at: the GEMM issues its tiles by LDS DMA
    assert dict((s, n) for s, _, n, _ in results)["gemm_fp8.hip"] > 0
    problems = [(src, h) for src, hs, _, _ in results for h in hs]
    assert not problems, f"{len(problems)} hazards, e.g. {problems[:5]}"
    m0 = [(src, b) for src, _, _, bs in results for b in bs]
    assert not m0, f"M0 used outside the DMA helpers: {m0[:5]}"
