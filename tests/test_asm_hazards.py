"""The GEMM's global->LDS copies are inline assembly, so the compiler's hazard checks do
not see what they read: the base address from an SGPR pair and the LDS address from M0.
On this architecture a vector-memory instruction that reads an SGPR (M0 included)
written by a vector-ALU instruction needs 5 wait states in between (for instance an SGPR
reloaded from a spill with v_readlane, a v_cmp writing an SGPR pair, or a carry-out
written by v_add_co), and an LDS copy needs 1 wait state after a scalar write of M0.
This test compiles csrc/gemm.hip for gfx950 and checks, in the assembly of code built
here, every copy against both rules (each instruction counts one wait state, s_nop N
counts N + 1), following the code backwards across block boundaries into every
predecessor block (fall-through and branch sources)."""
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

VALU_SGPR_WAITS = 5   # VALU writes an SGPR -> a VMEM instruction reads it
SALU_M0_WAITS = 1     # SALU writes M0 -> an LDS copy reads it

# vector-ALU instructions whose second operand is a scalar destination (carry-out, VOP3b)
_VOP3B = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
          "v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale_")


def _sgprs(spec):
    """Scalar registers named by an operand ('s5', 's[4:5]', 'm0', 'vcc', ...)."""
    spec = spec.strip().rstrip(",")
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", spec)
    if m:
        return {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+", spec) or spec in ("m0", "vcc", "vcc_lo", "vcc_hi", "exec", "exec_lo", "exec_hi"):
        return {"vcc_lo", "vcc_hi"} if spec == "vcc" else {spec}
    return set()


def _operands(text):
    parts = text.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def valu_sgpr_dests(text):
    """Scalar registers a vector-ALU instruction writes."""
    op = text.split()[0]
    if not op.startswith("v_"):
        return set()
    ops = _operands(text)
    out = set()
    if ops:
        out |= _sgprs(ops[0])             # v_readlane / v_readfirstlane / v_cmp_*_e64 ...
    if op.startswith(_VOP3B) and len(ops) > 1:
        out |= _sgprs(ops[1])             # carry-out
    if re.match(r"v_cmpx?_\w+_e32", op) or (op.endswith("_e32") and op.startswith(_VOP3B)):
        out |= {"vcc_lo", "vcc_hi"}
    return out


def salu_dests(text):
    op = text.split()[0]
    if not op.startswith("s_") or op.startswith(("s_nop", "s_waitcnt", "s_barrier", "s_branch", "s_cbranch",
                                                   "s_endpgm", "s_sleep", "s_setprio")):
        return set()
    ops = _operands(text)
    return _sgprs(ops[0]) if ops else set()


def _parse(asm_lines):
    """Instructions and the control-flow predecessors of every label."""
    instrs, labels = [], {}
    for l in asm_lines:
        s = l.split(";")[0].strip()
        if re.fullmatch(r"[.\w]+:", s):  # a label (block start)
            labels[s[:-1]] = len(instrs)
            continue
        if not s or s.startswith("."):    # directives
            continue
        instrs.append(s.split(";")[0].strip())
    starts = {idx: name for name, idx in labels.items()}
    preds = {name: [] for name in labels}
    for n, text in enumerate(instrs):
        m = re.match(r"s_(c?branch\w*)\s+(\S+)", text)
        if m and m.group(2) in preds:
            preds[m.group(2)].append(n)
    for name, idx in labels.items():  # fall-through from the instruction before the label
        if idx > 0 and not instrs[idx - 1].startswith(("s_branch ", "s_endpgm", "s_setpc")):
            preds[name].append(idx - 1)
    return instrs, starts, preds


def _walk_back(instrs, starts, preds, n, budget):
    """Instructions within `budget` wait states before instruction n, on every path
    (a block start continues in each of its predecessors): (instruction, wait states
    between it and n)."""
    out, seen = [], set()
    stack = [(n, 0)]  # (position whose predecessors are visited next, wait states so far)
    while stack:
        p, waits = stack.pop()
        for k in (preds[starts[p]] if p in starts else [p - 1]):
            if k < 0 or (k, waits) in seen:
                continue
            seen.add((k, waits))
            text = instrs[k]
            out.append((text, waits))
            nop = re.match(r"s_nop\s+(\d+)", text)
            nxt = waits + (int(nop.group(1)) + 1 if nop else 1)
            if nxt < budget:
                stack.append((k, nxt))
    return out


def hazards(asm_lines):
    """(copy, offending instruction, wait states) for each violation."""
    instrs, starts, preds = _parse(asm_lines)
    out = []
    for n, text in enumerate(instrs):
        m = re.match(r"global_load_lds_\w+\s+v\d+,\s*(s\[\d+:\d+\])", text)
        if not m:
            continue
        reads = _sgprs(m.group(1)) | {"m0"}
        for prev, waits in _walk_back(instrs, starts, preds, n, VALU_SGPR_WAITS):
            if valu_sgpr_dests(prev) & reads:
                out.append((text, prev, waits))
            elif waits < SALU_M0_WAITS and "m0" in salu_dests(prev):
                out.append((text, prev, waits))
    return out


def test_hazard_scan_finds_planted_cases():
    copy = "global_load_lds_dword v1, s[2:3]"
    # a base register reloaded by v_readlane: 1 wait state is too few, 5 are enough
    assert len(hazards(["v_readlane_b32 s3, v244, 4", "s_nop 0", copy])) == 1
    assert hazards(["v_readlane_b32 s3, v244, 4", "s_nop 4", copy]) == []
    # M0 written by a vector-ALU instruction
    assert len(hazards(["v_readfirstlane_b32 m0, v7", "s_nop 3", copy])) == 1
    assert hazards(["v_readfirstlane_b32 m0, v7", "s_nop 4", copy]) == []
    # M0 written by a scalar instruction right before the copy (needs one wait state)
    assert len(hazards(["s_mov_b32 m0, s9", copy])) == 1
    assert hazards(["s_mov_b32 m0, s9", "s_nop 0", copy]) == []
    # carry-out and compare destinations
    assert len(hazards(["v_add_co_u32_e64 v4, s[2:3], v5, v6", copy])) == 1
    assert len(hazards(["v_cmp_gt_u32_e64 s[2:3], v1, v2", "s_nop 1", copy])) == 1
    # a write in a predecessor block reached by a branch (the linear order hides it)
    lines = ["s_branch .LBB0_2", ".LBB0_1:", "v_readlane_b32 s2, v9, 0", "s_branch .LBB0_3",
             ".LBB0_2:", "s_nop 7", "s_nop 7", ".LBB0_3:", copy]
    assert len(hazards(lines)) == 1
    # the same write far enough back on every path is fine
    lines[3:3] = ["s_nop 4"]
    assert hazards(lines) == []


def test_gemm_copies_respect_sgpr_and_m0_wait_states():
    from dequant_matmul_iq4_amd import build as B
    hipcc = B.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        r = subprocess.run([hipcc, *flags, "--offload-device-only", "-S", "-o", out,
                            os.path.join(B.CSRC, "gemm.hip")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = open(out).read().split("\n")
    assert sum("global_load_lds" in l for l in lines) > 50
    bad = hazards(lines)
    assert not bad, bad[:5]
