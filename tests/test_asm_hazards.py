"""The GEMM's global->LDS copies are inline assembly, so the compiler's hazard checks do
not see that they read their base address from an SGPR pair.  On this architecture a
vector-memory instruction that reads an SGPR written by a vector-ALU instruction (for
instance an SGPR reloaded from a spill with v_readlane) needs 5 wait states in between.
This test compiles csrc/gemm.hip for gfx950 and checks, in the assembly of code built
here, that no copy reads a base SGPR written by a vector-ALU instruction within those
5 wait states (each instruction counts one, s_nop N counts N + 1)."""
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

WAIT_STATES = 5


def _sgprs(spec):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", spec)
    if m:
        return {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {spec} if re.fullmatch(r"s\d+", spec) else set()


def hazards(asm_lines):
    """(line index, copy, offending instruction) for each violation."""
    out = []
    instrs = [(i, l.strip()) for i, l in enumerate(asm_lines)
              if l.strip() and not l.strip().startswith((";", ".")) and not l.strip().endswith(":")]
    for n, (i, text) in enumerate(instrs):
        m = re.match(r"global_load_lds_\w+\s+v\d+,\s*(s\[\d+:\d+\])", text)
        if not m:
            continue
        base = _sgprs(m.group(1))
        waits = 0
        for _, prev in reversed(instrs[:n]):
            if waits >= WAIT_STATES:
                break
            op = prev.split()[0]
            if op.startswith("v_"):
                dst = prev.split()[1].rstrip(",")
                if _sgprs(dst) & base:
                    out.append((i, text, prev))
                    break
            nop = re.match(r"s_nop\s+(\d+)", prev)
            waits += int(nop.group(1)) + 1 if nop else 1
    return out


def test_hazard_scan_finds_a_planted_case():
    planted = ["v_readlane_b32 s3, v244, 4", "s_nop 0", "global_load_lds_dword v1, s[2:3]"]
    assert len(hazards(planted)) == 1
    assert hazards(["v_readlane_b32 s3, v244, 4", "s_nop 4", "global_load_lds_dword v1, s[2:3]"]) == []


def test_gemm_copies_respect_vmem_sgpr_wait_states():
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
    assert any("global_load_lds" in l for l in lines)
    bad = hazards(lines)
    assert not bad, bad[:5]
