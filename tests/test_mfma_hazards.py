"""Wait states around the decode kernel's inline-assembly MFMAs (CPU only).

The compiler does not know that the inline assembly in kv8_decode.hip holds
MFMA instructions, so it inserts none of the wait states an MFMA needs.
This test compiles the kernel for gfx950 and checks the generated code:

* a VALU write of an MFMA source register (A, B or C operand) is followed by
  at least two wait states before the MFMA reads it;
* a VGPR written by an MFMA (the score accumulators) is not read or written
  by a non-MFMA instruction within 18 wait states of the MFMA (the result
  latency of a 32x32 XDL operation, counted conservatively).

Wait states are counted as one per instruction and N + 1 per s_nop N; a
label inside the window ends the search (the kernel places none there).
"""
import os
import re
import shutil
import subprocess

import pytest

from fp8_e4m3_latent_amd import build

SRC = os.path.join(build.CSRC, "kv8_decode.hip")
RAW_WS = 2     # VALU write -> MFMA read
RESULT_WS = 18  # MFMA write of a VGPR -> other read or write


def _regs(tok):
    m = re.match(r"^([vas])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([vas])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(line):
    s = line.split(";")[0].strip()
    if not s or s.startswith("."):
        return None
    if s.endswith(":"):
        return ("LABEL", [])
    parts = s.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return (parts[0], ops)


def _wait_states(op, ops):
    return int(ops[0], 0) + 1 if op.startswith("s_nop") else 1


def _defs_uses(op, ops):
    """(registers written, registers read) of a non-MFMA instruction."""
    if op.startswith(("ds_write", "global_store", "buffer_store", "scratch_store", "flat_store")):
        return set(), set().union(*[_regs(o) for o in ops]) if ops else set()
    if op.startswith("v_permlane"):
        both = _regs(ops[0]) | _regs(ops[1])
        return both, both
    if not ops:
        return set(), set()
    uses = set().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
    return _regs(ops[0]), uses


@pytest.fixture(scope="module")
def asm_lines(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "kv8_decode.s")
    subprocess.run([hipcc, *build.flags(), "--cuda-device-only", "-S", SRC, "-o", out],
                   check=True, capture_output=True)
    ins = [x for x in (_parse(l) for l in open(out)) if x]
    assert sum(1 for op, _ in ins if op.startswith("v_mfma")) > 0
    return ins


def test_valu_writes_reach_mfma_operands_after_two_wait_states(asm_lines):
    bad = []
    for i, (op, ops) in enumerate(asm_lines):
        if not op.startswith("v_mfma"):
            continue
        srcs = set().union(*[_regs(o) for o in ops[1:4]])
        ws, j = 0, i - 1
        while j >= 0 and ws < RAW_WS:
            pop, pops = asm_lines[j]
            if pop == "LABEL":
                bad.append((i, "label inside the window"))
                break
            if pop.startswith("v_") and not pop.startswith("v_mfma"):
                defs, _ = _defs_uses(pop, pops)
                if defs & srcs:
                    bad.append((i, "%s %s" % (pop, ",".join(pops))))
            ws += _wait_states(pop, pops)
            j -= 1
    assert not bad, bad[:5]


def test_mfma_vgpr_results_are_not_touched_before_their_latency(asm_lines):
    bad = []
    for i, (op, ops) in enumerate(asm_lines):
        if not op.startswith("v_mfma") or not ops[0].startswith("v"):
            continue
        dst = _regs(ops[0])
        ws, j = 0, i + 1
        while j < len(asm_lines) and ws < RESULT_WS:
            pop, pops = asm_lines[j]
            if pop == "LABEL":
                break
            if pop.startswith("v_mfma"):
                # a later MFMA accumulating into the same registers is allowed
                # (back-to-back dependent MFMAs), any other operand use is not
                mdst = _regs(pops[0])
                msrc = set().union(*[_regs(o) for o in pops[1:3]])
                if msrc & dst or (mdst & dst and _regs(pops[3]) != dst):
                    bad.append((i, "%s %s" % (pop, ",".join(pops))))
            elif not pop.startswith("s_"):
                defs, uses = _defs_uses(pop, pops)
                if (defs | uses) & dst:
                    bad.append((i, "%s %s" % (pop, ",".join(pops))))
            ws += _wait_states(pop, pops)
            j += 1
    assert not bad, bad[:5]
