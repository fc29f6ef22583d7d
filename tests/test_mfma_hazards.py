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

It also checks that the innermost loop of the kernel (the tile loop) holds
no scratch (spill) access: a reload there waits for every tile copy in
flight, which stalls the copy pipeline.
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
def asm_text(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "kv8_decode.s")
    subprocess.run([hipcc, *build.flags(), "--cuda-device-only", "-S", SRC, "-o", out],
                   check=True, capture_output=True)
    return open(out).read().split("\n")


@pytest.fixture(scope="module")
def asm_lines(asm_text):
    ins = [x for x in (_parse(l) for l in asm_text) if x]
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


def test_no_scratch_access_in_the_tile_loop(asm_text):
    # the decode kernel's loops: labels the compiler annotates with their
    # depth; the tile loop is the one at depth 2 (inside the restart pass)
    kern = "absorb_decode_kernel"
    start = next(i for i, l in enumerate(asm_text)
                 if kern in l and l.split(";")[0].rstrip().endswith(":"))
    end = next(i for i in range(start, len(asm_text)) if asm_text[i].strip() == "s_endpgm")
    body = asm_text[start:end]
    # the loop header's label line, and then a comment naming it a depth-2
    # loop header (on the same line or the next)
    header = None
    for i, l in enumerate(body):
        if "Loop Header: Depth=2" in l:
            k = i
            while not re.match(r"^\.LBB\d+_\d+:", body[k]):
                k -= 1
            header = body[k].split(":")[0][1:]
            break
    assert header, "no depth-2 loop found"
    first = next(i for i, l in enumerate(body) if l.startswith("." + header + ":"))
    last = max(i for i, l in enumerate(body) if ("Header=" + header[1:]) in l or
               l.startswith("." + header + ":"))
    # through the loop's backward branch
    j = last
    while "s_cbranch" not in body[j] and "s_branch" not in body[j]:
        j += 1
    loop = body[first:j + 1]
    assert sum(1 for l in loop if "v_mfma" in l) >= 68, "tile loop not found"
    bad = [l.strip() for l in loop if "scratch_" in l]
    assert not bad, bad[:5]
