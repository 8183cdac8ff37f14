"""Static check of the compiled gfx950 kernels (CPU only; needs hipcc).

The K/V tile loads are inline-asm `buffer_load_dwordx4 ... lds`, which the compiler's hazard
recognizer does not see.  On gfx9 parts a buffer load may read an SGPR that a vector
instruction (v_readfirstlane, v_readlane, v_cmp ...) wrote only 5 wait states later;
otherwise it reads the register's previous value (for the buffer descriptor: a stale base or
range, i.e. wrong or zero-filled tiles).  This test compiles the kernels to assembly and
checks every such load against the instructions before it.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunk_windowed_softmax_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile_asm(tmp_path, source="kernels.hip"):
    out = tmp_path / (source + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           os.path.join(CSRC, source), "-o", str(out), "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text().split("\n")


_LABEL = re.compile(r"(\.LBB\w+):")
_BRANCH = re.compile(r"s_(?:branch|cbranch_\w+)\s+(\.LBB\w+)")


def _sgpr_hazards(lines, window=8):
    """(line, writer, load) for each buffer load whose descriptor or offset SGPRs a vector
    instruction wrote fewer than 5 wait states before it, on any path into the load: the
    scan walks back through the load's block and, at a block label, into every predecessor
    (the fall-through block and every branch to the label), at most `window` instructions
    deep on each path."""
    branches = {}
    for i, line in enumerate(lines):
        b = _BRANCH.search(line)
        if b:
            branches.setdefault(b.group(1), []).append(i)
    found = []
    for i, line in enumerate(lines):
        m = re.search(r"buffer_load_dwordx4 \w+, s\[(\d+):(\d+)\], (\w+)", line)
        if not m:
            continue
        regs = set(range(int(m.group(1)), int(m.group(2)) + 1))
        so = re.match(r"s(\d+)$", m.group(3))  # the scalar offset, when it is a register
        if so:
            regs.add(int(so.group(1)))
        stack, visited = [(i - 1, 0, 0)], set()
        while stack:
            j, waits, seen = stack.pop()
            while j >= 0 and seen < window and waits < 5:
                t = lines[j].strip()
                if not t or t.startswith(";"):
                    j -= 1
                    continue
                lab = _LABEL.match(t)
                if lab:  # also enter every block that branches here
                    for src in branches.get(lab.group(1), []):
                        if (src, waits, seen) not in visited:
                            visited.add((src, waits, seen))
                            stack.append((src, waits, seen))
                    j -= 1
                    continue
                if t.startswith("."):
                    j -= 1
                    continue
                if t.startswith("s_endpgm"):
                    break
                seen += 1
                nop = re.match(r"s_nop (\d+)", t)
                if nop:
                    waits += int(nop.group(1)) + 1
                    j -= 1
                    continue
                if t.split()[0].startswith("v_") and len(t.split()) > 1:
                    dst = t.split()[1].rstrip(",")
                    d = re.match(r"s\[(\d+):(\d+)\]$", dst) or re.match(r"s(\d+)$", dst)
                    if d:
                        lo = int(d.group(1))
                        hi = int(d.group(2)) if d.re.groups > 1 else lo
                        if regs & set(range(lo, hi + 1)):
                            found.append((i, t, line.strip()))
                waits += 1
                j -= 1
    return sorted(set(found))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("source", ["kernels.hip", "attn_fp8.hip"])
def test_no_valu_sgpr_hazard_before_tile_loads(tmp_path, source):
    lines = _compile_asm(tmp_path, source)
    loads = [l for l in lines if "buffer_load_dwordx4" in l and " lds" in l]
    assert loads, "no tile loads found in the compiled kernels"
    assert _sgpr_hazards(lines) == []


def test_hazard_scan_finds_a_planted_case():
    lines = ["\tv_readfirstlane_b32 s46, v2", "\tv_add_u32_e32 v0, s7, v25", "\ts_nop 0",
             "\tbuffer_load_dwordx4 v0, s[44:47], 0 offen lds"]
    assert len(_sgpr_hazards(lines)) == 1
    lines[2] = "\ts_nop 4"
    assert _sgpr_hazards(lines) == []
    # the scalar offset register is checked too
    lines = ["\tv_readlane_b32 s12, v255, 3", "\ts_nop 0", "\tbuffer_load_dwordx4 v0, s[44:47], s12 offen lds"]
    assert len(_sgpr_hazards(lines)) == 1
    # a writer in a predecessor block: reached by falling through a label ...
    lines = ["\tv_readfirstlane_b32 s46, v2", ".LBB0_3:", "\ts_nop 0",
             "\tbuffer_load_dwordx4 v0, s[44:47], 0 offen lds"]
    assert len(_sgpr_hazards(lines)) == 1
    # ... or by a branch to it from elsewhere (here a loop back edge after the load)
    lines = ["\ts_mov_b32 s46, 0", "\ts_nop 7", ".LBB0_3:", "\ts_nop 0",
             "\tbuffer_load_dwordx4 v0, s[44:47], 0 offen lds", "\ts_nop 7", "\tv_readfirstlane_b32 s46, v2",
             "\ts_cbranch_scc1 .LBB0_3"]
    assert len(_sgpr_hazards(lines)) == 1
    lines.insert(7, "\ts_nop 4")
    assert _sgpr_hazards(lines) == []
