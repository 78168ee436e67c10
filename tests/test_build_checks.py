"""Checks on the compiled GEMM kernels (CPU: hipcc cross-compiles for gfx950).

The bf16 GEMM's main loops wait for their operand loads with hand-written
`s_waitcnt vmcnt(N)` barriers: N counts the direct-to-LDS loads issued after
the ones the next step needs.  That count is only right if no other
vector-memory instruction sits in the loop -- a register spill reload
(scratch_load) or any other load would shift it, and the barrier would let a
stage be read before its data landed.  So every loop that issues MFMAs must
hold no scratch access and no vector-memory load except the buffer loads into
LDS.
"""
import os
import re
import subprocess
import sys

import pytest

from patch_merge_mlp_amd import build as b


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "vlb_gemm.s"
    src = os.path.join(b.CSRC, "vlb_gemm.hip")
    cmd = [b.HIPCC, *[f for f in b.compile_flags() if f != "-fPIC"], "--cuda-device-only", "-S",
           src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernels(asm):
    """(name, body) of every bf16 GEMM kernel in the assembly."""
    out = []
    for m in re.finditer(r"^(_Z\S*k_gemm_bf16\S*):", asm, re.M):
        start = m.end()
        end = asm.find("s_endpgm", start)
        out.append((m.group(1), asm[start:end]))
    return out


def loops(body):
    """Bodies of the innermost loops: the basic blocks that the assembler annotates
    as the loop header or as inside that header's loop, concatenated."""
    blocks = re.split(r"^(?=\.LBB\d+_\d+:|; %bb\.\d+:)", body, flags=re.M)
    groups = {}
    for blk in blocks:
        first = blk.split("\n", 1)[0]
        m = re.match(r"\.LBB(\d+_\d+):.*Loop Header", first)
        h = m.group(1) if m else None
        m2 = re.search(r"in Loop: Header=BB(\d+_\d+)", first)
        h = h or (m2.group(1) if m2 else None)
        if h:
            groups.setdefault(h, []).append(blk)
    return ["".join(v) for v in groups.values()]


def test_gemm_main_loops_hold_only_operand_loads(gemm_asm):
    ks = kernels(gemm_asm)
    assert len(ks) >= 10, "bf16 GEMM kernels not found in the assembly"
    checked = 0
    for name, body in ks:
        for lp in loops(body):
            if "v_mfma" not in lp:
                continue
            checked += 1
            assert "scratch_" not in lp, f"{name}: spill code inside an MFMA loop"
            for ins in re.findall(r"^\s+((?:buffer|global|flat)_load\S*)([^\n]*)", lp, re.M):
                assert ins[0].startswith("buffer_load") and " lds" in ins[1], \
                    f"{name}: {ins[0]}{ins[1]} inside an MFMA loop"
    assert checked >= len(ks), "expected one MFMA loop per kernel at least"


def test_gemm_main_loops_keep_accumulators_in_place(gemm_asm):
    """The accumulators live in AGPRs for the whole product; a copy between
    register files inside the main loop (register pressure pushing the
    allocator to shuffle them) costs hundreds of VALU slots per step and once
    slowed the gathered-operand Linear1 by 15%."""
    for name, body in kernels(gemm_asm):
        for lp in loops(body):
            if "v_mfma" not in lp:
                continue
            moves = re.findall(r"^\s+v_accvgpr_(?:mov|read|write)_b32", lp, re.M)
            assert not moves, f"{name}: {len(moves)} accumulator moves inside an MFMA loop"
