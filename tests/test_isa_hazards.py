"""Lint of the gfx950 assembly of the MFMA kernels (CPU only: hipcc
cross-compiles the device code, nothing runs).

A VALU write of a VGPR followed by an MFMA that reads it as an operand needs
two wait states between them (CDNA3/CDNA4 ISA guides, data-dependency hazard
table). The compiler inserts them for instructions it knows to be VALU; an
inline-asm statement that writes a VGPR is opaque to it, which once left one
wait state before MFMA reads of unpacked codes and gave wrong results. This
test compiles each MFMA source with the library's own flags, walks every basic
block and checks that each MFMA operand register last written by a vector ALU
instruction in the same block was written at least two wait states earlier
(`s_nop n` counts n + 1, every other instruction 1)."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from group_wise_affine_qlinear_amd import build as qb

MFMA_SOURCES = ["gemm.hip", "gemm2.hip", "gemm3.hip", "skinny.hip"]
REQUIRED = 2


def _hipcc():
    try:
        return qb.hipcc()
    except RuntimeError:
        return None


def _vregs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(op, args):
    return int(args[0]) + 1 if op == "s_nop" else 1


def scan(asm):
    """(mfma count, list of violations) over all functions of an assembly file."""
    n_mfma, bad = 0, []
    func = None
    clock = 0
    last_valu = {}
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            # new function or basic block: forget what came before
            if line.startswith("_Z"):
                func = line[:-1]
            last_valu.clear()
            continue
        if line.startswith("."):
            continue
        parts = line.replace(",", " ").split()
        op, args = parts[0], parts[1:]
        if op.startswith("v_mfma"):
            n_mfma += 1
            for tok in args[1:4]:
                for r in _vregs(tok):
                    if r in last_valu and clock - last_valu[r] < REQUIRED:
                        bad.append((func, line, r, clock - last_valu[r]))
        clock += _wait_states(op, args)
        if op.startswith("v_") and not op.startswith("v_mfma") and args:
            for r in _vregs(args[0]):
                last_valu[r] = clock
    return n_mfma, bad


def test_scanner_flags_a_short_window():
    """The scanner itself: one instruction between a VALU write and an MFMA
    read is flagged, two are not."""
    short = "k:\nv_and_or_b32 v7, v0, s0, v12\ns_mov_b32 s1, s2\nv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], 0\n"
    ok = "k:\nv_and_or_b32 v7, v0, s0, v12\ns_mov_b32 s1, s2\ns_nop 0\nv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], 0\n"
    nop = "k:\nv_and_or_b32 v7, v0, s0, v12\ns_nop 1\nv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], 0\n"
    assert len(scan(short)[1]) == 1
    assert scan(ok)[1] == [] and scan(nop)[1] == []


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_mfma_operands_written_by_valu_have_two_wait_states(tmp_path):
    flags = [f for f in qb.COMMON_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")]

    def compile_one(src):
        out = tmp_path / (src + ".s")
        cmd = [_hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(qb.CSRC, src), "-o", str(out)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return src, out.read_text()

    with ThreadPoolExecutor(max_workers=len(MFMA_SOURCES)) as ex:
        results = list(ex.map(compile_one, MFMA_SOURCES))
    for src, asm in results:
        n, bad = scan(asm)
        assert n > 0, f"{src}: no MFMA found"
        assert not bad, (src, bad[:5])
