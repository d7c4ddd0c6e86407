"""Wait states in front of the hand-issued MFMAs.

The GEMM and attention kernels issue their MFMAs from inline assembly, and the compiler's
hazard checks do not look inside inline assembly: it may write an MFMA operand with a VALU
instruction (a move, a rebuilt constant) right before the MFMA reads it. gfx950 needs two
wait states between a VALU write of a VGPR and an MFMA that reads it; with fewer the MFMA
can read the old value. This test compiles the device code of each kernel source to gfx950
assembly with the library's own flags and checks every MFMA against the instructions just
before it (s_nop n counts n + 1 wait states, every other instruction one)."""

import os
import re
import shutil
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_transformer_amd import build

KERNEL_SOURCES = ["tsp_gemm.hip", "tsp_attn.hip", "tsp_attn_bwd.hip"]


def _vregs(tok):
    tok = tok.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _instructions(text):
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        yield s


def valu_mfma_hazards(text, need=2):
    """(VALU instruction, MFMA) pairs where the MFMA reads a VGPR the VALU instruction wrote
    fewer than `need` wait states before."""
    ins = list(_instructions(text))
    found = []
    for k, s in enumerate(ins):
        if not s.startswith("v_mfma"):
            continue
        ops = s.split(None, 1)[1].split(",")
        srcs = set().union(*(_vregs(o) for o in ops[1:]))
        waits = 0
        for j in range(k - 1, max(k - 8, -1), -1):
            p = ins[j]
            if p.startswith("s_nop"):
                waits += int(p.split()[1]) + 1
                continue
            if waits >= need:
                break
            parts = p.split(None, 1)
            if parts[0].startswith("v_") and not parts[0].startswith("v_mfma") and len(parts) > 1:
                if _vregs(parts[1].split(",")[0]) & srcs:
                    found.append((p, s))
            waits += 1
    return found


def test_scanner_flags_a_planted_hazard():
    text = "v_mov_b32_e32 v5, v2\nv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
    assert len(valu_mfma_hazards(text)) == 1
    safe = "v_mov_b32_e32 v5, v2\ns_nop 1\nv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
    assert valu_mfma_hazards(safe) == []
    other = "v_mov_b32_e32 v12, v2\nv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
    assert valu_mfma_hazards(other) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_valu_write_right_before_an_mfma_reads_it():
    with tempfile.TemporaryDirectory() as td:
        def one(src):
            return src, open(build.device_asm(src, os.path.join(td, src + ".s"))).read()
        with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
            texts = list(ex.map(one, KERNEL_SOURCES))
    report = []
    for src, text in texts:
        assert "v_mfma" in text, src
        report += [f"{src}: {p}  ->  {m}" for p, m in valu_mfma_hazards(text)]
    assert not report, "\n".join(report[:20])
