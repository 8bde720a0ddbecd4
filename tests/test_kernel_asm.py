"""Static checks on the gfx950 assembly of the attention kernel (CPU only).

The kernel issues its global->LDS tile copies as inline asm, which the
compiler's hazard recogniser does not look inside.  GFX9 requires five wait
states between a VALU instruction that writes an SGPR (for instance a
v_readlane reloading a spilled SGPR) and a vector-memory instruction that
reads it as its address base or M0, and one between an SALU write of M0 and an
LDS DMA.  A missing wait lets the copy use a stale base address.  This test
compiles the kernel to assembly with the library's own flags and checks every
LDS DMA against both rules, and that no kernel variant spills to scratch.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from spatiotemporal_attention_amd import build as B

VALU_SGPR_WAIT = 5
SALU_M0_WAIT = 1


def _compile(src):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
               os.path.join(B.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read()


@pytest.fixture(scope="module")
def asm_text():
    return _compile("attn_fwd_kernel.hip")


@pytest.fixture(scope="module")
def natten_asm_text():
    return _compile("natten_fwd_kernel.hip")


def _sregs(tok: str):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    if tok == "m0":
        return {"m0"}
    return set()


def _instructions(lines):
    for l in lines:
        t = l.strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            yield t


def lds_dma_hazards(asm: str):
    """(instruction, offending writer, wait states) for every LDS DMA that
    follows a VALU write of its SGPR base / M0, or an SALU write of M0, too
    closely.  Only straight-line predecessors are examined."""
    ins = list(_instructions(asm.split("\n")))
    bad = []
    for i, t in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        parts = t.replace(",", " ").split()
        reads = _sregs(parts[2]) | {"m0"}
        ws = 0
        for j in range(i - 1, max(-1, i - 16), -1):
            u = ins[j]
            op = u.split()[0]
            if op == "s_nop":
                ws += int(u.split()[1], 0) + 1
            else:
                dst = u.replace(",", " ").split()[1] if len(u.split()) > 1 else ""
                written = _sregs(dst) & reads
                if written and op.startswith("v_") and ws < VALU_SGPR_WAIT:
                    bad.append((t, u, ws))
                    break
                if "m0" in written and op.startswith("s_") and ws < SALU_M0_WAIT:
                    bad.append((t, u, ws))
                    break
                ws += 1
            if ws >= VALU_SGPR_WAIT or op.startswith(("s_cbranch", "s_branch")):
                break
    return bad


def test_every_lds_dma_has_its_wait_states(asm_text):
    n = sum(1 for t in _instructions(asm_text.split("\n")) if t.startswith("global_load_lds"))
    assert n > 0
    assert lds_dma_hazards(asm_text) == []


def test_checker_flags_a_planted_hazard():
    planted = "\n".join([
        "v_readlane_b32 s9, v169, 1",
        "s_add_i32 m0, s4, 0x400",
        "s_nop 0",
        "global_load_lds_dwordx4 v134, s[8:9]",
    ])
    assert len(lds_dma_hazards(planted)) == 1
    fixed = planted.replace("s_nop 0", "s_nop 4")
    assert lds_dma_hazards(fixed) == []


def test_no_kernel_spills_to_scratch(asm_text):
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", asm_text)]
    assert len(sizes) == 4  # D in {64, 128} x {unmasked, segment-masked}
    assert sizes == [0, 0, 0, 0]


def test_neighbourhood_kernel_wait_states_and_no_spills(natten_asm_text):
    n = sum(1 for t in _instructions(natten_asm_text.split("\n")) if t.startswith("global_load_lds"))
    assert n > 0
    assert lds_dma_hazards(natten_asm_text) == []
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", natten_asm_text)]
    assert sizes == [0, 0]  # D in {64, 128}


@pytest.fixture(scope="module")
def bwd_asm_text():
    return _compile("attn_bwd_kernel.hip")


def test_backward_kernels_wait_states_and_no_spills(bwd_asm_text):
    n = sum(1 for t in _instructions(bwd_asm_text.split("\n")) if t.startswith("global_load_lds"))
    assert n > 0
    assert lds_dma_hazards(bwd_asm_text) == []
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", bwd_asm_text)]
    assert len(sizes) == 10  # prep x {64, 128}; dK/dV and dQ x {64, 128} x {unmasked, masked}
    assert sizes == [0] * 10
