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
# MFMA data hazards the hardware does not interlock (CDNA3/CDNA4 ISA, "required
# independent instructions"): a VALU write of a VGPR/AGPR an MFMA then reads
# (2 wait states), and an 8-pass XDL MFMA (v_mfma_f32_32x32x16_bf16) writing a
# register a non-MFMA instruction then reads (11).  The compiler pads its own
# MFMAs; the backward kernels issue some as inline asm, which it does not.
VALU_TO_MFMA_WAIT = 2
MFMA_TO_READ_WAIT = 11


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


def _regs(tok: str):
    tok = tok.strip()
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _split(t: str):
    parts = t.split(None, 1)
    args = [] if len(parts) < 2 else [a.strip() for a in re.split(r",(?![^\[]*\])", parts[1])]
    return parts[0], args


def _ends_block(t: str) -> bool:
    return t.endswith(":") or t.startswith(("s_cbranch", "s_branch", "s_setpc"))


def mfma_hazards(asm: str):
    """(kind, first, second, wait states) for every MFMA whose sources a VALU
    instruction wrote too shortly before, and every non-MFMA read of an MFMA
    result too shortly after.  Straight-line neighbours only."""
    ins = [t for t in (l.split(";")[0].strip() for l in asm.split("\n")) if t and not t.startswith(".")]
    bad = []
    for k, t in enumerate(ins):
        op, args = _split(t)
        if not op.startswith("v_mfma"):
            continue
        dst = _regs(args[0])
        srcs = set().union(*[_regs(a) for a in args[1:4]])
        ws = 0
        for j in range(k - 1, max(-1, k - 16), -1):
            u = ins[j]
            if _ends_block(u):
                break
            uop, uargs = _split(u)
            if uop == "s_nop":
                ws += int(uargs[0], 0) + 1
            else:
                if (uop.startswith("v_") and not uop.startswith("v_mfma") and uargs
                        and (_regs(uargs[0]) & srcs) and ws < VALU_TO_MFMA_WAIT):
                    bad.append(("valu->mfma", u, t, ws))
                    break
                ws += 1
            if ws >= VALU_TO_MFMA_WAIT:
                break
        ws = 0
        for j in range(k + 1, min(len(ins), k + 48)):
            u = ins[j]
            if _ends_block(u):
                break
            uop, uargs = _split(u)
            if uop == "s_nop":
                ws += int(uargs[0], 0) + 1
            elif uop.startswith("v_mfma"):
                ws += 1
            else:
                if uop.startswith(("ds_write", "global_store", "buffer_store", "flat_store")):
                    read = set().union(*[_regs(a) for a in uargs])
                else:
                    read = set().union(*[_regs(a) for a in uargs[1:]]) if uargs else set()
                if read & dst and ws < MFMA_TO_READ_WAIT:
                    bad.append(("mfma->read", t, u, ws))
                    break
                ws += 1
            if ws >= MFMA_TO_READ_WAIT:
                break
    return bad


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
    # D in {64, 128} x {unmasked, segment-masked} x {plain, 3D-rotary-embedded queries},
    # the unmasked ones again with work stealing and split items, the scheduled masked
    # kernel for the same D and query variants with and without a split last
    # round, its three set-up kernels (tile summaries, block counts, block
    # order), the work counters' reset, and the combine kernel of split items
    # for each D and item order
    assert len(sizes) == 28
    assert sizes == [0] * 28


def test_neighbourhood_kernel_wait_states_and_no_spills(natten_asm_text):
    n = sum(1 for t in _instructions(natten_asm_text.split("\n")) if t.startswith("global_load_lds"))
    assert n > 0
    assert lds_dma_hazards(natten_asm_text) == []
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", natten_asm_text)]
    assert sizes == [0, 0]  # D in {64, 128}


@pytest.fixture(scope="module")
def bwd_asm_text():
    return _compile("attn_bwd_kernel.hip")


def _functions(asm: str):
    """name -> list of lines, one entry per kernel in the file."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end].split("\n")
    return out


def _loops(lines):
    """(header index, back-edge index) of every loop, from the compiler's
    loop-header annotations and the last branch back to the header."""
    res = []
    for h, l in enumerate(lines):
        if "Loop Header" in l:
            lab = l.strip().split(":")[0]
            back = [k for k, t in enumerate(lines) if k > h and t.strip().startswith("s_") and
                    "branch" in t and t.strip().split()[-1] == lab]
            if back:
                res.append((h, max(back)))
    return res


def test_backward_kernels_wait_states_and_no_spills_in_loops(bwd_asm_text):
    """The pipelined dK/dV kernel runs at one wave per SIMD with all 512
    registers: its steady-state loop must not touch scratch (a few bytes
    spilled around the loop, once per workgroup, are tolerated)."""
    n = sum(1 for t in _instructions(bwd_asm_text.split("\n")) if t.startswith("global_load_lds"))
    assert n > 0
    assert lds_dma_hazards(bwd_asm_text) == []
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", bwd_asm_text)]
    # prep x {64, 128}; dK/dV and dQ x {64, 128} x {unmasked, masked}; block count and rank
    assert len(sizes) == 12
    assert max(sizes) <= 128
    for name, lines in _functions(bwd_asm_text).items():
        for h, b in _loops(lines):
            body = [t.strip() for t in lines[h:b + 1]]
            if any(t.startswith("v_mfma") for t in body):
                assert not any(t.startswith("scratch_") for t in body), name


@pytest.mark.parametrize("src", ["attn_fwd_kernel.hip", "natten_fwd_kernel.hip", "attn_bwd_kernel.hip"])
def test_mfma_wait_states(src, asm_text, natten_asm_text, bwd_asm_text):
    text = {"attn_fwd_kernel.hip": asm_text, "natten_fwd_kernel.hip": natten_asm_text,
            "attn_bwd_kernel.hip": bwd_asm_text}[src]
    assert sum(1 for t in _instructions(text.split("\n")) if t.startswith("v_mfma")) > 0
    assert mfma_hazards(text) == []


def test_mfma_checker_flags_planted_hazards():
    valu = "\n".join(["v_cvt_pk_bf16_f32 v47, v1, v2",
                      "v_mfma_f32_32x32x16_bf16 a[0:15], v[40:43], v[44:47], a[0:15]"])
    assert [b[0] for b in mfma_hazards(valu)] == ["valu->mfma"]
    assert mfma_hazards(valu.replace("\nv_mfma", "\ns_nop 1\nv_mfma")) == []
    read = "\n".join(["v_mfma_f32_32x32x16_bf16 v[0:15], v[40:43], a[44:47], v[0:15]",
                      "s_nop 7", "v_exp_f32_e32 v50, v3"])
    assert [b[0] for b in mfma_hazards(read)] == ["mfma->read"]
    assert mfma_hazards(read.replace("s_nop 7", "s_nop 7\ns_nop 3")) == []
    acc = "\n".join(["v_mfma_f32_32x32x16_bf16 a[0:15], v[40:43], v[44:47], a[0:15]",
                     "v_mfma_f32_32x32x16_bf16 a[0:15], v[48:51], v[44:47], a[0:15]"])
    assert mfma_hazards(acc) == []  # back-to-back accumulation is interlocked
