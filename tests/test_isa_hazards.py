"""Static checks of the gfx950 assembly the library's sources compile to.

The kernels issue most matrix products through inline assembly, which the
compiler's hazard tracking does not look into, so the built code is checked
for both directions:
- no vector-ALU instruction writes a register that a matrix instruction then
  reads within fewer than two wait states;
- no instruction other than a matrix product reads the result of an
  inline-assembly product within fewer than 18 wait states (the sources
  place 21; compiler-selected products are left to the compiler's own
  tracking) before the result is overwritten.
Each instruction counts one wait state, ``s_nop n`` counts n + 1 and an
intervening matrix product 8.  It also checks that no packed fp32 vector
instruction was emitted (the build turns the feature off).

CPU only: compiles every source with the library's own flags and
``--cuda-device-only -S`` (about a minute on 8 cores).
"""

from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from exact_io_aware_fa2_amd import _build as b

REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)$")


def _regs(tok: str) -> set[str]:
    m = REG.match(tok.strip())
    if not m:
        return set()
    if m.group(1):
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {f"{m.group(4)}{m.group(5)}"}


def _instructions(body: str, with_asm: bool = False):
    in_asm = False
    for line in body.split("\n"):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        yield (parts[0], ops, in_asm) if with_asm else (parts[0], ops)


def _is_vector_write(op: str) -> bool:
    return (op.startswith("v_") and "mfma" not in op and not op.startswith(("v_readfirstlane", "v_readlane",
                                                                             "v_cmp")))


def hazards(asm: str):
    """(kernel, writer, reader, wait states) for each vector write read too early by a product."""
    found = []
    for m in re.finditer(r"^(_ZN2fa\S+):", asm, re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)
        insts = list(_instructions(asm[start:end]))
        for i, (op, ops) in enumerate(insts):
            if not _is_vector_write(op) or not ops:
                continue
            dst = _regs(ops[0])
            if not dst:
                continue
            ws = 0
            for op2, ops2 in insts[i + 1:i + 4]:
                if "mfma" in op2:
                    src = set().union(*(_regs(t) for t in ops2[1:])) if len(ops2) > 1 else set()
                    if dst & src:
                        found.append((m.group(1), f"{op} {ops[0]}", op2, ws))
                        break
                ws += int(ops2[0], 0) + 1 if op2 == "s_nop" else 1
                if ws >= 2:
                    break
    return found


def result_hazards(asm: str, need: int = 18):
    """(kernel, product, reader, wait states) for each read of an inline-assembly
    product's result by a non-product instruction within `need` wait states."""
    found = []
    for m in re.finditer(r"^(_ZN2fa\S+):", asm, re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)
        insts = list(_instructions(asm[start:end], with_asm=True))
        for i, (op, ops, in_asm) in enumerate(insts):
            if "mfma" not in op or not ops or not in_asm:
                continue
            dst = _regs(ops[0])
            ws = 0
            for op2, ops2, _ in insts[i + 1:i + 40]:
                if op2.startswith(("s_cbranch", "s_branch")) or op2 == "s_barrier":
                    break
                if "mfma" in op2:
                    if ops2 and dst & _regs(ops2[0]):
                        break  # accumulated into or overwritten by a later product
                    ws += 8
                else:
                    src = set().union(*(_regs(t) for t in ops2[1:])) if len(ops2) > 1 else set()
                    if dst & src:
                        found.append((m.group(1), op, f"{op2} {','.join(ops2[:2])}", ws))
                        break
                    ws += int(ops2[0], 0) + 1 if op2 == "s_nop" else 1
                if ws >= need:
                    break
    return found


@pytest.fixture(scope="module")
def assembly():
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in b.SOURCES:
            dst = os.path.join(tmp, src.replace(".hip", ".s"))
            cmd = [cc, *b.compile_flags(), "--cuda-device-only", "-S", os.path.join(b.CSRC, src), "-o", dst]
            procs.append((src, dst, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        for src, dst, p in procs:
            text, _ = p.communicate()
            assert p.returncode == 0, (src, text.decode(errors="replace")[-2000:])
            with open(dst) as f:
                out[src] = f.read()
    return out


def test_scan_catches_a_planted_hazard():
    planted = ("_ZN2fa1xEv:\n\tv_accvgpr_write_b32 a3, v7\n"
               "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], 0\n.Lfunc_end0:\n")
    assert hazards(planted) == [("_ZN2fa1xEv", "v_accvgpr_write_b32 a3", "v_mfma_f32_32x32x16_bf16", 0)]
    spaced = planted.replace("\tv_mfma", "\ts_nop 1\n\tv_mfma")
    assert hazards(spaced) == []
    one = planted.replace("\tv_mfma", "\ts_waitcnt lgkmcnt(0)\n\tv_mfma")
    assert [h[3] for h in hazards(one)] == [1]


def test_scan_catches_an_early_result_read():
    planted = ("_ZN2fa1xEv:\n\t;;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]\n"
               "\t;;#ASMEND\n\ts_nop 6\n\tv_accvgpr_mov_b32 a207, a31\n.Lfunc_end0:\n")
    assert [h[3] for h in result_hazards(planted)] == [7]
    assert result_hazards(planted.replace("s_nop 6", "s_nop 7\n\ts_nop 7\n\ts_nop 4")) == []
    # a compiler-selected product (no asm markers) is the compiler's to guard
    assert result_hazards(planted.replace(";;#ASMSTART", ";").replace(";;#ASMEND", ";")) == []


def test_no_early_read_of_a_product_result(assembly):
    bad = {src: result_hazards(asm) for src, asm in assembly.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


def test_no_vector_write_feeds_a_product_too_early(assembly):
    bad = {src: hazards(asm) for src, asm in assembly.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


def test_no_packed_fp32_vector_instructions(assembly):
    pat = re.compile(r"^\s+v_pk_(add|mul|fma|mov)_f32\b", re.M)
    found = {src: len(pat.findall(asm)) for src, asm in assembly.items()}
    assert not any(found.values()), found
