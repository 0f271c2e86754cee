"""Static check of the hand-placed MFMAs in the generated gfx950 assembly.

The one-wave-per-SIMD kernels issue some matrix products from inline
assembly, which the compiler's hazard recognizer does not see.  A VALU
instruction that writes a source register (A, B or C) of such a product
must be at least two wait states ahead of it, or the product can read the
old value; the kernels keep such operands out of VALU reach (loaded from
LDS, or pinned and separated by an explicit gap).  This test compiles the
library sources to assembly with the library's own flags and rejects any
inline-assembly product with a VALU write of one of its sources among the
three issue slots before it (s_nop n counting n + 1).  Products the
compiler emits from builtins are its own responsibility and not checked."""
import os
import re
import shutil
import tempfile

import pytest

from rank_latent_causal_amd import build as hip_build

GAP = 3


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def _instructions(lines):
    """(opcode, operands, from inline asm) per instruction, per kernel."""
    kernels, cur, in_asm = {}, None, False
    for l in lines:
        m = re.match(r"^(_Z\S+):", l)
        if m:
            cur = kernels.setdefault(m.group(1), [])
            continue
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if cur is None or not t or t.startswith((".", ";")):
            continue
        t = t.split(";")[0].strip()
        op = t.split()[0]
        args = [a for a in re.split(r",\s*|\s+", t[len(op):].strip()) if a]
        cur.append((op, args, in_asm))
    return kernels


def _violations(ins):
    bad = []
    for i, (op, args, in_asm) in enumerate(ins):
        if not (in_asm and op.startswith("v_mfma")):
            continue
        srcs = set().union(*(_regs(a) for a in args[1:4]))
        k, seen = i - 1, 0
        while k >= 0 and seen < GAP:
            op2, a2, _ = ins[k]
            if op2 == "s_nop":
                seen += int(a2[0], 0) + 1 if a2 else 1
            else:
                seen += 1
                if op2.startswith("v_") and not op2.startswith("v_mfma") and a2 and _regs(a2[0]) & srcs:
                    bad.append(f"{op2} {' '.join(a2)} -> {op} {' '.join(args)}")
            k -= 1
    return bad


def test_checker_flags_a_planted_hazard():
    """The scan itself: a VALU write right before an assembly product."""
    lines = ["_Zk:", "\tv_mov_b32_e32 v5, v9", ";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], 0",
             ";;#ASMEND", "\tv_mov_b32_e32 v20, v9", "\ts_nop 2", ";;#ASMSTART",
             "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[8:11], a[0:15]", ";;#ASMEND"]
    bad = _violations(_instructions(lines)["_Zk"])
    assert len(bad) == 1 and "v5" in bad[0]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_inline_asm_products_have_no_valu_source_hazard():
    src = os.path.join(hip_build.HERE, "csrc", "mla_absorb.hip")
    with tempfile.TemporaryDirectory() as d:
        lines = open(hip_build.device_asm(src, os.path.join(d, "mla_absorb.s"))).read().split("\n")
    kernels = _instructions(lines)
    n_asm = sum(1 for ins in kernels.values() for op, _, a in ins if a and op.startswith("v_mfma"))
    assert n_asm > 1000, "expected the one-wave-per-SIMD kernels' assembly products"
    bad = {k: v for k, v in ((k, _violations(ins)) for k, ins in kernels.items()) if v}
    assert not bad, "\n".join(f"{k}: {v[:3]}" for k, v in bad.items())
