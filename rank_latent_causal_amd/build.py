"""Compile the gfx950 HIP library (libmla_absorb.so) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("mla_absorb.hip", "kda.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in os.listdir(os.path.join(HERE, "csrc")) if f.endswith(".h")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmla_absorb.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# device code generation flags, shared by the library and its assembly listing
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17",
         # packed fp32 VALU forms are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the one-wave-per-SIMD kernels unroll their 32-product phases
         # completely (operand arrays must stay in registers); the default
         # size limit for "#pragma unroll" loops is below that of the decode
         # kernel's phase, which then keeps a loop with dynamically
         # indexed operands and spills
         "-mllvm", "-pragma-unroll-threshold=65536",
         f"-I{INCLUDE}"]


def _compile(srcs, out_path: str, verbose: bool) -> str:
    cmd = [hipcc(), *FLAGS, "-fPIC", "-shared", *srcs, "-o", out_path + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def device_asm(src: str, out_path: str) -> str:
    """The gfx950 assembly that the library build generates for one source."""
    cmd = [hipcc(), *FLAGS, "--cuda-device-only", "-S", src, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    return out_path


def build(out_path: str = LIB, verbose: bool = False) -> str:
    """The MLA / KDA library."""
    _compile(SRCS, out_path, verbose)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
