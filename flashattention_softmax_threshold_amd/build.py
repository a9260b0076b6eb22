"""Build libblasst.so (HIP kernels for gfx950 + the C-ABI host code) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libblasst.so")
SOURCES = ["api.cpp", "prefill.hip", "prefill_mfma.hip", "decode.hip", "mla.hip", "mla128.hip",
           "noalloc.hip"]
ARCH = os.environ.get("BLASST_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Keep the compiler from forming packed fp32 instructions on its own.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file additions. The 64-head MLA decode kernel keeps its O accumulator in ordinary VGPRs
# (MFMA C/D operands in the VGPR form) and its query fragments in AGPRs: with the default choice
# the compiler copies the 128 accumulator registers out of AGPRs at the top of every key tile.
# The 128-head kernel holds O^T in a0 .. a255 through inline assembly only; every MFMA the
# compiler emits there must be in the VGPR form.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"mla.hip": VGPR_FORM, "mla128.hip": VGPR_FORM}
# Files whose kernels own the accumulation registers through inline assembly: the build fails if
# the compiled code uses one outside those statements (a spill there would overwrite O^T).
AGPR_OWNERS = {"mla128.hip"}
_AGPR_OPERAND = re.compile(r"(?<![\w.])a(\d+|\[\d+:\d+\])(?!\w)")


def _check_agprs(src: str) -> None:
    """Compile src to device assembly and reject any accumulation-register operand outside the
    inline-assembly statements."""
    asm = os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-S", "--offload-device-only",
           os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    inside, bad = False, []
    with open(asm) as f:
        for ln, line in enumerate(f, 1):
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                inside = True
            elif t.startswith(";;#ASMEND"):
                inside = False
            elif not inside and t and t[0] not in ";.":
                parts = t.split(";")[0].split(None, 1)
                if len(parts) == 2 and _AGPR_OPERAND.search(parts[1]):
                    bad.append(f"{asm}:{ln}: {t}")
    if bad:
        raise RuntimeError(f"{src}: compiler-generated code uses accumulation registers:\n" +
                           "\n".join(bad[:10]))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if src in AGPR_OWNERS:
        _check_agprs(src)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
