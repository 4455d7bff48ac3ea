"""Build libsage.so (the gfx950 HIP library behind include/sage.h) in-tree.

Every translation unit is compiled with hipcc for gfx950 only, in parallel,
then linked into ``quantized_attention_channel_amd/libsage.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsage.so")
SOURCES = ["sage_abi.hip", "quant_kernels.hip", "attn_kernel.hip", "fp4_kernels.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Werror",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature: drop that warning only
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, defines=(), lib: str = LIB, obj: str = OBJ) -> str:
    """Compile every source for gfx950 and link `lib`. `defines` (NAME=VALUE
    strings) build a variant, e.g. the phase-trace diagnostic library, into its
    own object directory and library path."""
    os.makedirs(obj, exist_ok=True)
    objs = [os.path.join(obj, s.replace(".hip", ".o")) for s in SOURCES]
    dflags = [f"-D{d}" for d in defines]
    cmds = [[HIPCC, *FLAGS, *dflags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = lib + ".tmp"
    # -z defs: a symbol left undefined (e.g. a kernel stub the host pass did not
    # emit) fails the link here instead of the first dlopen
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]))
    os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
