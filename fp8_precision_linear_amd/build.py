"""Compile the HIP sources into libfp8lin.so (gfx950), in-tree.

Each translation unit is compiled in parallel with hipcc, then linked into a
shared library next to this file.  Objects go to ``_build/`` at the repository
root.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8lin.so")
SOURCES = ["quant.hip", "gemm_fwd.hip", "gemm_dgrad.hip", "gemm_wgrad.hip", "gemm_group.hip", "swiglu.hip",
           "capi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain fp32 instructions only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
