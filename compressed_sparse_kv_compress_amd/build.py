"""Builds libcskv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled with hipcc for gfx950 only; packed fp32 instructions
are disabled (-packed-fp32-ops). Objects go to <repo>/_build/cskv.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcskv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx feature name; that warning is expected
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def compile_sources(srcs, objdir, flags, jobs=None):
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        futs = [ex.submit(_run, [HIPCC, *flags, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            msg = f.result()
            if msg.strip():
                print(msg, file=sys.stderr)
    return objs


def link_shared(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = compile_sources(srcs, os.path.join(ROOT, "_build", "cskv"), FLAGS)
    link_shared(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
