"""Host-sanitized build of libcskv.so, for the CPU tests of the C ABI's
argument checks: the host code (validation, planning, error text) compiled
with AddressSanitizer and UndefinedBehaviorSanitizer, the device code as in
the product build (no GPU sanitizer). The library is loaded with clang's
sanitizer runtime preloaded (`runtime()`); it is never used on a GPU.
"""
from __future__ import annotations

import glob
import os

import build as _b   # the product build's compiler, flags and helpers

OUT_DIR = os.path.join(_b.ROOT, "_build", "cskv_hostsan")
LIB = os.path.join(OUT_DIR, "libcskv_hostsan.so")
_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def runtime() -> str:
    """clang's shared AddressSanitizer runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(_b.HIPCC), "..", "llvm", "lib", "clang", "*", "lib",
                                         "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("clang's libclang_rt.asan-x86_64.so was not found under the ROCm llvm tree")
    return os.path.realpath(hits[-1])


def build() -> str:
    """Builds (or reuses, when newer than every source) the sanitized library."""
    srcs = sorted(os.path.join(_b.CSRC, f) for f in os.listdir(_b.CSRC) if f.endswith(".hip"))
    deps = srcs + sorted(glob.glob(os.path.join(_b.CSRC, "*.h"))) + [os.path.join(_b.ROOT, "include", "cskv.h")]
    if os.path.exists(LIB) and os.path.getmtime(LIB) > max(os.path.getmtime(d) for d in deps):
        return LIB
    flags = [f for f in _b.FLAGS if f != "-O3"] + ["-O1", "-g"] + _SAN
    objs = _b.compile_sources(srcs, os.path.join(OUT_DIR, "obj"), flags)
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    _b._run([_b.HIPCC, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-shared-libsan", *_SAN[:4], "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB
