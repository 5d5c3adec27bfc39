"""Compile the HIP library for gfx950 (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mla_decode.hip")
SOURCES = [SRC, os.path.join(HERE, "csrc", "mla_append.hip"), os.path.join(HERE, "csrc", "mla_absorb.hip")]
LIB = os.path.join(HERE, "libmla_decode.so")
# read-bandwidth probes for the benchmark (not part of the decode path)
PROBE_SRC = os.path.join(HERE, "csrc", "hbm_probe.hip")
PROBE_LIB = os.path.join(HERE, "libmla_probe.so")
# the same library with AddressSanitizer and UndefinedBehaviorSanitizer in
# its host code only (the GPU code is built as usual), for the host-side
# tests; loaded with the sanitizer runtime preloaded
HOSTSAN_LIB = os.path.join(HERE, "libmla_decode_hostsan.so")
HOSTSAN_FLAGS = [
    "-O1", "-g",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # never emit packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(sources, lib, verbose, extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"  # host pass does not know the GPU feature
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "packed-fp32" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """Compile ``libmla_decode.so`` (and the benchmark's ``libmla_probe.so``);
    returns the decode library's path.  Always recompiles."""
    _compile(SOURCES, LIB, verbose, extra)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    # MFMAs issued from inline asm: the compiler cannot see their operand
    # hazards, so the compiled code is checked for them
    from mla_latent_cache_absorbed_amd import isa_check
    probs = []
    for src in SOURCES:
        probs += isa_check.check_source(src, HIPCC, [*FLAGS, *extra])
    if probs:
        raise RuntimeError("MFMA operand hazards in the compiled code:\n" + "\n".join(probs))
    return LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), or "" if it is not installed."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm")
    for pat in ("lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"):
        hits = sorted(glob.glob(os.path.join(llvm, pat)))
        if hits:
            return hits[-1]
    return ""


def build_host_sanitized(verbose: bool = False) -> str:
    """Compile ``libmla_decode_hostsan.so`` unless it is newer than every
    source and header; returns its path."""
    deps = SOURCES + [os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))]
    if os.path.exists(HOSTSAN_LIB) and os.path.getmtime(HOSTSAN_LIB) > max(map(os.path.getmtime, deps)):
        return HOSTSAN_LIB
    _compile(SOURCES, HOSTSAN_LIB, verbose, HOSTSAN_FLAGS)
    return HOSTSAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
