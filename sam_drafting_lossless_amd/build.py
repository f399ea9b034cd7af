"""Compiles the HIP library for gfx950 in-tree.

    python -m sam_drafting_lossless_amd.build

produces ``sam_drafting_lossless_amd/libspecsam.so`` (the product library,
C ABI in ``include/specsam.h``) and ``libspecsam_harness.so`` (synthetic
target-model and measurement kernels used by tests and bench.py; not part of
the verification or drafting path).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

LIB = os.path.join(PKG, "libspecsam.so")
HARNESS_LIB = os.path.join(PKG, "libspecsam_harness.so")

LIB_SOURCES = ["api.hip", "stream.hip", "trunc.hip", "tree.hip", "verify.hip", "sam.hip"]
HARNESS_SOURCES = ["harness.hip"]

# Packed FP32 instructions are disabled: hipcc would otherwise form them from
# ordinary float code. Multiply-adds are fused only within one source
# expression (-ffp-contract=on, not hipcc's default "fast", which fuses across
# statements as the scheduler finds them): the rounding of every sum is then
# a property of the source, the same in each template instantiation of a
# kernel (so, for instance, the stream pass's plain and histogram variants
# give bit-identical partials for a row that is not truncated).
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-ffp-contract=on",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
OBJ_DIR = os.path.join(ROOT, "_build")


def _compile(sources, out, extra=()):
    """Compiles each source to an object in parallel, then links them."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    failed = [src for src, p in zip(sources, procs) if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
                    "-o", out + ".tmp"], check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> None:
    """Always recompiles both libraries."""
    _compile(LIB_SOURCES, LIB)
    if all(os.path.exists(os.path.join(CSRC, s)) for s in HARNESS_SOURCES):
        _compile(HARNESS_SOURCES, HARNESS_LIB)
    if verbose:
        print("built", LIB, HARNESS_LIB)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
