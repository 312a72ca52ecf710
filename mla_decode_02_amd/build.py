"""Build libmla_decode.so (HIP, gfx950) in-tree with hipcc.

    python mla_decode_02_amd/build.py   (a script: importing the package needs the built library)
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_decode.so")
# The measurement build: the same sources with the kernels' phase timestamps
# (MLA_PHASE_STAMPS=1, include/mla_decode_phases.h); used by bench.py --phases.
PHASES_LIB = os.path.join(PKG, "libmla_decode_phases.so")

# Every HIP translation unit is built for gfx950 only, without packed-fp32
# instruction selection (v_pk_{add,mul,fma}_f32).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments ahead of the parameter structs arrive in SGPRs at wave start
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


# The files the library is compiled from, in the order the digest reads them.
SOURCES = [os.path.join(CSRC, "mla_decode.hip"), os.path.join(CSRC, "mla_plan.cpp"),
           os.path.join(CSRC, "mla_plan.h"), os.path.join(INCLUDE, "mla_decode.h"),
           os.path.join(INCLUDE, "mla_decode_phases.h")]


def source_digest() -> str:
    """First 16 hex digits of SHA-256 over the library's source files. The build
    stores it in the library (mla_source_digest), so a library left over from
    other sources can be told apart from one built from the tree as it stands."""
    h = hashlib.sha256()
    for path in SOURCES:
        with open(path, "rb") as f:
            data = f.read()
        h.update(os.path.basename(path).encode() + b"\0" + len(data).to_bytes(8, "little") + data)
    return h.hexdigest()[:16]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False, phases: bool = True) -> str:
    """Compile the HIP kernels and the host planner and link the shared library
    (and, with phases, the measurement build beside it)."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    plan_o = os.path.join(obj_dir, "mla_plan.o")
    hip_o = os.path.join(obj_dir, "mla_decode.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f'-DMLA_SOURCE_DIGEST="{source_digest()}"',
          "-I", INCLUDE, "-c",
          os.path.join(CSRC, "mla_plan.cpp"), "-o", plan_o], verbose)
    _run(["hipcc", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "mla_decode.hip"),
          "-o", hip_o], verbose)
    tmp = LIB + ".tmp"
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, hip_o, plan_o], verbose)
    os.replace(tmp, LIB)
    if phases:
        phases_o = os.path.join(obj_dir, "mla_decode_phases.o")
        _run(["hipcc", *HIP_FLAGS, "-DMLA_PHASE_STAMPS=1", "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, "mla_decode.hip"), "-o", phases_o], verbose)
        tmp = PHASES_LIB + ".tmp"
        _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, phases_o, plan_o], verbose)
        os.replace(tmp, PHASES_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
