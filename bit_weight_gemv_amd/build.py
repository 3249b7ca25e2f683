"""Build libq4.so (gfx950) in-tree with hipcc.

    python -m bit_weight_gemv_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled in the device pass (-Xclang -target-feature -Xclang
-packed-fp32-ops), and linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libq4.so")
# A measurement reference kept out of libq4: the plain streaming read of a
# packed matrix's bytes (bench.py times it beside each GEMV).
FLOOR_SOURCE = "q4_floor.hip"
FLOOR_LIB = os.path.join(HERE, "libq4floor.so")
SOURCES = ["q4_api.cpp", "q4_pack.hip", "q4_gemv.hip", "q4_gemm_smalln.hip", "q4_gemm_rows4.hip", "q4_gather.hip", "q4_quant.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libq4.so failed")
    os.replace(tmp, LIB)
    tmp = FLOOR_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", "-x", "hip", os.path.join(CSRC, FLOOR_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build of libq4floor.so failed")
    os.replace(tmp, FLOOR_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
