"""Build libthl.so (HIP kernels for gfx950 + host C++) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libthl.so")
PROBE_LIB = os.path.join(HERE, "libthl_probe.so")
SOURCES = ["gemm.hip", "layout.cpp", "gemm_inst_bf16.hip", "gemm_inst_f16.hip", "gemm_inst_i8.hip",
           "gemm_inst_e4m3.hip", "gemm_inst_e2m1.hip", "gemm_inst_bf16_ops.hip", "gemm_inst_f16_ops.hip",
           "gemm_inst_skinny.hip", "gemm_inst_e5m2.hip",
           "gemm_inst_mx8.hip", "gemm_inst_mx8e5.hip", "gemm_inst_mx8mix.hip", "gemm_inst_e4e5.hip",
           "gemm_inst_e5e4.hip", "gemm_inst_mxout16.hip", "gemm_inst_mxout8.hip", "convert.hip"]
HEADERS = ["convert.hpp", "gemm_args.hpp", "gemm_kernels.hpp", "gemm_launch.hpp", "gemm_skinny.hpp", "index_maps.hpp", "layout.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are switched off for every HIP compile.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [l for l in out.splitlines() if "not a recognized feature" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp])
    os.replace(tmp, LIB)
    # the measurement probe, a library of its own outside the GEMM boundary
    tmp = PROBE_LIB + ".tmp"
    subprocess.check_call([HIPCC] + FLAGS + ["-shared", "-x", "hip", os.path.join(CSRC, "mfma_probe.hip"), "-o", tmp],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
