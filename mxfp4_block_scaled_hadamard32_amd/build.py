"""Builds libmx.so (the HIP kernels and the C ABI of include/mx.h) for gfx950 with hipcc.

The library is built in-tree, next to this file, so it travels with the source tree.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmx.so")
SOURCES = ["mx_api.hip", "quant.hip", "gemm.hip"]
# measurement aid for the matrix-core roofline (include/mx_probe.h), a library of its own
PROBE_LIB = os.path.join(HERE, "libmx_probe.so")
PROBE_SOURCES = ["mfma_probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                      # fp32 rounding exactly as written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 VALU ops
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(verbose: bool = False, extra=()) -> str:
    compile_lib(LIB, SOURCES, verbose, extra)
    compile_lib(PROBE_LIB, PROBE_SOURCES, verbose, extra)
    return LIB


def compile_lib(lib: str, sources, verbose: bool = False, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
