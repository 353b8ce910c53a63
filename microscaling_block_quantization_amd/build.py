"""Build libmx.so (the HIP kernels and the C ABI of include/mx.h) for gfx950.

Every translation unit is compiled with hipcc for gfx950 only, then linked into
one shared library next to this file.  Flags that the bit-exact contract
relies on: no FMA contraction, IEEE fp32 division, fp32 denormals kept.
Packed fp32 instructions are disabled (they are not needed for bandwidth-bound
code and are kept out of every kernel).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmx.so")
# the measurement's context kernels (copy, stream, matrix-instruction loop):
# a library of their own, so that libmx.so exports only the method's ABI
CEIL_LIB = os.path.join(HERE, "libmx_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "quant_rows.hip", "quant_tiles.hip", "misc.hip", "gemm_mxfp4.hip", "gemm_lds.hip", "gemm_upcvt.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
         "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    if verbose and errs:
        print("\n".join(errs), flush=True)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEIL_SOURCES], CEIL_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
