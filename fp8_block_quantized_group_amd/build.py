"""Build the gfx950 HIP library ``libmoe_fp8.so`` in-tree with hipcc.

    python -m fp8_block_quantized_group_amd.build

Each source compiles to its own object (the grouped GEMM once per scale
scheme), in parallel, and the objects link into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_fp8.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["moe_api.hip", "quant_kernels.hip", "route_kernels.hip", "reduce_kernels.hip"]
# the grouped GEMM's scale schemes (kQuantUe8m0, kQuantF32, kQuantBf16,
# kQuantMxfp8, kSchemeMxfp8W4)
GEMM_SCHEMES = [0, 1, 2, 3, 4]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no hand-written or compiler-formed packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return res.returncode, out, cmd


def build(verbose: bool = False, extra_flags=(), lib: str = LIB) -> str:
    """Compile every HIP source and link one shared library; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ_DIR, s.replace(".hip", ".o"))
        jobs.append([HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, s), "-o", obj])
    for sc in GEMM_SCHEMES:
        obj = os.path.join(OBJ_DIR, f"grouped_gemm_s{sc}.o")
        jobs.append([HIPCC, *FLAGS, *extra_flags, f"-DMOE_GEMM_SCHEME={sc}", "-c",
                     os.path.join(CSRC, "grouped_gemm.hip"), "-o", obj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, jobs))
    for rc, out, cmd in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
    objs = [cmd[-1] for cmd in jobs]
    tmp = lib + ".tmp"
    rc, out, cmd = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}): {' '.join(cmd)}\n{out}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
