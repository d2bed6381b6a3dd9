"""Compile forward_from_c.c, the plain C caller of the C ABI that the GPU
tests run, next to its source (gcc, C11, linked against the in-tree
libmoe_fp8.so and the HIP runtime)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "fp8_block_quantized_group_amd")
SRC = os.path.join(HERE, "forward_from_c.c")
EXE = os.path.join(HERE, "forward_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", EXE + ".tmp",
           "-L", PKG, "-lmoe_fp8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../fp8_block_quantized_group_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
