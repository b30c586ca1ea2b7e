"""Compile tests/c/qmm_abi_call.c (plain C, host only) against libqmm.so and
the HIP runtime.  Test infrastructure: the GPU test that drives the C ABI
from C runs the program this builds.  Always recompiles."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "qmm_abi_call")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "gemv_only_quant_amd")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", EXE + ".tmp", os.path.join(HERE, "qmm_abi_call.c"),
           "-L", pkg, "-lqmm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gemv_only_quant_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
