"""Build libqmm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Always recompiles.  Objects are built in parallel into _build/ and linked
into gemv_only_quant_amd/libqmm.so.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # packed fp32 VALU ops stay off (hipcc only warns on the host pass)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fvisibility=hidden", "-Wall", "-Wno-unused-result", "-Wno-unknown-pragmas",
          "-I", os.path.join(ROOT, "include"),
          # the first 56 bytes of kernel arguments arrive in SGPRs at wave start
          # instead of through a scalar memory load (about 0.3 us of every
          # short launch); no kernel reads the grid size from the dispatch, a
          # load as well
          "-mllvm", "-amdgpu-kernarg-preload-count=16"]
SOURCES = ["qmm_api.cpp", "gemv_lowbit.hip", "gemv_tile.hip", "gemv_int8.hip", "repack.hip",
           "gemm_mfma.hip", "gemm_large.hip", "gemm_medium.hip", "ternary.hip", "ternary_large.hip",
           "quantize.hip"]


def _stale(src, obj):
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC)
                                        if h.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "qmm.h"))
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def _compile(src, verbose, incremental=False, defines=(), tag=""):
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    if incremental and not _stale(src, obj):
        return obj
    lang = ["-x", "hip"]
    cmd = [HIPCC] + COMMON + [f"-D{d}" for d in defines] + lang + ["-c", os.path.join(CSRC, src),
                                                                    "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    """Compile every source (or only stale ones with incremental=True) and link."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


PHASES_LIB = os.path.join(PKG, "libqmm_phases.so")


def build_phases(verbose: bool = False) -> str:
    """The phase-stamp library (measurement only, never loaded by the
    package): the product objects, with the tile GEMV built with
    QMM_PHASE_STAMPS (per-wave real-time stamps, a read-only reference
    kernel), plus calibrate.hip (a register-only MFMA loop).  Read by
    bench.py --phases."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [_compile(s, verbose, incremental=True) for s in SOURCES if s != "gemv_tile.hip"]
    objs.append(_compile("gemv_tile.hip", verbose, defines=("QMM_PHASE_STAMPS",), tag=".phases"))
    objs.append(_compile("calibrate.hip", verbose))
    tmp = PHASES_LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                   check=True)
    os.replace(tmp, PHASES_LIB)
    return PHASES_LIB


if __name__ == "__main__":
    if "--phases" in sys.argv:
        build_phases(verbose="-v" in sys.argv)
    else:
        build(verbose="-v" in sys.argv, incremental="-i" in sys.argv)
