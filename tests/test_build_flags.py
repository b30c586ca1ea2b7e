"""The build's code-generation flags, checked on the CPU: every HIP source is
compiled with packed fp32 VALU instructions disabled and with the kernel
arguments preloaded into SGPRs, and one kernel file compiled with those flags
shows both in its gfx950 assembly."""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "qmm_build", os.path.join(ROOT, "gemv_only_quant_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_common_flags():
    b = _build_module()
    flags = b.COMMON
    i = flags.index("-packed-fp32-ops")
    assert flags[i - 1] == "-Xclang" and flags[i - 2] == "-target-feature"
    assert "-amdgpu-kernarg-preload-count=16" in flags
    assert flags[flags.index("-amdgpu-kernarg-preload-count=16") - 1] == "-mllvm"
    assert f"--offload-arch={b.ARCH}" in flags and b.ARCH == "gfx950"


@pytest.mark.skipif(not os.path.exists(_build_module().HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_kernel_assembly(tmp_path):
    """gemv_int8.hip to gfx950 assembly with the build's flags: every kernel
    descriptor preloads its arguments, and no packed fp32 add / mul / fma
    appears."""
    b = _build_module()
    out = tmp_path / "gemv_int8.s"
    flags = [f for f in b.COMMON if f not in ("-fPIC",)]
    cmd = [b.HIPCC] + flags + ["-x", "hip", "--cuda-device-only", "-S", "-o", str(out),
                               os.path.join(b.CSRC, "gemv_int8.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    kernels = asm.count(".amdhsa_kernel ")
    assert kernels > 0
    preload = [l for l in asm.splitlines() if ".amdhsa_user_sgpr_kernarg_preload_length" in l]
    assert len(preload) == kernels
    assert all(int(l.split()[-1]) > 0 for l in preload)
    for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
        assert op not in asm, op
