"""The C ABI driven from C: a plain C program (tests/c/qmm_abi_call.c, no
Python or torch in its process) makes a successful qmm_gemv call on the
headline decode workload, whose every output is checked against the oracle,
and times eager calls (host cost of one call, device time per call)."""
import json
import os
import subprocess

import numpy as np
import pytest

import synth_inputs as si
from gpu_util import assert_within_bound, full_reference, log_parity

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "qmm_abi_call")


def test_gemv_called_from_c(tmp_path):
    assert os.path.exists(EXE), "tests/c/qmm_abi_call is not built (run the package build)"
    name = "int4_g128_asym_gemv_m1_k4096_n4096"
    case = si.workload(name)
    files = {}
    for key, arr in (("x", case.np_x()), ("Q", case.np_Q()), ("S", case.np_scales()),
                     ("Z", case.np_zeros())):
        files[key] = str(tmp_path / f"{key}.bin")
        np.ascontiguousarray(arr).tofile(files[key])
    ypath = str(tmp_path / "y.bin")
    cmd = [EXE, str(case.M), str(case.N), str(case.K), str(case.w_bit), str(case.group_size),
           str(case.x_dtype), files["x"], files["Q"], files["S"], files["Z"], ypath, "2000"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    timing = json.loads(r.stdout.strip().splitlines()[-1])
    y = np.fromfile(ypath, np.float32).reshape(case.M, case.N)
    y_ref, a_ref = full_reference(name)
    ratio = assert_within_bound(y, y_ref, a_ref, "qmm_gemv from C")
    log_parity(name + "_from_c", entry="qmm_gemv (C caller)", outputs=int(y.size),
               max_err_over_bound=ratio, **timing)
