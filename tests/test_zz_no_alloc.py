"""qmm_gemm_noalloc, the allocation-free entry point: through the C ABI its
output equals qmm_gemm_ex's (the same plan and kernels, so bit for bit) and
stays within the bound against the oracle, on two calls in a row, the second
with a smaller input; and a shape whose split needs more scratch than the
library holds is refused before anything is launched."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import assert_within_bound

qmm = pytest.importorskip("gemv_only_quant_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _both(case):
    d = case.to("cuda")
    Qt = qmm.pack(d.Q, case.N, case.K, case.w_bit)
    y_ws = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    y_na = torch.full_like(y_ws, float("nan"))
    ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    qmm.qmm_gemm_ex(d.x, Qt, d.scales, d.zeros, y_ws, case.M, case.N, case.K, case.w_bit,
                    case.group_size, workspace=ws)
    qmm.qmm_gemm_noalloc(d.x, Qt, d.scales, d.zeros, y_na, case.M, case.N, case.K, case.w_bit,
                         case.group_size)
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_na.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_equals_gemm_ex_on_two_calls():
    # a split plan (64 column tiles over K = 14336), then a smaller input whose
    # plan splits too (4 tiles, K = 4096): the second call reuses the scratch
    # the first left behind
    cases = [si.workload("int4_g128_asym_smalln_m16_k14336_n1024"),
             si.lowbit_case(16, 64, 4096, 4, 128, si.BF16, False, seed=81)]
    for i, case in enumerate(cases):
        assert qmm.qmm_workspace_bytes(case.M, case.N, case.K, case.w_bit, case.group_size) > 0
        y_ws, y_na = _both(case)
        assert np.array_equal(y_ws, y_na), f"call {i}"
        y_ref, a_ref = oracle.qmm_mt(*case.oracle_args())
        assert_within_bound(y_na, y_ref, a_ref, f"noalloc call {i}")


@pytest.mark.gpu
def test_noalloc_exact_probe_and_unsplit_shape():
    # exact arithmetic: bit-equal to the oracle; then a shape that needs no
    # scratch at all (200 column tiles of 128 fill the CUs unsplit), int8
    case = si.exact_lowbit_case(9, 32, 8192, 2, 64, si.F16, False, seed=82)
    y_ws, y_na = _both(case)
    assert np.array_equal(y_na.astype(np.float64), oracle.qmm(*case.oracle_args())[0])
    case = si.int8_case(16, 25600, 1024, si.BF16, seed=83)
    assert qmm.qmm_workspace_bytes(16, 25600, 1024, 8, 0) == 0
    y_ws, y_na = _both(case)
    assert np.array_equal(y_ws, y_na)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """Forced to 4 strips per workgroup and 16 splits (tuning overrides, read
    once per process, hence the child process), int8 M=640 N=768 K=4096
    would need 31 MB of partial tiles: refused before any HIP call."""
    code = (
        "import gemv_only_quant_amd as q\n"
        "A = 0x10000\n"
        "need = q.qmm_workspace_bytes(640, 768, 4096, 8, 0)\n"
        "assert need > q.QMM_NOALLOC_SCRATCH_BYTES, need\n"
        "st = q._lib.qmm_gemm_noalloc(A, A, A, None, A, q.QMM_F32, 640, 768, 4096, 8, 0,\n"
        "                             q.QMM_BF16, 0)\n"
        "assert st == q.QMM_ERR_UNSUPPORTED, st\n"
        "assert 'scratch' in q.qmm_last_error(), q.qmm_last_error()\n")
    env = dict(os.environ, QMM_SKINNY_NT="4", QMM_SKINNY_SPLITS="16")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
