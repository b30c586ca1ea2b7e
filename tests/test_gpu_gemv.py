"""GPU parity of qmm_gemv (decode / skinny path, canonical layout) against
the oracle: tolerance on random data, bit-exact on the exact-arithmetic and
one-hot probes, full-size workloads in the launch configuration the
benchmark times."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import assert_within_bound, cpu, full_reference, log_parity

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu


def run_gemv(case, ws=None):
    d = case.to("cuda")
    y = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    qmm.qmm_gemv(d.x, d.Q, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                 case.group_size, workspace=ws)
    return cpu(y)


LOWBIT = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (1, 64, 128, 4, 128, si.F16, False),
    (1, 100, 384, 4, 128, si.BF16, False),     # ragged last column tile
    (3, 256, 1024, 4, 64, si.F16, True),
    (7, 192, 2048, 4, 128, si.BF16, False),    # K split over workgroups
    (16, 128, 4096, 4, 128, si.F16, False),
    (2, 320, 512, 4, 32, si.F16, False),
    (5, 64, 1024, 4, 256, si.BF16, True),
    (1, 128, 1024, 2, 64, si.F16, False),
    (4, 96, 2048, 2, 64, si.BF16, False),
    (9, 64, 512, 2, 128, si.F16, True),
    (1, 68, 256, 2, 32, si.BF16, False),
    (16, 64, 1024, 2, 256, si.F16, False),
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", LOWBIT)
def test_gemv_lowbit_within_bound(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=1 + M * 7 + N + K + w_bit)
    y = run_gemv(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemv w{w_bit} M{M} N{N} K{K}")


INT8 = [  # M, N, K, x_dtype
    (1, 1, 16, si.BF16),
    (1, 7, 1040, si.F16),     # K not a multiple of the 1024-wide lane sweep
    (2, 33, 2048, si.BF16),
    (5, 64, 512, si.F16),
    (16, 40, 4096, si.BF16),
    (3, 4100, 64, si.BF16),   # many rows per wave
    (8, 9000, 128, si.F16),
]


@pytest.mark.parametrize("M,N,K,xdt", INT8)
def test_gemv_int8_within_bound(M, N, K, xdt):
    case = si.int8_case(M, N, K, xdt, seed=M + N + K)
    y = run_gemv(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemv int8 M{M} N{N} K{K}")


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", [
    (1, 128, 1024, 4, 128, si.F16, False),
    (6, 64, 2048, 4, 64, si.BF16, True),
    (3, 96, 1024, 2, 64, si.BF16, False),
    (16, 64, 4096, 4, 128, si.BF16, False),
])
def test_gemv_lowbit_exact_probe_bit_exact(M, N, K, w_bit, gs, xdt, sym):
    case = si.exact_lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=K + M)
    y = run_gemv(case)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("M,N,K,xdt", [(1, 64, 1024, si.BF16), (4, 48, 4096, si.F16),
                                       (16, 16, 2048, si.BF16)])
def test_gemv_int8_exact_probe_bit_exact(M, N, K, xdt):
    case = si.exact_int8_case(M, N, K, xdt, seed=N)
    y = run_gemv(case)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemv_one_hot_reproduces_weights():
    """x = e_k makes y the k-th row of W, bit for bit (weights stay exact in
    fp32 on this path); sweeping k over group edges reads W back."""
    M, N, K = 16, 128, 1024
    base = si.lowbit_case(M, N, K, 4, 128, si.F16, False, seed=31)
    ks = [0, 1, 7, 8, 127, 128, 129, 255, 511, 512, 640, 767, 895, 1000, 1022, 1023]
    case = si.one_hot(base, ks)
    y = run_gemv(case)
    W = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), N, K, 4, 128)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], W[k]), k


def test_successive_calls_of_different_shapes():
    for i, (M, N, K) in enumerate([(2, 256, 4096), (1, 512, 2048), (2, 256, 4096), (3, 64, 8192)]):
        case = si.lowbit_case(M, N, K, 4, 128, si.F16, False, seed=50 + i)
        y = run_gemv(case)
        y_ref, a_ref = oracle.qmm(*case.oracle_args())
        assert_within_bound(y, y_ref, a_ref, f"call {i}")


def test_zero_m_leaves_output_untouched():
    case = si.lowbit_case(1, 64, 128, 4, 128, si.F16, False, seed=3).to("cuda")
    y = torch.full((1, 64), 7.0, device="cuda")
    qmm.qmm_gemv(case.x, case.Q, case.scales, case.zeros, y, 0, 64, 128, 4, 128)
    assert np.all(cpu(y) == 7.0)


# ------------------------------------------------------------ full sizes
@pytest.mark.parametrize("name", ["int8_gemv_m1_k1024_n1024",
                                  "int4_g128_asym_gemv_m1_k4096_n4096",
                                  "int4_pc_sym_gemv_m1_k4096_n4096",
                                  # the M = 16 workloads through the GEMV path, a
                                  # cross-check of the matrix-core path
                                  "int8_skinny_m16_k4096_n14336",
                                  "int4_g128_sym_m16_k8192_n8192"])
def test_gemv_full_size_all_outputs(name):
    """Every output of the full-size workload, in the launch configuration the
    benchmark times, against the oracle's."""
    case = si.workload(name)
    y = run_gemv(case)
    y_ref, a_ref = full_reference(name)
    ratio = assert_within_bound(y, y_ref, a_ref, name)
    log_parity(name, entry="qmm_gemv", outputs=int(y.size), max_err_over_bound=ratio)
