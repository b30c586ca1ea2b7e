"""GPU parity of the int8 x ternary product (liger-kernel mm_int8int2): the
repack is bit-exact against the oracle's layout reference and inverts
exactly; the product is integer arithmetic, so every output (all of them, at
full size too) must equal the oracle's exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import cpu

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(16, 256), (48, 512), (272, 1280)])
def test_t2_pack_bit_exact_and_inverse(N, K):
    case = si.t2_case(1, N, K, seed=N + K, codes=4)
    Wp = case.Wp.cuda()
    Wt = qmm.t2_pack(Wp, N, K)
    assert np.array_equal(cpu(Wt), oracle.t2_tile_pack(case.Wp.numpy(), N, K))
    back = torch.empty_like(Wp)
    qmm.qmm_t2_unpack_layout(Wt, back, N, K)
    assert torch.equal(back, Wp)


def run(case):
    d = case.to("cuda")
    Wt = qmm.t2_pack(d.Wp, case.N, case.K)
    y = torch.full((case.M, case.N), -7, dtype=torch.int32, device="cuda")
    qmm.qmm_i8t2_gemm(d.A, Wt, y, case.M, case.N, case.K)
    return cpu(y)


SHAPES = [  # M, N, K
    (1, 16, 256), (5, 48, 512), (16, 64, 1024),          # one 16-row tile, a strip per wave
    (17, 16, 256), (40, 272, 768), (128, 256, 512),      # 128-row tiles, ragged strips
    (129, 80, 256), (300, 48, 1280),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i8t2_exact(M, N, K):
    case = si.t2_case(M, N, K, seed=M * 7 + N + K)
    assert np.array_equal(run(case), oracle.i8t2_mm(case.A.numpy(), case.Wp.numpy(), M, N, K))


# 256-row tiles: one or two of them with ragged rows and strips, and at
# full height a plan of 256-column tiles followed by 192-column ones (at
# N = 4352: 16 x 16 full tiles, then 2 narrow ones, the second one past N).
LARGE = [  # M, N, K
    (65, 48, 256), (300, 272, 768), (513, 1040, 512), (4096, 4352, 256),
]


@pytest.mark.parametrize("M,N,K", LARGE)
def test_i8t2_large_exact(M, N, K):
    case = si.t2_case(M, N, K, seed=M + 3 * N + K, codes=4)
    want = oracle.i8t2_mm_mt(case.A.numpy(), case.Wp.numpy(), M, N, K)
    assert np.array_equal(run(case), want)


@pytest.mark.parametrize("M,N,K", [(3, 32, 512), (70, 64, 256)])
def test_i8t2_code_three_reads_as_two(M, N, K):
    case = si.t2_case(M, N, K, seed=M + K, codes=4)
    assert np.array_equal(run(case), oracle.i8t2_mm(case.A.numpy(), case.Wp.numpy(), M, N, K))


@pytest.mark.parametrize("M", [20, 300])
@pytest.mark.parametrize("code,want", [(2, -128), (0, 128), (3, -256)])
def test_i8t2_extremes(code, want, M):
    N, K = 32, 4096
    A = torch.full((M, K), -128, dtype=torch.int8)
    Wp = torch.full((K // 4, N), code * 0b01010101, dtype=torch.uint8)
    case = si.T2Case("extreme", M, N, K, A, Wp)
    assert np.all(run(case) == want * K)


def test_i8t2_full_size_decode_all_outputs():
    case = si.workload("i8t2_m16_k4096_n4096")
    y = run(case)
    assert np.array_equal(y, oracle.i8t2_mm(case.A.numpy(), case.Wp.numpy(), case.M, case.N,
                                            case.K))


def test_i8t2_full_size_prefill_all_outputs():
    """Every output of the full-size int8 x ternary prefill, exactly."""
    from gpu_util import full_reference_i8t2, log_parity
    name = "i8t2_m4096_k4096_n11008"
    case = si.workload(name)
    y = run(case)
    want = full_reference_i8t2(name)
    mism = int(np.count_nonzero(y != want))
    log_parity(name, entry="qmm_i8t2_gemm", outputs=int(y.size), mismatches=mism)
    assert mism == 0
