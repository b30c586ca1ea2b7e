"""GPU parity of the variants next to the main path: per-column scales
(group_size = QMM_PER_COLUMN, Marlin's groupsize -1) on every low-bit kernel,
and fp16 / bf16 outputs (qmm_gemv_ex / qmm_gemm_ex) on every matmul kernel.

16-bit outputs: the fp32 result (within the stated bound of the oracle) is
rounded once to nearest even, so the bound gains the output's own rounding,
|y16 - y_ref| <= bound * (1 + u) + u * |y_ref| + 2^-24 with u = 2^-11 (fp16)
or 2^-8 (bf16).  On the exact probe the fp32 result equals the oracle's, so
y16 must equal the oracle's value rounded to nearest even, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import ABS, REL, assert_within_bound, cpu

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu

PC = qmm.QMM_PER_COLUMN
TORCH_OUT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def run(case, entry, out="f32"):
    d = case.to("cuda")
    y = torch.full((case.M, case.N), float("nan"), dtype=TORCH_OUT[out], device="cuda")
    ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    if entry == "gemv":
        qmm.qmm_gemv_ex(d.x, d.Q, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                        case.group_size, workspace=ws)
    else:
        Qt = qmm.pack(d.Q, case.N, case.K, case.w_bit)
        qmm.qmm_gemm_ex(d.x, Qt, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                        case.group_size, workspace=ws)
    return cpu(y.float())


def assert_out_within_bound(y, y_ref, a_ref, out, what):
    if out == "f32":
        return assert_within_bound(y, y_ref, a_ref, what)
    u = UNIT[out]
    bound = (REL * a_ref + ABS) * (1 + u) + u * np.abs(y_ref) + 2.0 ** -24
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert np.all(err <= bound), f"{what}: max err/bound {np.max(err / bound):.3g}"


# ----------------------------------------------------------- per-column
PC_CASES = [  # entry, M, N, K, w_bit, x_dtype, symmetric
    ("gemv", 1, 64, 96, 4, si.F16, False),        # K/8 = 12 rows per column
    ("gemv", 5, 128, 4096, 4, si.BF16, True),
    ("gemv", 16, 36, 1024, 2, si.F16, False),
    ("gemm", 16, 64, 1152, 4, si.BF16, False),    # skinny, K % 256 != 0 -> runs g128
    ("gemm", 40, 32, 2048, 2, si.F16, True),      # skinny, int2
    ("gemm", 200, 48, 1024, 4, si.BF16, False),   # large-M kernel
    ("gemm", 130, 32, 768, 2, si.F16, False),     # large-M kernel, int2, K % 256 == 0
]


@pytest.mark.parametrize("entry,M,N,K,w_bit,xdt,sym", PC_CASES)
def test_per_column_within_bound(entry, M, N, K, w_bit, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, PC, xdt, sym, seed=M + N + K + w_bit)
    y = run(case, entry)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"per-column {entry} w{w_bit} M{M} N{N} K{K}")


@pytest.mark.parametrize("entry,M,N,K,w_bit", [("gemv", 3, 32, 512, 4), ("gemm", 16, 32, 1024, 4),
                                               ("gemm", 96, 16, 512, 2)])
def test_per_column_exact_probe_bit_exact(entry, M, N, K, w_bit):
    case = si.exact_lowbit_case(M, N, K, w_bit, PC, si.BF16, False, seed=M * K)
    y = run(case, entry)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("w_bit,K,sym", [(4, 1024, False), (2, 512, True)])
def test_per_column_dequant_bit_exact(layout, w_bit, K, sym):
    N = 48
    case = si.lowbit_case(1, N, K, w_bit, PC, si.F16, sym, seed=K + w_bit).to("cuda")
    Q = case.Q if layout == 0 else qmm.pack(case.Q, N, K, w_bit)
    w = cpu(qmm.dequant(Q, layout, case.scales, case.zeros, N, K, w_bit, PC))
    c = si.lowbit_case(1, N, K, w_bit, PC, si.F16, sym, seed=K + w_bit)
    ref = oracle.dequant(c.np_Q(), c.np_scales(), c.np_zeros(), N, K, w_bit, PC)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------ 16-bit outputs
OUT_CASES = [  # entry, M, N, K, w_bit, group, x_dtype
    ("gemv", 1, 256, 2048, 4, 128, si.F16),
    ("gemv", 7, 64, 1024, 2, 64, si.BF16),
    ("gemv", 3, 48, 1024, 8, 0, si.BF16),          # int8 GEMV
    ("gemm", 16, 128, 2048, 4, 128, si.BF16),      # skinny
    ("gemm", 16, 64, 1024, 8, 0, si.F16),          # skinny int8
    ("gemm", 32, 64, 1024, 8, 0, si.F16),          # medium int8, K split 2 ways
    ("gemm", 64, 80, 2048, 8, 0, si.BF16),         # medium int8, 64 rows, ragged tile
    ("gemm", 130, 80, 1024, 4, 64, si.BF16),       # large-M kernel
    ("gemm", 100, 32, 512, 2, 32, si.F16),         # large-M kernel, int2
]


def _case(M, N, K, w_bit, gs, xdt, seed):
    if w_bit == 8:
        return si.int8_case(M, N, K, xdt, seed=seed)
    return si.lowbit_case(M, N, K, w_bit, gs, xdt, False, seed=seed)


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("entry,M,N,K,w_bit,gs,xdt", OUT_CASES)
def test_16bit_output_within_bound(entry, M, N, K, w_bit, gs, xdt, out):
    case = _case(M, N, K, w_bit, gs, xdt, seed=300 + M + N + K + w_bit)
    y = run(case, entry, out)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_out_within_bound(y, y_ref, a_ref, out, f"{out} {entry} w{w_bit} M{M} N{N} K{K}")


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("entry,M,N,K,w_bit", [("gemv", 2, 64, 1024, 4), ("gemm", 16, 32, 2048, 4),
                                               ("gemm", 128, 16, 512, 2)])
def test_16bit_output_exact_probe_is_rounded_oracle(entry, M, N, K, w_bit, out):
    case = si.exact_lowbit_case(M, N, K, w_bit, 128, si.F16, False, seed=M + N + K)
    y = run(case, entry, out)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    want = torch.tensor(y_ref, dtype=torch.float32).to(TORCH_OUT[out]).float().numpy()
    assert np.array_equal(y, want)


def test_f32_through_ex_equals_plain_entry():
    case = si.lowbit_case(16, 64, 1024, 4, 128, si.BF16, False, seed=77)
    d = case.to("cuda")
    Qt = qmm.pack(d.Q, case.N, case.K, 4)
    y1 = torch.empty((16, 64), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    qmm.qmm_gemm(d.x, Qt, d.scales, d.zeros, y1, 16, 64, 1024, 4, 128)
    qmm.qmm_gemm_ex(d.x, Qt, d.scales, d.zeros, y2, 16, 64, 1024, 4, 128, y_dtype=qmm.QMM_F32)
    assert torch.equal(y1, y2)


def test_bf16_output_prefill_all_outputs():
    """The prefill workload through qmm_gemm_ex with bf16 y, in the launch
    configuration the benchmark times: every output against the oracle."""
    from gpu_util import full_reference, log_parity
    name = "int4_g128_asym_prefill_m4096_k4096_n11008"
    case = si.workload(name)
    y = run(case, "gemm", "bf16")
    y_ref, a_ref = full_reference(name)
    assert_out_within_bound(y, y_ref, a_ref, "bf16", "prefill bf16 out")
    u = UNIT["bf16"]
    bound = (REL * a_ref + ABS) * (1 + u) + u * np.abs(y_ref) + 2.0 ** -24
    log_parity(name + "_bf16_y", entry="qmm_gemm_ex", outputs=int(y.size),
               max_err_over_bound=float(np.max(np.abs(y.astype(np.float64) - y_ref) / bound)))
