"""Seeded random shapes through the entry points, every output against the
oracle.  The plans pick a kernel, a tile shape and a K split from M, N, K, the
width and the group size (tile GEMV, skinny with or without a K split, int8
medium, large with full and narrow column tiles; the canonical-layout GEMVs;
the int8 x ternary kernels), so shapes drawn across those boundaries reach
each kernel's ragged edges in combinations the hand-picked cases do not.
Each case prints its parameters first, so a failure names it."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import assert_within_bound, cpu

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu

M_CHOICES = [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 255, 256, 257, 300]
KB = {2: 256, 4: 128, 8: 64}  # tile-layout K block of each width


def draw_gemm(seed):
    rng = np.random.default_rng(1000 + seed)
    w_bit = int(rng.choice([2, 4, 8]))
    M = int(rng.choice(M_CHOICES))
    N = 16 * int(rng.integers(1, 41))
    xdt = int(rng.choice([si.F16, si.BF16]))
    if w_bit == 8:
        K = KB[8] * int(rng.integers(1, 41))
        return si.int8_case(M, N, K, xdt, seed=seed), None
    gs = int(rng.choice([32, 64, 128, 256, -1]))
    step = max(KB[w_bit], gs)
    K = step * int(rng.integers(1, max(2, 3072 // step)))
    sym = bool(rng.random() < 0.3)
    return si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=seed), sym


def draw_gemv(seed):
    rng = np.random.default_rng(2000 + seed)
    w_bit = int(rng.choice([2, 4, 8]))
    M = int(rng.choice([m for m in M_CHOICES if m <= 16]))
    xdt = int(rng.choice([si.F16, si.BF16]))
    if w_bit == 8:
        N = int(rng.integers(1, 600))
        K = 16 * int(rng.integers(1, 200))
        return si.int8_case(M, N, K, xdt, seed=seed)
    N = 4 * int(rng.integers(1, 150))
    gs = int(rng.choice([32, 64, 128, 256, -1]))
    step = max(32, gs)
    K = step * int(rng.integers(1, max(2, 4096 // step)))
    return si.lowbit_case(M, N, K, w_bit, gs, xdt, bool(rng.random() < 0.3), seed=seed)


def _check(case, y):
    y_ref, a_ref = oracle.qmm_mt(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"{case.M}x{case.N}x{case.K} w{case.w_bit} "
                                         f"g{case.group_size}")


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("with_ws", [True, False])
def test_fuzz_gemm(seed, with_ws):
    case, _ = draw_gemm(seed)
    print(f"gemm seed {seed} ws {with_ws}: M={case.M} N={case.N} K={case.K} w{case.w_bit} "
          f"g{case.group_size} x{case.x_dtype}", flush=True)
    d = case.to("cuda")
    Qt = qmm.pack(d.Q, case.N, case.K, case.w_bit)
    y = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    need = qmm.qmm_workspace_bytes(case.M, case.N, case.K, case.w_bit, case.group_size)
    ws = torch.zeros(max(need, 4096), dtype=torch.uint8, device="cuda") if with_ws and need else None
    qmm.qmm_gemm(d.x, Qt, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                 case.group_size, workspace=ws)
    _check(case, cpu(y))
    if ws is not None:  # the split left its tickets re-armed (the workspace
        # starts with 1024 of them, whatever the plan's tile count)
        assert int(ws[:4096].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_gemv(seed):
    case = draw_gemv(seed)
    print(f"gemv seed {seed}: M={case.M} N={case.N} K={case.K} w{case.w_bit} "
          f"g{case.group_size} x{case.x_dtype}", flush=True)
    d = case.to("cuda")
    y = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    qmm.qmm_gemv(d.x, d.Q, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                 case.group_size)
    _check(case, cpu(y))


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_i8t2(seed):
    rng = np.random.default_rng(3000 + seed)
    M = int(rng.choice(M_CHOICES))
    N = 16 * int(rng.integers(1, 41))
    K = 256 * int(rng.integers(1, 12))
    print(f"i8t2 seed {seed}: M={M} N={N} K={K}", flush=True)
    case = si.t2_case(M, N, K, seed=seed, codes=4)
    d = case.to("cuda")
    Wt = qmm.t2_pack(d.Wp, N, K)
    y = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    qmm.qmm_i8t2_gemm(d.A, Wt, y, M, N, K)
    assert np.array_equal(cpu(y), oracle.i8t2_mm_mt(case.A.numpy(), case.Wp.numpy(), M, N, K))
