"""GPU parity of qmm_gemm (matrix-core path on the tile layout) against the
oracle: tolerance on random data, bit-exact on the exact-arithmetic and
one-hot probes, every output of the full-size workloads."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import assert_within_bound, cpu, full_reference, log_parity, sample_points

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu


NO_WORKSPACE = "none"


def run_gemm(case, ws=None):
    """qmm_gemm on the case; ws None: the cached workspace the shape calls
    for; NO_WORKSPACE: a NULL workspace (the plan that splits nothing over
    workgroups); else the given tensor."""
    d = case.to("cuda")
    Qt = qmm.pack(d.Q, case.N, case.K, case.w_bit)
    y = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    elif isinstance(ws, str):
        ws = None
    qmm.qmm_gemm(d.x, Qt, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                 case.group_size, workspace=ws)
    return cpu(y)


LOWBIT = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (1, 16, 128, 4, 128, si.F16, False),
    (5, 48, 384, 4, 128, si.BF16, False),
    (16, 256, 1024, 4, 64, si.F16, True),
    (16, 336, 2048, 4, 32, si.BF16, False),   # ragged strips per workgroup
    (17, 64, 1024, 4, 256, si.F16, False),    # two 16-row tiles, ragged
    (32, 128, 4096, 4, 128, si.BF16, False),
    (33, 96, 512, 4, 128, si.F16, True),
    (64, 64, 1024, 4, 64, si.BF16, False),
    (100, 80, 768, 4, 128, si.F16, False),    # two 64-row tiles, ragged
    (1, 32, 256, 2, 64, si.F16, False),
    (16, 64, 1024, 2, 64, si.BF16, False),
    (24, 48, 512, 2, 128, si.F16, True),
    (64, 32, 1024, 2, 32, si.BF16, False),
    (40, 16, 512, 2, 256, si.F16, False),
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", LOWBIT)
def test_gemm_lowbit_within_bound(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=3 + M * 11 + N + K + w_bit)
    y = run_gemm(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemm w{w_bit} M{M} N{N} K{K}")


INT8 = [  # M, N, K, x_dtype
    (1, 16, 64, si.BF16),       # a single 64-deep block: half a pipeline stage
    (7, 80, 192, si.F16),
    (16, 64, 4096, si.BF16),
    (33, 32, 320, si.BF16),
    (64, 112, 1024, si.F16),
    (70, 16, 128, si.BF16),
    # 16-64 rows with K % 128 == 0 take the medium kernel: ragged rows, a
    # last tile with 5 of its 8 strips, 9 stages split 5 + 4
    (50, 592, 1152, si.BF16),
    # one 16-row tile: 17 strips over tiles of 8, 10 stages split 5 + 5
    (16, 272, 1280, si.F16),
    # 33 stages over 8 splits of 5: the last split has none (its workgroup
    # adds an all-zero partial)
    (20, 64, 4224, si.F16),
]


@pytest.mark.parametrize("M,N,K,xdt", INT8)
def test_gemm_int8_within_bound(M, N, K, xdt):
    case = si.int8_case(M, N, K, xdt, seed=M * 3 + N + K)
    y = run_gemm(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemm int8 M{M} N{N} K{K}")


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", [
    (16, 64, 1024, 4, 128, si.F16, False),
    (32, 48, 2048, 4, 64, si.BF16, True),
    (64, 32, 1024, 2, 64, si.BF16, False),
    (9, 16, 4096, 4, 256, si.BF16, False),
])
def test_gemm_lowbit_exact_probe_bit_exact(M, N, K, w_bit, gs, xdt, sym):
    case = si.exact_lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=K + M + 1)
    y = run_gemm(case)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("M,N,K,xdt", [(16, 32, 1024, si.BF16), (48, 16, 2048, si.F16),
                                        # odd count of 64-deep blocks: the last 128-deep
                                        # stage is half past K and its k steps are skipped
                                        (16, 32, 192, si.BF16), (33, 48, 320, si.F16),
                                        # medium kernel: split 4 and 8 ways, and at 16 rows
                                        (64, 112, 2048, si.BF16), (20, 64, 4224, si.F16),
                                        (16, 48, 640, si.BF16)])
def test_gemm_int8_exact_probe_bit_exact(M, N, K, xdt):
    case = si.exact_int8_case(M, N, K, xdt, seed=N + 1)
    y = run_gemm(case)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("ws", [None, NO_WORKSPACE])
def test_gemm_int8_medium_unsplit(ws):
    """192 column tiles of the medium kernel fill the CUs without a K split:
    the same plan with and without a workspace."""
    M, N, K = 40, 24576, 256
    assert qmm.qmm_workspace_bytes(M, N, K, 8, 0) == 0
    case = si.int8_case(M, N, K, si.BF16, seed=123)
    y = run_gemm(case, ws=ws)
    y_ref, a_ref = oracle.qmm_mt(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, "medium unsplit")


def test_gemm_one_hot_reproduces_weights():
    M, N, K = 16, 64, 512
    base = si.lowbit_case(M, N, K, 4, 128, si.BF16, False, seed=41)
    ks = [0, 1, 2, 7, 8, 31, 32, 127, 128, 200, 255, 256, 384, 500, 510, 511]
    case = si.one_hot(base, ks)
    # power-of-two scales keep every w exact in bf16 (the matrix cores see codes only,
    # but this also pins the scale/zero epilogue bit for bit)
    y = run_gemm(case)
    W = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), N, K, 4, 128)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], W[k]), k


def test_workspace_reused_across_calls():
    """Successive calls of different shapes sharing one caller-provided
    workspace buffer: each call's result is independent of the last."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    shapes = [(16, 4096, 4096), (1, 2048, 8192), (16, 4096, 4096), (3, 1024, 4096)]
    for i, (M, N, K) in enumerate(shapes):
        case = si.lowbit_case(M, N, K, 4, 128, si.F16, False, seed=60 + i)
        assert qmm.qmm_workspace_bytes(M, N, K, 4, 128) <= ws.numel()
        y = run_gemm(case, ws=ws)
        ms, ns = sample_points(M, N, 128, seed=i)
        y_ref, a_ref = oracle.qmm_at(*case.oracle_args(), ms, ns)
        assert_within_bound(y[ms, ns], y_ref, a_ref, f"call {i}")


# ------------------------------------------ decode GEMV on the tile layout
# qmm_gemm at M <= 2 (int2: M <= 4) runs the VALU GEMV that reads each strip as
# one contiguous run: passes of 32 or 16 blocks (int4) / 16 blocks (int2)
TILE = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (1, 16, 128, 4, 128, si.F16, False),       # one block: waves 1-3 idle
    (1, 4096, 4096, 4, 128, si.F16, False),    # the headline shape
    (1, 48, 4224, 4, 64, si.BF16, False),      # 33 blocks: a second pass of one block
    (2, 64, 8192, 4, 32, si.F16, True),        # two passes, g32 (4 groups per block)
    (2, 80, 1024, 4, 256, si.BF16, False),     # 8 blocks (passes of 16), a group over two
    (2, 128, 12288, 4, 128, si.F16, False),    # three passes
    (3, 64, 2048, 2, 64, si.F16, False),       # int2, M bucket 4
    (1, 32, 2048, 2, 64, si.BF16, False),      # int2, 4 groups per block
    (2, 16, 8448, 2, 32, si.F16, False),       # int2, 33 blocks, 8 groups per block
    (4, 48, 4096, 2, 128, si.BF16, True),      # int2 at M 4 (16 blocks per pass)
    (1, 16, 512, 2, 256, si.F16, False),
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", TILE)
def test_gemm_decode_tile_within_bound(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=40 + M + N + K + w_bit)
    y = run_gemm(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"tile gemv w{w_bit} M{M} N{N} K{K} g{gs}")


@pytest.mark.parametrize("M,N,K,w_bit,gs,sym", [(1, 64, 4096, 4, 128, False),
                                                 (2, 32, 4224, 4, 32, True),
                                                 (2, 48, 8192, 2, 64, False),
                                                 (4, 16, 2048, 2, 256, False)])
@pytest.mark.parametrize("xdt", [si.F16, si.BF16])
def test_gemm_decode_tile_exact_probe_bit_exact(M, N, K, w_bit, gs, sym, xdt):
    case = si.exact_lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=M * 5 + K)
    y = run_gemm(case)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemm_decode_tile_one_hot_reproduces_weights():
    """x = e_k, one row per k (M = 4 rows per call): y reads W back exactly."""
    M, N, K = 4, 32, 512
    base = si.lowbit_case(M, N, K, 4, 64, si.F16, False, seed=43)
    W = oracle.dequant(base.np_Q(), base.np_scales(), base.np_zeros(), N, K, 4, 64)
    for ks in ([0, 1, 7, 8], [31, 32, 127, 128], [129, 255, 300, 511]):
        case = si.one_hot(base, ks)
        y = run_gemm(case)
        for m, k in enumerate(ks):
            assert np.array_equal(y[m], W[k]), k


FULL = ["int4_g128_asym_gemv_m1_k4096_n4096", "int4_pc_sym_gemv_m1_k4096_n4096",
        "int8_skinny_m16_k4096_n14336", "int8_skinny_m32_k4096_n14336",
        "int8_skinny_m64_k4096_n14336", "int4_g128_sym_m16_k8192_n8192",
        "int4_g128_asym_smalln_m16_k14336_n1024",
        "int4_g128_asym_prefill_m4096_k4096_n11008", "int2_g64_asym_prefill_m4096_k4096_n11008"]


@pytest.mark.parametrize("name", FULL)
def test_gemm_full_size_all_outputs(name):
    """Every output of the full-size workload, in the launch configuration the
    benchmark times, against the oracle's (threaded over columns)."""
    case = si.workload(name)
    y = run_gemm(case)
    y_ref, a_ref = full_reference(name)
    ratio = assert_within_bound(y, y_ref, a_ref, name)
    log_parity(name, entry="qmm_gemm", outputs=int(y.size), max_err_over_bound=ratio)


# ------------------------------------------------ large-M (prefill) kernel
LARGE = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (65, 16, 128, 4, 128, si.F16, False),      # one ragged 256-row tile, one strip
    (512, 1024, 1024, 4, 128, si.BF16, False), # 2 x 4 = 8 tiles: the XCD-aware tile order
    (512, 1024, 512, 2, 64, si.F16, False),    # the same grid for int2
    (256, 240, 1024, 4, 128, si.BF16, False),  # ragged strips in the last wave
    (300, 272, 512, 4, 64, si.F16, True),      # ragged M tile and N tile
    (512, 256, 2048, 4, 32, si.BF16, False),
    (130, 64, 1024, 4, 256, si.BF16, False),
    (257, 96, 512, 2, 64, si.BF16, False),
    (128, 48, 1024, 2, 128, si.F16, True),
    (96, 32, 768, 2, 32, si.F16, False),
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", LARGE)
def test_gemm_large_within_bound(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=7 + M + N * 3 + K + w_bit)
    y = run_gemm(case)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemm large w{w_bit} M{M} N{N} K{K}")


# The large-M plan on 256 CUs: small grids run 192-column tiles only; these
# shapes reach the 256-column kernel alone (one round of 16 x 16 tiles, where
# narrow tiles would need two) and the split of full tiles followed by narrow
# ones, with ragged rows and strips at the edges of each.
LARGE_SPLIT = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (4000, 4048, 256, 4, 128, si.BF16, False),  # full tiles only; last M tile and wave ragged
    (4096, 4096, 256, 2, 64, si.F16, False),    # full tiles only, int2
    (3900, 6320, 256, 4, 64, si.F16, True),     # 16 full + 12 narrow column tiles, the last
                                                # with 7 of its 12 strips inside N
    (4096, 6400, 256, 2, 64, si.BF16, False),   # 16 full + 12 narrow column tiles, int2
    (3900, 4416, 256, 4, 128, si.BF16, False),  # narrow tiles only (2 rounds of them beat
                                                # 2 rounds of full ones)
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", LARGE_SPLIT)
def test_gemm_large_full_and_narrow_tiles(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=11 + M + N + K + w_bit)
    y = run_gemm(case)
    y_ref, a_ref = oracle.qmm_mt(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"gemm large split w{w_bit} M{M} N{N} K{K}")


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", [
    (300, 48, 1024, 4, 128, si.BF16, False),
    (512, 1024, 1024, 4, 128, si.BF16, False),  # 8 tiles: the XCD-aware tile order
    (260, 32, 2048, 2, 64, si.F16, False),
    (128, 16, 512, 4, 32, si.BF16, True),
    (3900, 6320, 256, 4, 128, si.F16, False),   # full then narrow column tiles
    (4000, 4048, 256, 2, 64, si.BF16, False),   # full tiles only
])
def test_gemm_large_exact_probe_bit_exact(M, N, K, w_bit, gs, xdt, sym):
    """Power-of-two scales keep (q - z) * s exact in 16 bits, so the
    pre-scaled operands and every summation order are exact."""
    case = si.exact_lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=M + K)
    y = run_gemm(case)
    y_ref, _ = oracle.qmm_mt(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemm_large_one_hot_reproduces_weights():
    M, N, K = 128, 64, 512
    base = si.exact_lowbit_case(M, N, K, 4, 128, si.BF16, False, seed=42)
    ks = [(37 * m) % K for m in range(M)]
    case = si.one_hot(base, ks)
    y = run_gemm(case)
    W = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), N, K, 4, 128)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], W[k]), (m, k)


# ------------------------------------ small N, long K: K split over workgroups
# Shapes whose tiles alone leave most CUs idle (M >= 5: smaller low-bit
# batches take the decode GEMV above).  With a workspace, K is split
# over several workgroups per tile and the last to arrive adds the partials;
# with a NULL workspace the planner gives each workgroup 8 waves instead
# (>= 16 stages of K), so both plans are checked on the same shapes.
MANYWAVES = [  # M, N, K, w_bit, group, x_dtype, symmetric
    (16, 64, 4096, 4, 128, si.F16, False),      # 4 tiles, 32 stages
    (5, 256, 8192, 4, 64, si.BF16, False),      # ragged M
    (6, 32, 6144, 4, 256, si.F16, True),        # 48 stages: uneven shares
    (16, 80, 5120, 4, 32, si.BF16, False),      # 40 stages, g32
    (30, 48, 4096, 4, 128, si.F16, False),      # two 16-row tiles
    (16, 48, 8192, 2, 64, si.BF16, False),      # int2
    (9, 16, 2176, 4, 128, si.BF16, False),      # 17 stages: uneven splits, idle waves
    (64, 112, 4096, 4, 128, si.BF16, False),    # 64-row tile, 7 strips
]


@pytest.mark.parametrize("plan", ["split", "waves"])
@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", MANYWAVES)
def test_gemm_small_grid_within_bound(M, N, K, w_bit, gs, xdt, sym, plan):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=900 + M + N + K)
    if plan == "split":
        assert qmm.qmm_workspace_bytes(M, N, K, w_bit, gs) > 0
    y = run_gemm(case, ws=None if plan == "split" else NO_WORKSPACE)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"{plan} w{w_bit} M{M} N{N} K{K}")


@pytest.mark.parametrize("plan", ["split", "waves"])
@pytest.mark.parametrize("M,N,K,xdt", [(16, 64, 8192, si.BF16), (7, 32, 4096, si.F16),
                                        (40, 48, 4096, si.BF16)])
def test_gemm_small_grid_int8_within_bound(M, N, K, xdt, plan):
    case = si.int8_case(M, N, K, xdt, seed=950 + M + K)
    y = run_gemm(case, ws=None if plan == "split" else NO_WORKSPACE)
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(y, y_ref, a_ref, f"{plan} int8 M{M} N{N} K{K}")


@pytest.mark.parametrize("plan", ["split", "waves"])
@pytest.mark.parametrize("M,N,K,w_bit,gs", [(16, 64, 4096, 4, 128), (5, 32, 8192, 2, 64),
                                             (20, 16, 4096, 4, 64), (33, 32, 2048, 4, 32)])
def test_gemm_small_grid_exact_probe_bit_exact(M, N, K, w_bit, gs, plan):
    case = si.exact_lowbit_case(M, N, K, w_bit, gs, si.BF16, False, seed=M + N)
    y = run_gemm(case, ws=None if plan == "split" else NO_WORKSPACE)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_split_workspace_rearmed_over_calls():
    """One zero-filled workspace through calls of different shapes (different
    tile and split counts): each result is right, and after every call the
    tickets are back at zero.  The int8 shape at 16 x 10240 x 1024 has 80
    tiles (K split 2 ways): its tickets 64-79 lie where a layout that put the
    partial tiles right after each plan's own tickets would have left the
    partials of a call with at most 64 tiles."""
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    shapes = [(16, 64, 4096, 4, 128), (16, 1024, 14336, 4, 128), (16, 10240, 1024, 8, 0),
              (7, 32, 8192, 2, 64), (16, 10240, 1024, 8, 0), (16, 64, 4096, 4, 128),
              (40, 48, 4096, 8, 0), (5, 16, 2048, 4, 128)]
    for i, (M, N, K, wb, gs) in enumerate(shapes):
        need = qmm.qmm_workspace_bytes(M, N, K, wb, gs)
        assert 0 < need <= ws.numel(), (M, N, K, need)
        case = (si.int8_case(M, N, K, si.BF16, seed=70 + i) if wb == 8 else
                si.exact_lowbit_case(M, N, K, wb, gs, si.F16, False, seed=70 + i))
        y_ref, a_ref = oracle.qmm(*case.oracle_args())
        for rep in range(3):
            y = run_gemm(case, ws=ws)
            if wb == 8:
                assert_within_bound(y, y_ref, a_ref, f"call {i}.{rep}")
            else:
                assert np.array_equal(y.astype(np.float64), y_ref), f"call {i}.{rep}"
            # the workspace starts with 1024 tickets (4 KiB), whatever the plan
            assert int(torch.count_nonzero(ws[:4096])) == 0, f"tickets left armed after {i}"


@pytest.mark.parametrize("N", [48, 128])
def test_split_read_back_both_paths(N):
    """The last workgroup of a K-split tile reads the partials from its own
    XCD's L2 when the ticket shows every split ran there, else past the L2s.
    N=128: 8 tiles x 4 splits, 32 workgroups remapped so that a tile's splits
    share an XCD; N=48: 3 tiles x 4 splits, 12 workgroups (not a multiple of
    8, so no remap), a tile's splits on different XCDs.  Both exact against
    the oracle, twice on one workspace."""
    M, K = 16, 4096
    need = qmm.qmm_workspace_bytes(M, N, K, 4, 128)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    case = si.exact_lowbit_case(M, N, K, 4, 128, si.F16, False, seed=90 + N)
    y_ref, _ = oracle.qmm(*case.oracle_args())
    for rep in range(2):
        y = run_gemm(case, ws=ws)
        assert np.array_equal(y.astype(np.float64), y_ref), f"call {rep}"
        assert int(torch.count_nonzero(ws[:4096])) == 0


def test_split_undersized_workspace_refused():
    M, N, K = 16, 64, 4096
    need = qmm.qmm_workspace_bytes(M, N, K, 4, 128)
    assert need > 0
    case = si.lowbit_case(M, N, K, 4, 128, si.F16, False, seed=5)
    with pytest.raises(qmm.QmmError) as e:
        run_gemm(case, ws=torch.zeros(need - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == qmm.QMM_ERR_ARG
