"""HIP-graph replay of every kernel family: a call captured once and replayed
several times, with eager calls of another shape on the same workspace (or,
for the allocation-free entry point, the same scratch) between replays, must
write exactly what the eager call wrote (same kernels, same inputs: bit for
bit).  The bench times graph replays, so this is what its numbers stand on;
the K-split plans also show that their tickets are re-armed by every replay."""
import pytest
import torch

import synth_inputs as si

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu

REPLAYS = 3


def _lowbit_call(case, y, ws, noalloc=False):
    d = case.to("cuda")
    Qt = qmm.pack(d.Q, case.N, case.K, case.w_bit)

    def call():
        if noalloc:
            qmm.qmm_gemm_noalloc(d.x, Qt, d.scales, d.zeros, y, case.M, case.N, case.K,
                                 case.w_bit, case.group_size)
        else:
            qmm.qmm_gemm(d.x, Qt, d.scales, d.zeros, y, case.M, case.N, case.K, case.w_bit,
                         case.group_size, workspace=ws)
    return call


def _t2_call(case, y):
    d = case.to("cuda")
    Wt = qmm.t2_pack(d.Wp, case.N, case.K)
    return lambda: qmm.qmm_i8t2_gemm(d.A, Wt, y, case.M, case.N, case.K)


def _workspace(*cases):
    need = max(qmm.qmm_workspace_bytes(c.M, c.N, c.K, c.w_bit, c.group_size) for c in cases)
    return torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda") if need else None


def _replay_matches_eager(call, y, disturb):
    call()
    torch.cuda.synchronize()
    want = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        y.fill_(-7)
        disturb()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {r}"


# (what, main case, disturbing case): the disturbing call runs eagerly between
# replays on the same workspace; both plans are noted beside them
LOWBIT = [
    ("tile GEMV", si.lowbit_case(1, 256, 1024, 4, 128, si.F16, False, seed=501),
     si.lowbit_case(2, 128, 512, 4, 128, si.F16, False, seed=511)),
    # 16 column tiles, K split 4 ways (tickets and partial tiles in the
    # workspace); the disturbing shape splits too
    ("skinny K split", si.lowbit_case(16, 256, 4096, 4, 128, si.BF16, False, seed=502),
     si.lowbit_case(16, 128, 4096, 4, 128, si.BF16, False, seed=512)),
    # 8 column tiles of 128, K split 4 ways
    ("int8 medium K split", si.int8_case(32, 1024, 2048, si.BF16, seed=503),
     si.int8_case(32, 512, 2048, si.BF16, seed=513)),
    ("prefill", si.lowbit_case(300, 512, 512, 4, 128, si.BF16, False, seed=504),
     si.lowbit_case(260, 256, 256, 2, 64, si.F16, False, seed=514)),
]


@pytest.mark.parametrize("what,case,other", LOWBIT, ids=[c[0] for c in LOWBIT])
def test_graph_replay_equals_eager(what, case, other):
    ws = _workspace(case, other)
    if what.endswith("split"):
        assert qmm.qmm_workspace_bytes(case.M, case.N, case.K, case.w_bit, case.group_size) > 0
    y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    y2 = torch.empty((other.M, other.N), dtype=torch.float32, device="cuda")
    _replay_matches_eager(_lowbit_call(case, y, ws), y, _lowbit_call(other, y2, ws))


def test_graph_replay_noalloc_split():
    """The allocation-free entry point's static scratch: its tickets are
    cleared by a fill kernel inside the captured work, and an eager call of
    another split shape between replays leaves the scratch dirty."""
    case = si.lowbit_case(16, 256, 4096, 4, 128, si.BF16, False, seed=505)
    other = si.lowbit_case(16, 64, 8192, 4, 128, si.F16, True, seed=515)
    assert qmm.qmm_workspace_bytes(case.M, case.N, case.K, case.w_bit, case.group_size) > 0
    y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    y2 = torch.empty((other.M, other.N), dtype=torch.float32, device="cuda")
    _replay_matches_eager(_lowbit_call(case, y, None, noalloc=True), y,
                          _lowbit_call(other, y2, None, noalloc=True))


def test_graph_replay_ternary_prefill():
    case = si.t2_case(300, 512, 512, seed=506, codes=4)
    other = si.t2_case(70, 256, 768, seed=516)
    y = torch.empty((case.M, case.N), dtype=torch.int32, device="cuda")
    y2 = torch.empty((other.M, other.N), dtype=torch.int32, device="cuda")
    _replay_matches_eager(_t2_call(case, y), y, _t2_call(other, y2))
