"""GPU: dequant export and the tile-layout repack are bit-exact against the
oracle (integer and exact-fp32 work: no tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import cpu

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu


def _random_f16_scales(G, N, seed):
    """fp16 scales over all finite bit patterns (subnormals and negatives too)."""
    g = torch.Generator().manual_seed(seed)
    bits = torch.randint(0, 65536, (G, N), generator=g, dtype=torch.int32)
    exp = (bits >> 10) & 0x1F
    bits = torch.where(exp == 0x1F, bits & ~(1 << 14), bits)  # no inf / NaN
    return bits.to(torch.int16).view(torch.float16)


LOWBIT = [  # N, K, w_bit, group, symmetric
    (64, 256, 4, 128, False),
    (48, 512, 4, 64, True),
    (32, 512, 4, 32, False),
    (16, 1024, 4, 256, False),
    (64, 512, 2, 64, False),
    (32, 1024, 2, 128, True),
    (48, 512, 2, 32, False),
]


@pytest.mark.parametrize("N,K,w_bit,gs,sym", LOWBIT)
def test_dequant_canonical_bit_exact(N, K, w_bit, gs, sym):
    case = si.lowbit_case(1, N, K, w_bit, gs, si.F16, sym, seed=N + K + w_bit)
    case.scales = _random_f16_scales(K // gs, N, seed=K)
    d = case.to("cuda")
    w = cpu(qmm.dequant(d.Q, qmm.QMM_LAYOUT_CANON, d.scales, d.zeros, N, K, w_bit, gs))
    ref = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), N, K, w_bit, gs)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(16, 64), (48, 320)])
def test_dequant_int8_bit_exact(N, K):
    case = si.int8_case(1, N, K, seed=N)
    d = case.to("cuda")
    w = cpu(qmm.dequant(d.Q, qmm.QMM_LAYOUT_CANON, d.scales, None, N, K, 8, 0))
    ref = oracle.dequant(case.np_Q(), case.np_scales(), None, N, K, 8, 0)
    assert np.array_equal(w, ref)


PACKS = [  # N, K, w_bit
    (16, 128, 4), (48, 384, 4), (64, 1024, 4),
    (16, 256, 2), (32, 768, 2),
    (16, 64, 8), (48, 320, 8),
]


@pytest.mark.parametrize("N,K,w_bit", PACKS)
def test_pack_matches_reference_and_inverts(N, K, w_bit):
    if w_bit == 8:
        case = si.int8_case(1, N, K, seed=K)
    else:
        case = si.lowbit_case(1, N, K, w_bit, 64, si.F16, False, seed=K + w_bit)
    d = case.to("cuda")
    packed = qmm.pack(d.Q, N, K, w_bit)
    ref = oracle.mfma_pack(case.np_Q(), N, K, w_bit)
    got = cpu(packed).reshape(-1)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
    back = torch.empty_like(d.Q)
    qmm.qmm_unpack_layout(packed, back, N, K, w_bit)
    assert np.array_equal(cpu(back), case.np_Q())


@pytest.mark.parametrize("N,K,w_bit,gs,sym", [(64, 256, 4, 128, False), (32, 512, 2, 64, False),
                                              (16, 256, 4, 32, True)])
def test_dequant_tile_layout_bit_exact(N, K, w_bit, gs, sym):
    case = si.lowbit_case(1, N, K, w_bit, gs, si.BF16, sym, seed=3 * N + K)
    case.scales = _random_f16_scales(K // gs, N, seed=N)
    d = case.to("cuda")
    packed = qmm.pack(d.Q, N, K, w_bit)
    w = cpu(qmm.dequant(packed, qmm.QMM_LAYOUT_MFMA, d.scales, d.zeros, N, K, w_bit, gs))
    ref = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), N, K, w_bit, gs)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_dequant_int8_tile_layout():
    N, K = 32, 192
    case = si.int8_case(1, N, K, seed=77)
    d = case.to("cuda")
    packed = qmm.pack(d.Q, N, K, 8)
    w = cpu(qmm.dequant(packed, qmm.QMM_LAYOUT_MFMA, d.scales, None, N, K, 8, 0))
    assert np.array_equal(w, case.Q.numpy().T.astype(np.float32))


@pytest.mark.parametrize("name", ["int4_g128_prefill", "int2_g64_prefill", "int8_skinny"])
def test_pack_full_size_round_trip(name):
    """Repack at the prefill / skinny weight sizes: GPU pack equals the oracle
    permutation on sampled words, and the inverse restores every byte."""
    if name == "int4_g128_prefill":
        case = si.workload("int4_g128_asym_prefill_m4096_k4096_n11008")
    elif name == "int2_g64_prefill":
        case = si.workload("int2_g64_asym_prefill_m4096_k4096_n11008")
    else:
        case = si.workload("int8_skinny_m16_k4096_n14336")
    N, K, wb = case.N, case.K, case.w_bit
    Qd = case.Q.to("cuda")
    packed = qmm.pack(Qd, N, K, wb)
    back = torch.empty_like(Qd)
    qmm.qmm_unpack_layout(packed, back, N, K, wb)
    assert torch.equal(back, Qd)
    got = cpu(packed).reshape(-1)
    unit = 1 if wb == 8 else 4
    rng = np.random.default_rng(1)
    Qc = case.np_Q()
    for k, n in zip(rng.integers(0, K, 300), rng.integers(0, N, 300)):
        where, shift = oracle.mfma_locate(N, K, wb, int(k), int(n))
        if wb == 8:
            assert got[where] == Qc[n, k]
        else:
            code = (int(got[where]) & 0xFFFFFFFF) >> shift & ((1 << wb) - 1)
            assert code == oracle.q_at(Qc, N, wb, int(k), int(n))
    del unit
