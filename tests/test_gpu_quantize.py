"""GPU parity of the round-to-nearest quantizer (qmm_quantize) with the
oracle: codes, scales and zero points bit for bit, for every input dtype,
width, group size and degenerate group, and end to end through the GEMV."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import assert_within_bound, cpu

qmm = pytest.importorskip("gemv_only_quant_amd")
pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def weights(K, N, dtype, seed, degenerate=False):
    g = torch.Generator().manual_seed(seed)
    W = 0.02 * torch.randn((K, N), generator=g)
    if degenerate:
        W[:, 1] = 0.25                    # constant column
        W[: K // 4, 2] = 0.0              # an all-zero stretch
        W[:, 3] = W[:, 3].abs() + 0.1     # all positive
        if dtype == "f32":
            W[:, 4] = 1e6 * W[:, 4]       # fp16 scale overflows to infinity
    return W.to(DT[dtype])


def check(W, K, N, w_bit, gs, sym):
    qw, sc, qz = qmm.quantize(W.cuda(), w_bit, gs, sym)
    rq, rs, rz = oracle.rtn_quantize(W.float().numpy(), N, K, w_bit, gs, sym)
    assert np.array_equal(cpu(qw), rq)
    assert np.array_equal(cpu(sc.view(torch.int16)).view(np.uint16), rs)
    if sym:
        assert qz is None
    else:
        assert np.array_equal(cpu(qz), rz)
    return qw, sc, qz


CASES = [  # K, N, w_bit, group, symmetric, dtype
    (512, 100, 4, 128, False, "f32"),
    (640, 64, 4, 64, False, "f16"),       # G = 10: a second, partial zero-word row
    (512, 48, 2, 32, False, "bf16"),
    (1024, 36, 2, 256, True, "f16"),
    (768, 40, 4, 32, True, "bf16"),
    (4096, 20, 4, -1, False, "f32"),      # per-column
    (2048, 12, 2, -1, True, "f16"),
]


@pytest.mark.parametrize("K,N,w_bit,gs,sym,dt", CASES)
def test_quantize_bit_exact(K, N, w_bit, gs, sym, dt):
    check(weights(K, N, dt, seed=K + N + w_bit, degenerate=True), K, N, w_bit, gs, sym)


@pytest.mark.parametrize("sym", [False, True])
def test_quantize_then_gemv(sym):
    """GPU quantization feeding the GEMV: the operands equal the oracle's, and
    the product is within the bound of the oracle's product on them."""
    K, N = 2048, 256
    W = weights(K, N, "f16", seed=31)
    qw, sc, qz = check(W, K, N, 4, 128, sym)
    x = (torch.randn((3, K), generator=torch.Generator().manual_seed(32))).half()
    y = qmm.gemv(x.cuda(), qw, sc, qz, 4, 128)
    case = si.Case("rtn", 3, N, K, 4, 128, si.F16, x, qw.cpu(), sc.cpu(),
                   None if qz is None else qz.cpu())
    y_ref, a_ref = oracle.qmm(*case.oracle_args())
    assert_within_bound(cpu(y), y_ref, a_ref, "quantize -> gemv")


def test_quantize_full_size():
    K = N = 4096
    check(weights(K, N, "f16", seed=4096), K, N, 4, 128, False)


@pytest.mark.parametrize("sym,w_bit", [(False, 4), (True, 4), (False, 2)])
def test_quantize_ties_bit_exact(sym, w_bit):
    """Groups whose scale is exactly 2^-6, filled with weights at exact
    half-integer multiples of it (ties, rounded to even) and one ulp to
    either side of them: every rounding decision sits on a boundary."""
    K, N, gs = 256, 64, 32
    qmax = (1 << w_bit) - 1
    lo, hi = (-(1 << (w_bit - 1)) + 1, (1 << (w_bit - 1)) - 1) if sym else (0, qmax)
    rng = np.random.default_rng(w_bit + 2 * sym)
    step = np.float32(2.0 ** -6)
    k = rng.integers(lo, hi, (K, N)).astype(np.float32)           # ties between k and k + 1
    W = (k + np.float32(0.5)) * step
    nudge = rng.integers(-1, 2, (K, N))                              # -1, 0, +1 ulp
    W = np.where(nudge < 0, np.nextafter(W, np.float32(-1)),
                 np.where(nudge > 0, np.nextafter(W, np.float32(1)), W)).astype(np.float32)
    W[0::gs] = lo * step                                             # range fixes s = 2^-6
    W[1::gs] = hi * step
    check(torch.from_numpy(W), K, N, w_bit, gs, sym)
    _, sc, _ = oracle.rtn_quantize(W, N, K, w_bit, gs, sym)
    assert np.all(sc == 0x2400)                                      # 2^-6 in fp16
