"""Pins for the CPU oracle: each check ties it to something other than itself
(the formats' definitions via torch's own converters, constants printed on
the pages, hand-worked packing examples, exact rational arithmetic, textbook
special cases).  CPU only."""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- codecs
def _all16():
    return np.arange(65536, dtype=np.uint16)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_decode_exhaustive_matches_torch(fmt):
    bits = _all16()
    ours = oracle.f16_to_f32(bits) if fmt == "f16" else oracle.bf16_to_f32(bits)
    tdt = torch.float16 if fmt == "f16" else torch.bfloat16
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(tdt).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    # bitwise equality (keeps -0.0 and subnormals honest)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_int8_codes_exact_in_f16_and_bf16():
    q = torch.arange(-128, 128, dtype=torch.int32)
    for dt in (torch.float16, torch.bfloat16):
        assert torch.equal(q.to(dt).to(torch.int32), q)


# ------------------------------------------------ page-printed constants
def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_marlin_magic_constants_pin_symmetric_zero():
    consts = {r[0]: (int(r[1], 16), float(r[2])) for r in _read_table(
        "marlin_symmetric_int4_constants.txt")}
    for name, (bits, value) in consts.items():
        assert oracle.f16_to_f32(np.array([bits]))[0] == value, name
    dec = lambda b: float(oracle.f16_to_f32(np.array([b], np.uint16))[0])
    EX, SUB, MUL, ADD = (consts[k][0] for k in ("EX", "SUB", "MUL", "ADD"))
    one = np.array([[0x3C00]], np.uint16)  # scale 1.0
    for q in range(16):
        lo = dec(EX | q) - dec(SUB)
        hi = dec(EX | (q << 4)) * dec(MUL) + dec(ADD)
        assert lo == hi == q - 8
        # the oracle's symmetric int4 dequant (zeros = None) gives the same value
        qw = np.array([[q]], np.int32)  # code q at k = 0
        w = oracle.w_at(qw, one, None, 1, 8, 4, 8, 0, 0)
        assert w == q - 8


def test_canonical_pack_golden_words():
    for r in _read_table("canonical_pack_words.txt"):
        w_bit, word, codes = int(r[0]), int(r[1], 16), [int(c) for c in r[2:]]
        pack = 32 // w_bit
        assert len(codes) == pack
        qw = np.array([[word]], np.uint32).view(np.int32)
        got = oracle.unpack_q(qw, 1, pack, w_bit)[:, 0].tolist()
        assert got == codes


# ---------------------------------------------------------------- unpack
def _brute_code(word, field, w_bit):
    """Per-element extractor written on Python integers."""
    return (int(word) & 0xFFFFFFFF) >> (field * w_bit) & ((1 << w_bit) - 1)


@pytest.mark.parametrize("w_bit", [2, 4])
def test_unpack_matches_bitwise_brute_force(w_bit):
    pack = 32 // w_bit
    rng = np.random.default_rng(7 + w_bit)
    N, K = 5, 3 * pack
    qw = rng.integers(-2**31, 2**31, size=(K // pack, N), dtype=np.int64).astype(np.int32)
    got = oracle.unpack_q(qw, N, K, w_bit)
    for k in range(K):
        for n in range(N):
            assert got[k, n] == _brute_code(qw[k // pack, n], k % pack, w_bit)
    G = 11  # not a multiple of pack: last zero row partly used
    qz = rng.integers(-2**31, 2**31, size=(-(-G // pack), N), dtype=np.int64).astype(np.int32)
    z = oracle.unpack_z(qz, N, G, w_bit)
    for g in range(G):
        for n in range(N):
            assert z[g, n] == _brute_code(qz[g // pack, n], g % pack, w_bit)


@pytest.mark.parametrize("w_bit", [2, 4])
def test_pack_unpack_round_trip_every_value_every_slot(w_bit):
    pack = 32 // w_bit
    levels = 1 << w_bit
    # column n holds code (n + k) % levels at k: every value in every slot
    N, K = levels, 2 * pack
    codes = np.array([[(n + k) % levels for n in range(N)] for k in range(K)], np.uint32)
    words = np.zeros((K // pack, N), np.uint32)
    for k in range(K):
        words[k // pack] |= codes[k] << np.uint32((k % pack) * w_bit)
    got = oracle.unpack_q(words.view(np.int32), N, K, w_bit)
    assert np.array_equal(got, codes.astype(np.uint8))


# ------------------------------------------------- exact rational brute force
def _exact_lowbit(case):
    """y and sum |x w| in exact rationals, from codes extracted on Python ints
    and fp16/bf16 values decoded by torch."""
    M, N, K, wb, gs = case.M, case.N, case.K, case.w_bit, case.group_size
    pack = 32 // wb
    x = case.x.float().tolist()
    s = case.scales.float().tolist()
    Q = case.Q.tolist()
    Z = None if case.zeros is None else case.zeros.tolist()
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            g = 0 if gs == -1 else k // gs  # -1: per-column, one group
            q = _brute_code(Q[k // pack][n], k % pack, wb)
            z = (1 << (wb - 1)) if Z is None else _brute_code(Z[g // pack][n], g % pack, wb)
            w = (q - z) * Fraction(s[g][n])
            for m in range(M):
                p = Fraction(x[m][k]) * w
                y[m][n] += p
                a[m][n] += abs(p)
    return y, a


def _exact_int8(case):
    M, N, K = case.M, case.N, case.K
    x = case.x.float().tolist()
    Q = case.Q.tolist()
    s = case.scales.tolist()
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                p = Fraction(x[m][k]) * Q[n][k]
                acc += p
                a[m][n] += abs(p * Fraction(s[n]))
            y[m][n] = acc * Fraction(s[n])
    return y, a


def _assert_close_exact(y, ab, y_ex, a_ex, rel=1e-12):
    for m in range(len(y_ex)):
        for n in range(len(y_ex[0])):
            scale = float(a_ex[m][n]) + 1e-300
            assert abs(y[m, n] - float(y_ex[m][n])) <= rel * scale, (m, n)
            assert abs(ab[m, n] - float(a_ex[m][n])) <= rel * scale, (m, n)


LOWBIT_TINY = [
    # M, N, K, w_bit, group, x_dtype, symmetric
    (1, 3, 128, 4, 128, si.F16, False),
    (3, 5, 256, 4, 128, si.BF16, False),
    (2, 4, 128, 4, 64, si.F16, True),
    (2, 3, 128, 2, 64, si.BF16, False),
    (3, 2, 256, 2, 128, si.F16, True),
    (1, 7, 512, 4, 32, si.F16, False),   # G = 16 > pack: two zero rows
    (2, 5, 160, 4, -1, si.BF16, False),  # per-column: one scale row, zero in field 0
    (3, 4, 96, 2, -1, si.F16, True),     # per-column, symmetric
]


@pytest.mark.parametrize("M,N,K,w_bit,gs,xdt,sym", LOWBIT_TINY)
def test_oracle_matches_exact_rationals_lowbit(M, N, K, w_bit, gs, xdt, sym):
    case = si.lowbit_case(M, N, K, w_bit, gs, xdt, sym, seed=M * 100 + N * 10 + w_bit)
    y, ab = oracle.qmm(*case.oracle_args())
    _assert_close_exact(y, ab, *_exact_lowbit(case))


@pytest.mark.parametrize("w_bit,K,gs", [(4, 512, 64), (2, 512, 128), (4, 1024, 32)])
def test_per_column_equals_grouped_with_repeated_scales(w_bit, K, gs):
    """Per-column scales (Marlin's groupsize -1) are the grouped case whose
    every group carries the same scale and zero: build that grouped operand
    by repeating the single scale row and writing the zero into every field
    of every zero word, and the oracle's results must agree bit for bit."""
    pc = si.lowbit_case(3, 6, K, w_bit, -1, si.F16, False, seed=K + gs)
    G, pack = K // gs, 32 // w_bit
    scales = pc.np_scales().repeat(G, axis=0)
    z = (pc.np_zeros()[0].astype(np.int64) & ((1 << w_bit) - 1)).astype(np.uint32)
    word = np.zeros_like(z)
    for f in range(pack):
        word |= z << np.uint32(f * w_bit)
    zeros = np.tile(word.view(np.int32), ((G + pack - 1) // pack, 1))
    args = list(pc.oracle_args())
    y_pc, a_pc = oracle.qmm(*args)
    args[3], args[4], args[-1] = scales, zeros, gs
    y_g, a_g = oracle.qmm(*args)
    assert np.array_equal(y_pc, y_g) and np.array_equal(a_pc, a_g)


@pytest.mark.parametrize("M,N,K,xdt", [(1, 4, 64, si.BF16), (3, 5, 96, si.F16)])
def test_oracle_matches_exact_rationals_int8(M, N, K, xdt):
    case = si.int8_case(M, N, K, xdt, seed=M + N + K)
    y, ab = oracle.qmm(*case.oracle_args())
    _assert_close_exact(y, ab, *_exact_int8(case))


# ------------------------------------------------------ textbook reductions
def test_unit_scale_zero_zero_reduces_to_integer_matmul():
    """s = 1, z = 0: W is the code matrix; compare with a torch fp64 matmul
    of codes extracted by torch bit operations."""
    M, N, K, w_bit, gs = 3, 16, 256, 4, 128
    case = si.lowbit_case(M, N, K, w_bit, gs, si.F16, False, seed=11)
    case.scales = torch.ones_like(case.scales)
    case.zeros = torch.zeros_like(case.zeros)
    y, _ = oracle.qmm(*case.oracle_args())
    words = case.Q.to(torch.int64) & 0xFFFFFFFF
    shifts = torch.arange(8, dtype=torch.int64) * 4
    codes = ((words.unsqueeze(1) >> shifts.view(1, 8, 1)) & 15).reshape(K, N)
    ref = case.x.double() @ codes.double()
    assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-9)


def test_int8_equals_linear_times_scale():
    """tiny-llm int8_matmul docstring: same values as F.linear(x, q) * scale
    (without rounding the matmul before scaling)."""
    case = si.int8_case(4, 24, 320, si.BF16, seed=5)
    y, _ = oracle.qmm(*case.oracle_args())
    ref = torch.nn.functional.linear(case.x.double(), case.Q.double()) * case.scales.double()
    assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_exact_probe_is_exact():
    """On the exact-arithmetic probe every fp32 summation order is exact, so an
    fp32 torch matmul of the dequantized weights must equal the oracle bit
    for bit."""
    case = si.exact_lowbit_case(4, 32, 512, 4, 128, si.BF16, False, seed=3)
    y, _ = oracle.qmm(*case.oracle_args())
    W = torch.from_numpy(oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(),
                                        case.N, case.K, 4, 128))
    ref = case.x.float() @ W
    assert np.array_equal(y, ref.double().numpy())


def test_dequant_one_hot_column():
    """x = e_k picks row k of W: y[m][n] == W[k][n] exactly."""
    case = si.lowbit_case(3, 8, 256, 4, 128, si.F16, False, seed=9)
    case = si.one_hot(case, [0, 131, 255])
    y, _ = oracle.qmm(*case.oracle_args())
    W = oracle.dequant(case.np_Q(), case.np_scales(), case.np_zeros(), 8, 256, 4, 128)
    for m, k in enumerate([0, 131, 255]):
        assert np.array_equal(y[m], W[k].astype(np.float64))


def test_sampled_equals_full():
    case = si.lowbit_case(3, 32, 256, 2, 64, si.BF16, False, seed=4)
    y, ab = oracle.qmm(*case.oracle_args())
    ms = np.array([0, 2, 1, 2])
    ns = np.array([0, 31, 17, 5])
    ys, abs_ = oracle.qmm_at(*case.oracle_args(), ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(abs_, ab[ms, ns])


def test_bad_arguments_rejected():
    case = si.lowbit_case(1, 4, 128, 4, 128, si.F16, False, seed=1)
    args = list(case.oracle_args())
    args[-1] = 96  # K % group_size != 0
    with pytest.raises(ValueError):
        oracle.qmm(*args)


# ---------------------------------------------------- MFMA layout reference
@pytest.mark.parametrize("w_bit,K", [(4, 256), (2, 512), (8, 128)])
def test_mfma_layout_is_a_bijection(w_bit, K):
    N = 32
    seen = set()
    for k in range(K):
        for n in range(N):
            where, shift = oracle.mfma_locate(N, K, w_bit, k, n)
            unit = 32 if w_bit != 8 else 8
            for b in range(w_bit if w_bit != 8 else 8):
                bit = where * unit + shift + b
                assert bit not in seen
                seen.add(bit)
    assert len(seen) == oracle.mfma_bytes(N, K, w_bit) * 8


@pytest.mark.parametrize("w_bit", [2, 4, 8])
def test_mfma_pack_preserves_codes(w_bit):
    N = 32
    K = {4: 256, 2: 512, 8: 128}[w_bit]
    if w_bit == 8:
        case = si.int8_case(1, N, K, seed=2)
    else:
        case = si.lowbit_case(1, N, K, w_bit, 64, si.F16, False, seed=2)
    packed = oracle.mfma_pack(case.np_Q(), N, K, w_bit)
    Qc = case.np_Q()
    for k in range(0, K, 7):
        for n in range(N):
            where, shift = oracle.mfma_locate(N, K, w_bit, k, n)
            if w_bit == 8:
                assert packed[where] == Qc[n, k]
            else:
                code = _brute_code(packed[where], 0, 32) >> shift & ((1 << w_bit) - 1)
                assert code == _brute_code(Qc[k // (32 // w_bit), n], k % (32 // w_bit), w_bit)


# ------------------------------------------------------- planted mistakes
MUTATIONS = [
    ("(float)(q - z) * s", "(float)(z - q) * s"),                       # sign of zero point
    ("0 : k / group_size;", "0 : k / group_size + (k % 2);"),           # group index
    ("group_size == -1 ? 0 :", "group_size == -1 ? (k & 1) :"),         # per-column group
    ("(k % pack) * w_bit", "(k / pack % pack) * w_bit"),                # unpack shift
    ("return 1u << (w_bit - 1);", "return 0u;"),                         # symmetric zero
    ("acc += p;", "acc += (k + 1 < K) ? p : 0.0;"),                      # dropped term
    ("return (float)q8[(size_t)n * K + k];", "return (float)q8[(size_t)k * N + n];"),  # transposed
    ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),        # decode
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_catch_planted_mistakes():
    """Each mutation of the oracle source must make one of the exact pins fail."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.c")).read()
    lowbit = si.lowbit_case(2, 6, 256, 4, 64, si.F16, False, seed=21)
    lowsym = si.lowbit_case(2, 6, 256, 4, 64, si.F16, True, seed=22)
    int8c = si.int8_case(2, 5, 64, si.BF16, seed=23)
    lowpc = si.lowbit_case(2, 6, 256, 2, -1, si.F16, False, seed=24)
    truth = [(c, _exact_lowbit(c) if c.w_bit != 8 else _exact_int8(c))
             for c in (lowbit, lowsym, int8c, lowpc)]
    import ctypes
    with tempfile.TemporaryDirectory() as d:
        for old, new in MUTATIONS:
            assert src.count(old) >= 1, old
            cpath = os.path.join(d, "m.c")
            with open(cpath, "w") as f:
                f.write(src.replace(old, new))
            shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.h"), d)
            so = os.path.join(d, f"m{abs(hash(new))}.so")
            subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-o", so, cpath, "-lm"],
                           check=True)
            saved = oracle.lib()
            try:
                oracle._lib = _bind(ctypes.CDLL(so))
                caught = False
                for c, (y_ex, a_ex) in truth:
                    y, ab = oracle.qmm(*c.oracle_args())
                    try:
                        _assert_close_exact(y, ab, y_ex, a_ex)
                    except AssertionError:
                        caught = True
                assert caught, f"mutation not caught: {new}"
            finally:
                oracle._lib = saved


def _bind(L):
    """Give a freshly loaded oracle library the argtypes the wrapper uses."""
    ref = oracle.lib()
    for name in dir(ref):
        if name.startswith("orc_"):
            fn, r = getattr(L, name), getattr(ref, name)
            fn.argtypes, fn.restype = r.argtypes, r.restype
    return L
