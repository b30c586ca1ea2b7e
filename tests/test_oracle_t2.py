"""Pins of the oracle's int8 x ternary product (liger-kernel
ops/experimental/mm_int8int2.py): a hand-worked example, the page's pack and
unpack rules restated independently here, the integer matmul they reduce to,
special cases, the int32 range, the tile-layout reference's bijectivity, and
planted mistakes that a pin must catch."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_ternary_worked_example.txt")


def load_golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rows.setdefault(key, []).append([int(v) for v in vals])
    M, N, K = rows["M"][0][0], rows["N"][0][0], rows["K"][0][0]
    return (M, N, K, np.array(rows["A"], np.int8), np.array(rows["Wp"], np.uint8),
            np.array(rows["W"], np.int64), np.array(rows["C"], np.int64))


def page_pack(W):
    """pack_weights as the page states it: values + 1 as 2-bit codes; row_dim
    = ceil(K/4); quarter i (rows i*row_dim ..) OR-ed into bits 2i."""
    K, N = W.shape
    codes = (W + 1).astype(np.uint8)
    R = (K + 3) // 4
    packed = np.zeros((R, N), np.uint8)
    for i in range(min(4, K // R + 1)):
        start, end = i * R, min(i * R + R, K)
        if start < end:
            packed[: end - start] |= codes[start:end] << np.uint8(2 * i)
    return packed


def page_unpack(P, K):
    """unpack_weights as the page states it: quarter i = (P & (3 << 2i)) >> 2i,
    stacked, minus 1."""
    R = P.shape[0]
    out = np.zeros((4 * R,) + P.shape[1:], np.int64)
    for i in range(4):
        out[i * R:(i + 1) * R] = (P.astype(np.int64) & (3 << (2 * i))) >> (2 * i)
    return out[:K] - 1


def test_worked_example():
    M, N, K, A, Wp, W, C = load_golden()
    assert np.array_equal(page_pack(W), Wp)                       # the fixture's packing
    assert np.array_equal(oracle.i8t2_mm(A, Wp, M, N, K), C)      # the hand-computed sums
    for k in range(K):
        for n in range(N):
            assert oracle.t2_at(Wp, N, K, k, n) == W[k, n]


@pytest.mark.parametrize("K,N", [(4, 1), (16, 3), (64, 5), (256, 16)])
def test_pack_round_trip_every_position(K, N):
    rng = np.random.default_rng(K + N)
    W = rng.integers(-1, 2, (K, N))
    P = page_pack(W)
    got = np.array([[oracle.t2_at(P, N, K, k, n) for n in range(N)] for k in range(K)])
    assert np.array_equal(got, W)


@pytest.mark.parametrize("M,N,K,codes", [(1, 16, 64, 3), (3, 5, 256, 3), (7, 32, 1024, 4)])
def test_equals_integer_matmul(M, N, K, codes):
    case = si.t2_case(M, N, K, seed=M * N + K, codes=codes)
    A, P = case.A.numpy(), case.Wp.numpy()
    W = page_unpack(P, K)  # code 3 reads as +2 (the page's mask-and-subtract)
    want = A.astype(np.int64) @ W
    assert np.array_equal(oracle.i8t2_mm(A, P, M, N, K), want)
    ms = np.array([0, M - 1, M // 2], np.int32)
    ns = np.array([N - 1, 0, N // 3], np.int32)
    assert np.array_equal(oracle.i8t2_mm_at(A, P, M, N, K, ms, ns), want[ms, ns])


@pytest.mark.parametrize("code,sign", [(1, 0), (2, 1), (0, -1)])
def test_constant_codes(code, sign):
    """All codes 1: W = 0, C = 0; all 2: W = +1, C = row sums; all 0: minus them."""
    M, N, K = 3, 4, 64
    A = si.t2_case(M, N, K, seed=1).A.numpy()
    P = np.full((K // 4, N), code * 0b01010101, np.uint8)
    C = oracle.i8t2_mm(A, P, M, N, K)
    rows = A.astype(np.int64).sum(axis=1)
    assert np.array_equal(C, sign * np.repeat(rows[:, None], N, axis=1))


def test_int32_range():
    """-128 * (+1) over K = 2^20 fits int32; -128 * (+2) (code 3) over more
    than 2^23 does not and is reported."""
    A = np.full((1, 1 << 20), -128, np.int8)
    P = np.full(((1 << 20) // 4, 1), 0b10101010, np.uint8)
    assert oracle.i8t2_mm(A, P, 1, 1, 1 << 20)[0, 0] == -128 << 20
    K = (1 << 23) + 4
    A = np.full((1, K), -128, np.int8)
    P = np.full((K // 4, 1), 0xFF, np.uint8)
    with pytest.raises(ValueError, match="int32"):
        oracle.i8t2_mm(A, P, 1, 1, K)


@pytest.mark.parametrize("N,K", [(16, 256), (48, 512)])
def test_tile_layout_is_a_bijection(N, K):
    seen = set()
    for k in range(K):
        for n in range(N):
            b, sh = oracle.t2_tile_locate(N, K, k, n)
            assert sh % 2 == 0 and b < N * K // 4
            seen.add((b, sh))
    assert len(seen) == N * K
    case = si.t2_case(1, N, K, seed=N)
    T = oracle.t2_tile_pack(case.Wp.numpy(), N, K)
    k, n = K - 3, N - 2
    b, sh = oracle.t2_tile_locate(N, K, k, n)
    assert ((int(T[b]) >> sh) & 3) - 1 == oracle.t2_at(case.Wp.numpy(), N, K, k, n)


MUTATIONS = [
    ("(k % R) * N + n] >> (2 * (k / R))", "(k / R) * N + n] >> (2 * (k % R))"),  # quarter/row swapped
    ("return code - 1;", "return code;"),                                          # dropped -1
    ("A[(size_t)m * K + k] * w[k]", "A[(size_t)k * M + m] * w[k]"),              # transposed A
    ("int R = K / 4;", "int R = K / 8 + (K < 8);"),                                # wrong row count
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_catch_planted_mistakes():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.c")).read()
    M, N, K, A, Wp, W, C = load_golden()
    case = si.t2_case(3, 8, 64, seed=5)
    A2, P2 = case.A.numpy(), case.Wp.numpy()
    want2 = A2.astype(np.int64) @ page_unpack(P2, 64)
    with tempfile.TemporaryDirectory() as d:
        shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.h"), d)
        for old, new in MUTATIONS:
            assert src.count(old) >= 1, old
            cpath = os.path.join(d, "m.c")
            with open(cpath, "w") as f:
                f.write(src.replace(old, new))
            so = os.path.join(d, f"m{abs(hash(new))}.so")
            subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-o", so, cpath, "-lm"],
                           check=True)
            L = ctypes.CDLL(so)
            L.orc_i8t2_mm.argtypes = oracle.lib().orc_i8t2_mm.argtypes
            caught = False
            for (m_, n_, k_, a_, p_, want) in [(M, N, K, A, Wp, C), (3, 8, 64, A2, P2, want2)]:
                out = np.zeros((m_, n_), np.int32)
                L.orc_i8t2_mm(np.ascontiguousarray(a_).ctypes.data,
                              np.ascontiguousarray(p_).ctypes.data, m_, n_, k_, out.ctypes.data)
                caught |= not np.array_equal(out, want)
            assert caught, f"mutation not caught: {new}"
