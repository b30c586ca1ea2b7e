"""Pins of the oracle's round-to-nearest quantizer (the step before the path:
fp weights -> qw, scales, qzeros in the operand shapes of BitDistiller's
quant_matmul_kernel; the formula is this project's reading, the pages give
only the shapes): the fp16 encoder against torch's, the exact case that must
come back unchanged, the half-step reconstruction bound, the symmetric code
range, a brute force on tiny inputs, and planted mistakes."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle


def test_f16_encoder_round_trips_every_fp16_value():
    bits = np.arange(65536, dtype=np.uint16)
    finite = bits[(bits & 0x7C00) != 0x7C00]
    vals = torch.from_numpy(finite.view(np.int16)).view(torch.float16).float().numpy()
    assert np.array_equal(oracle.f32_to_f16(vals), finite)


def test_f16_encoder_matches_torch_on_ties_and_edges():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3e-5),   # subnormal range
        rng.standard_normal(20000).astype(np.float32) * np.float32(60000),  # overflow edge
        (np.arange(2048, 4096, dtype=np.float32) + np.float32(0.5)),        # exact ties
        np.array([65504, 65519.99, 65520, 2 ** -25, 2 ** -24 * 1.5, -0.0], np.float32)])
    want = torch.from_numpy(v).half().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(v), want)


def _codes(qw, K, N, w_bit):
    pack = 32 // w_bit
    k = np.arange(K)
    words = qw.view(np.uint32)[k // pack]
    return ((words >> ((k % pack) * w_bit)[:, None].astype(np.uint32)) & ((1 << w_bit) - 1)).astype(np.int64)


def _zeros(qz, G, N, w_bit):
    pack = 32 // w_bit
    g = np.arange(G)
    words = qz.view(np.uint32)[g // pack]
    return ((words >> ((g % pack) * w_bit)[:, None].astype(np.uint32)) & ((1 << w_bit) - 1)).astype(np.int64)


def _f16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()


@pytest.mark.parametrize("w_bit,gs", [(4, 128), (2, 64), (4, 32)])
def test_exact_grid_comes_back_unchanged(w_bit, gs):
    """W = (q - z) s with s an fp16 power of two, z inside the range, and each
    group's codes reaching 0 and 2^b - 1: the quantizer must return s, z and q."""
    K, N, qmax = 4 * gs, 24, (1 << w_bit) - 1
    rng = np.random.default_rng(w_bit * gs)
    G = K // gs
    s = np.float32(2.0) ** -rng.integers(4, 12, (G, N)).astype(np.float32)
    z = rng.integers(1, qmax, (G, N))
    q = rng.integers(0, qmax + 1, (K, N))
    q[0::gs] = 0
    q[1::gs] = qmax                      # every group spans the full code range
    W = ((q - np.repeat(z, gs, axis=0)) * np.repeat(s, gs, axis=0)).astype(np.float32)
    qw, sc, qz = oracle.rtn_quantize(W, N, K, w_bit, gs, False)
    assert np.array_equal(_f16(sc), s)
    assert np.array_equal(_zeros(qz, G, N, w_bit), z)
    assert np.array_equal(_codes(qw, K, N, w_bit), q)


@pytest.mark.parametrize("w_bit,gs,sym", [(4, 128, False), (4, 64, True), (2, 32, False),
                                          (4, -1, False), (2, -1, True)])
def test_reconstruction_within_half_a_step(w_bit, gs, sym):
    K, N = 512, 40
    W = (np.random.default_rng(K + N + w_bit).standard_normal((K, N)) * 0.02).astype(np.float32)
    qw, sc, qz = oracle.rtn_quantize(W, N, K, w_bit, gs, sym)
    g_of_k = np.zeros(K, np.int64) if gs == -1 else np.arange(K) // gs
    G = 1 if gs == -1 else K // gs
    s = _f16(sc)[g_of_k]
    z = (np.full((G, N), 1 << (w_bit - 1)) if sym else _zeros(qz, G, N, w_bit))[g_of_k]
    q = _codes(qw, K, N, w_bit)
    assert q.min() >= 0 and q.max() <= (1 << w_bit) - 1
    w_hat = (q - z) * s.astype(np.float64)
    inside = (q > 0) & (q < (1 << w_bit) - 1)          # not clamped
    err = np.abs(W.astype(np.float64) - w_hat)
    assert np.all(err[inside] <= 0.5 * s[inside] * (1 + 1e-6))
    # the oracle's own dequant reads the same operands back
    w_or = oracle.dequant(qw, sc, qz, N, K, w_bit, gs)
    assert np.array_equal(w_or.astype(np.float64), w_hat)
    if sym:  # max |w| maps to +-(2^(b-1) - 1): code 0 is never used
        assert q.min() >= 1


def _brute(W, N, K, w_bit, gs, sym):
    """Element by element in numpy fp32 scalars, torch for the fp16 rounding."""
    qmax = np.float32((1 << w_bit) - 1)
    G, pack = K // gs, 32 // w_bit
    q = np.zeros((K, N), np.int64)
    S = np.zeros((G, N), np.float32)
    Z = np.zeros((G, N), np.int64)
    for n in range(N):
        for g in range(G):
            col = W[g * gs:(g + 1) * gs, n]
            mn, mx = np.float32(min(col.min(), 0)), np.float32(max(col.max(), 0))
            if sym:
                s32 = np.float32(max(abs(mn), abs(mx))) / np.float32((1 << (w_bit - 1)) - 1)
            else:
                s32 = np.float32(mx - mn) / qmax
            s = np.float32(torch.tensor(float(s32), dtype=torch.float32).half().float().item())
            if s == 0:
                s = np.float32(1.0)
            z = np.float32(1 << (w_bit - 1)) if sym else np.clip(np.rint(np.float32(-mn) / s), 0, qmax)
            S[g, n], Z[g, n] = s, int(z)
            for i in range(gs):
                q[g * gs + i, n] = int(np.clip(np.rint(np.float32(col[i]) / s) + z, 0, qmax))
    return q, S, Z


@pytest.mark.parametrize("w_bit,gs,sym", [(4, 32, False), (2, 32, True), (4, 64, True)])
def test_brute_force_tiny(w_bit, gs, sym):
    K, N = 2 * gs, 3
    W = (np.random.default_rng(gs + w_bit).standard_normal((K, N)) * 0.05).astype(np.float32)
    W[5, 1] = W[0, 1]                          # repeated values
    W[:, 2] = np.float32(0.25)                 # a constant column: kept to half a step
    W[:gs, 0] = np.float32(0.0)                # an all-zero group: scale 1
    qw, sc, qz = oracle.rtn_quantize(W, N, K, w_bit, gs, sym)
    q, S, Z = _brute(W, N, K, w_bit, gs, sym)
    assert np.array_equal(_codes(qw, K, N, w_bit), q)
    assert np.array_equal(_f16(sc), S)
    if not sym:
        assert np.array_equal(_zeros(qz, K // gs, N, w_bit), Z)
    w_hat = oracle.dequant(qw, sc, qz, N, K, w_bit, gs)
    step = S[:, 2].repeat(gs)
    assert np.all(np.abs(w_hat[:, 2] - 0.25) <= 0.5 * step) and np.all(w_hat[:gs, 0] == 0)


MUTATIONS = [
    ("float q = rintf(W[(size_t)k * N + n] / s) + z;", "float q = floorf(W[(size_t)k * N + n] / s) + z;"),
    ("s32 = (mx - mn) / qmax;", "s32 = (mx - mn) / (qmax + 1.0f);"),
    ("z = rintf(-mn / s);", "z = rintf(mn / s);"),
    ("if (a == 0.0) return sign;\n", "if (a == 0.0) return sign;\n    a = a * (1.0 + 1e-3);\n"),
    ("float mn = 0.0f, mx = 0.0f;", "float mn = W[(size_t)g * gs * N + n], mx = mn;"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_catch_planted_mistakes():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.c")).read()
    K, N, gs = 64, 3, 32
    W = (np.random.default_rng(3).standard_normal((K, N)) * 0.05).astype(np.float32)
    W[:, 2] = np.abs(W[:, 2]) + np.float32(0.1)   # all positive: the range must still hold 0
    q0, S0, Z0 = _brute(W, N, K, 4, gs, False)
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
            L.orc_rtn_quantize.argtypes = oracle.lib().orc_rtn_quantize.argtypes
            qw = np.zeros((K // 8, N), np.int32)
            sc = np.zeros((K // gs, N), np.uint16)
            qz = np.zeros((1, N), np.int32)
            L.orc_rtn_quantize(W.ctypes.data, N, K, 4, gs, 0, qw.ctypes.data, sc.ctypes.data,
                               qz.ctypes.data)
            same = (np.array_equal(_codes(qw, K, N, 4), q0) and np.array_equal(_f16(sc), S0)
                    and np.array_equal(_zeros(qz, K // gs, N, 4), Z0))
            assert not same, f"mutation not caught: {new}"
