"""Pins for the oracle's tile-layout permutations (orc_mfma_locate / pack and
orc_t2_tile_locate): positions and whole words worked by hand from the layout
text in include/qmm.h (tests/golden/tile_layout_*.txt), and planted mistakes
in the oracle source (slot parity, k-octet order, block order, column order,
the ternary interleave) that these pins must catch.  CPU only."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WBIT = {"int4": 4, "int2": 2, "int8": 8}


def _rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _locate(layout, N, K, k, n):
    if layout == "t2":
        return oracle.t2_tile_locate(N, K, k, n)
    return oracle.mfma_locate(N, K, WBIT[layout], k, n)


def _position_failures():
    bad = []
    for layout, N, K, k, n, where, shift in _rows("tile_layout_positions.txt"):
        got = _locate(layout, int(N), int(K), int(k), int(n))
        if got != (int(where), int(shift)):
            bad.append((layout, k, n, got, (int(where), int(shift))))
    return bad


def _canonical_words(codes, w_bit):
    """(K, N) codes -> canonical (K/pack, N) int32 words, packed on Python ints
    (code k at bit (k % pack) * w_bit of word k / pack)."""
    K, N = codes.shape
    pack = 32 // w_bit
    words = np.zeros((K // pack, N), np.uint32)
    for k in range(K):
        words[k // pack] |= codes[k].astype(np.uint32) << np.uint32((k % pack) * w_bit)
    return words.view(np.int32)


def _word_failures():
    bad = []
    for layout, N, K, word, value in _rows("tile_layout_words.txt"):
        N, K, word, w_bit = int(N), int(K), int(word), WBIT[layout]
        levels = 16 if w_bit == 4 else 4
        codes = np.array([[k % levels] * N for k in range(K)], np.uint32)
        tile = oracle.mfma_pack(_canonical_words(codes, w_bit), N, K, w_bit).view(np.uint32)
        if int(tile[word]) != int(value, 16):
            bad.append((layout, word, hex(int(tile[word])), value))
    return bad


def test_tile_positions_match_hand_worked():
    assert _position_failures() == []


def test_tile_words_match_hand_worked():
    assert _word_failures() == []


def test_t2_tile_pack_places_codes_at_the_worked_positions():
    """The ternary packer writes each code (page layout: row k mod K/4, bit
    pair k div K/4, value + 1) at the hand-worked position."""
    N, K = 32, 512
    R = K // 4
    rng = np.random.default_rng(4)
    vals = rng.integers(-1, 2, size=(K, N))
    Wp = np.zeros((R, N), np.uint8)
    for k in range(K):
        Wp[k % R] |= ((vals[k] + 1) << (2 * (k // R))).astype(np.uint8)
    Wt = oracle.t2_tile_pack(Wp, N, K)
    for layout, n_, k_, k, n, where, shift in _rows("tile_layout_positions.txt"):
        if layout != "t2":
            continue
        code = (int(Wt[int(where)]) >> int(shift)) & 3
        assert code == vals[int(k), int(n)] + 1, (k, n)


MUTATIONS = [
    # int4 nibble slot parity: odd codes first
    ("int slot = (i % 2 == 0) ? i / 2 : 4 + i / 2;", "int slot = (i % 2 == 1) ? i / 2 : 4 + i / 2;"),
    # int4 k-octet and word index swapped
    ("int j = r / 32, c = (r % 32) / 8, i = r % 8;", "int j = (r % 32) / 8, c = r / 32, i = r % 8;"),
    # int2 halves swapped
    ("int slot = (i % 2 == 0) ? 4 * h + i / 2 : 8 + 4 * h + i / 2;",
     "int slot = (i % 2 == 0) ? 4 * (1 - h) + i / 2 : 8 + 4 * (1 - h) + i / 2;"),
    # int8 bytes of a lane in the wrong order
    ("*where = block * 1024 + (size_t)lane * 16 + 8 * h + i;",
     "*where = block * 1024 + (size_t)lane * 16 + 8 * (1 - h) + i;"),
    # K-block-major instead of strip-major blocks
    ("size_t block = (size_t)s * (K / KB) + kb;", "size_t block = (size_t)kb * (N / 16) + s;"),
    # columns mirrored inside a strip
    ("int lane = 16 * c + col;", "int lane = 16 * c + (15 - col);"),
    # ternary codes in natural order instead of the interleave
    ("int bit = 2 * (4 * (e % 4) + e / 4);", "int bit = 2 * (4 * (e / 4) + e % 4);"),
    # ternary lane groups in the wrong order
    ("int lane = 16 * g + n % 16;", "int lane = 16 * (3 - g) + n % 16;"),
]


def _bind(L):
    ref = oracle.lib()
    for name in dir(ref):
        if name.startswith("orc_"):
            fn, r = getattr(L, name), getattr(ref, name)
            fn.argtypes, fn.restype = r.argtypes, r.restype
    return L


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_layout_pins_catch_planted_mistakes():
    """Each mutation of the oracle's layout code must fail a hand-worked pin."""
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "qmm_oracle.c")).read()
    with tempfile.TemporaryDirectory() as d:
        shutil.copy(os.path.join(here, "qmm_oracle.h"), d)
        for i, (old, new) in enumerate(MUTATIONS):
            assert src.count(old) >= 1, old
            cpath = os.path.join(d, f"m{i}.c")
            with open(cpath, "w") as f:
                f.write(src.replace(old, new))
            so = os.path.join(d, f"m{i}.so")
            subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-pthread", "-o", so,
                            cpath, "-lm"], check=True)
            saved = oracle.lib()
            try:
                oracle._lib = _bind(ctypes.CDLL(so))
                caught = bool(_position_failures()) or bool(_word_failures())
            finally:
                oracle._lib = saved
            assert caught, f"mutation not caught: {new}"
