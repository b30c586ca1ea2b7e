"""ctypes front end of the CPU oracle (oracle/qmm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg.  The product path never imports it.

Arrays are numpy; 16-bit floats travel as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32_n.argtypes = [P, P, S]
        L.orc_bf16_to_f32_n.argtypes = [P, P, S]
        L.orc_q_at.argtypes = [P, I, I, I, I]
        L.orc_q_at.restype = ctypes.c_uint32
        L.orc_z_at.argtypes = [P, I, I, I, I]
        L.orc_z_at.restype = ctypes.c_uint32
        L.orc_w_at.argtypes = [P, P, P, I, I, I, I, I, I]
        L.orc_w_at.restype = ctypes.c_float
        L.orc_unpack_q.argtypes = [P, I, I, I, P]
        L.orc_unpack_z.argtypes = [P, I, I, I, P]
        L.orc_dequant.argtypes = [P, P, P, I, I, I, I, P]
        L.orc_qmm.argtypes = [P, I, P, P, P, I, I, I, I, I, P, P]
        L.orc_qmm_at.argtypes = [P, I, P, P, P, I, I, I, I, I, I, P, P, P, P]
        L.orc_qmm_mt.argtypes = [P, I, P, P, P, I, I, I, I, I, P, P, I]
        L.orc_i8t2_mm_mt.argtypes = [P, P, I, I, I, P, I]
        L.orc_mfma_locate.argtypes = [I, I, I, I, I, ctypes.POINTER(S), ctypes.POINTER(I)]
        L.orc_mfma_bytes.argtypes = [I, I, I]
        L.orc_mfma_bytes.restype = S
        L.orc_mfma_pack.argtypes = [P, P, I, I, I]
        L.orc_t2_at.argtypes = [P, I, I, I, I]
        L.orc_i8t2_mm.argtypes = [P, P, I, I, I, P]
        L.orc_i8t2_mm_at.argtypes = [P, P, I, I, I, I, P, P, P]
        L.orc_t2_tile_bytes.argtypes = [I, I]
        L.orc_t2_tile_bytes.restype = S
        L.orc_t2_tile_locate.argtypes = [I, I, I, I, ctypes.POINTER(S), ctypes.POINTER(I)]
        L.orc_t2_tile_pack.argtypes = [P, P, I, I]
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_rtn_quantize.argtypes = [P, I, I, I, I, I, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments")


def f16_to_f32(bits):
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_f16_to_f32_n(_ptr(b), _ptr(out), b.size)
    return out


def bf16_to_f32(bits):
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_f32_n(_ptr(b), _ptr(out), b.size)
    return out


def q_at(qw, N, w_bit, k, n):
    qw = _c(qw, np.int32)
    return int(lib().orc_q_at(_ptr(qw), N, w_bit, k, n))


def unpack_q(qw, N, K, w_bit):
    qw = _c(qw, np.int32)
    out = np.empty((K, N), np.uint8)
    _check(lib().orc_unpack_q(_ptr(qw), N, K, w_bit, _ptr(out)), "unpack_q")
    return out


def unpack_z(qz, N, G, w_bit):
    qz = _c(qz, np.int32)
    out = np.empty((G, N), np.uint8)
    _check(lib().orc_unpack_z(_ptr(qz), N, G, w_bit, _ptr(out)), "unpack_z")
    return out


def _operands(Q, scales, zeros, w_bit):
    if w_bit == 8:
        return _c(Q, np.int8), _c(scales, np.float32), None
    return _c(Q, np.int32), _c(scales, np.uint16), _c(zeros, np.int32)


def w_at(Q, scales, zeros, N, K, w_bit, group_size, k, n):
    Q, scales, zeros = _operands(Q, scales, zeros, w_bit)
    return float(lib().orc_w_at(_ptr(Q), _ptr(scales), _ptr(zeros), N, K, w_bit,
                                group_size, k, n))


def dequant(Q, scales, zeros, N, K, w_bit, group_size):
    """W (K, N) fp32; int8 returns the raw code (row scale not applied)."""
    Q, scales, zeros = _operands(Q, scales, zeros, w_bit)
    out = np.empty((K, N), np.float32)
    _check(lib().orc_dequant(_ptr(Q), _ptr(scales), _ptr(zeros), N, K, w_bit,
                             group_size, _ptr(out)), "dequant")
    return out


def qmm(x_bits, x_dtype, Q, scales, zeros, M, N, K, w_bit, group_size):
    """(y_ref, abs_ref), each (M, N) float64.  x_dtype: 0 fp16, 1 bf16."""
    x = _c(x_bits, np.uint16)
    Q, scales, zeros = _operands(Q, scales, zeros, w_bit)
    y = np.empty((M, N), np.float64)
    ab = np.empty((M, N), np.float64)
    _check(lib().orc_qmm(_ptr(x), x_dtype, _ptr(Q), _ptr(scales), _ptr(zeros),
                         M, N, K, w_bit, group_size, _ptr(y), _ptr(ab)), "qmm")
    return y, ab


def host_threads():
    """Host threads for the threaded calls: the CPUs this process may run on,
    at most 16 (a GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def qmm_mt(x_bits, x_dtype, Q, scales, zeros, M, N, K, w_bit, group_size, threads=None):
    """qmm() with the columns divided over host threads: bit-identical results."""
    x = _c(x_bits, np.uint16)
    Q, scales, zeros = _operands(Q, scales, zeros, w_bit)
    y = np.empty((M, N), np.float64)
    ab = np.empty((M, N), np.float64)
    _check(lib().orc_qmm_mt(_ptr(x), x_dtype, _ptr(Q), _ptr(scales), _ptr(zeros),
                            M, N, K, w_bit, group_size, _ptr(y), _ptr(ab),
                            threads or host_threads()), "qmm_mt")
    return y, ab


def qmm_at(x_bits, x_dtype, Q, scales, zeros, M, N, K, w_bit, group_size, ms, ns):
    """(y_ref, abs_ref) at the outputs (ms[i], ns[i]) only."""
    x = _c(x_bits, np.uint16)
    Q, scales, zeros = _operands(Q, scales, zeros, w_bit)
    ms = _c(ms, np.int32)
    ns = _c(ns, np.int32)
    y = np.empty(ms.shape, np.float64)
    ab = np.empty(ms.shape, np.float64)
    _check(lib().orc_qmm_at(_ptr(x), x_dtype, _ptr(Q), _ptr(scales), _ptr(zeros),
                            M, N, K, w_bit, group_size, ms.size, _ptr(ms), _ptr(ns),
                            _ptr(y), _ptr(ab)), "qmm_at")
    return y, ab


def mfma_locate(N, K, w_bit, k, n):
    where = ctypes.c_size_t()
    shift = ctypes.c_int()
    _check(lib().orc_mfma_locate(N, K, w_bit, k, n, ctypes.byref(where),
                                 ctypes.byref(shift)), "mfma_locate")
    return where.value, shift.value


def mfma_bytes(N, K, w_bit):
    return int(lib().orc_mfma_bytes(N, K, w_bit))


def mfma_pack(Q, N, K, w_bit):
    """Canonical weight -> MFMA tile layout (int32 words, or int8 bytes)."""
    nbytes = mfma_bytes(N, K, w_bit)
    if w_bit == 8:
        Q = _c(Q, np.int8)
        out = np.empty(nbytes, np.int8)
    else:
        Q = _c(Q, np.int32)
        out = np.empty(nbytes // 4, np.int32)
    _check(lib().orc_mfma_pack(_ptr(Q), _ptr(out), N, K, w_bit), "mfma_pack")
    return out


# ------------------------------------------- int8 x ternary (liger-kernel page)
def t2_at(Wp, N, K, k, n):
    """Ternary weight value (code - 1) of element (k, n) of the packed (K/4, N) uint8."""
    Wp = _c(Wp, np.uint8)
    return lib().orc_t2_at(_ptr(Wp), N, K, k, n)


def i8t2_mm(A, Wp, M, N, K):
    """C (M, N) int32 = A (M, K) int8 times the ternary weight, exact."""
    A, Wp = _c(A, np.int8), _c(Wp, np.uint8)
    C = np.zeros((M, N), np.int32)
    rc = lib().orc_i8t2_mm(_ptr(A), _ptr(Wp), M, N, K, _ptr(C))
    if rc == -2:
        raise ValueError("oracle i8t2_mm: a sum leaves the int32 range")
    _check(rc, "i8t2_mm")
    return C


def i8t2_mm_mt(A, Wp, M, N, K, threads=None):
    """i8t2_mm() with the columns divided over host threads (exact either way)."""
    A, Wp = _c(A, np.int8), _c(Wp, np.uint8)
    C = np.zeros((M, N), np.int32)
    rc = lib().orc_i8t2_mm_mt(_ptr(A), _ptr(Wp), M, N, K, _ptr(C), threads or host_threads())
    if rc == -2:
        raise ValueError("oracle i8t2_mm_mt: a sum leaves the int32 range")
    _check(rc, "i8t2_mm_mt")
    return C


def i8t2_mm_at(A, Wp, M, N, K, ms, ns):
    A, Wp = _c(A, np.int8), _c(Wp, np.uint8)
    ms, ns = _c(ms, np.int32), _c(ns, np.int32)
    C = np.zeros(ms.size, np.int32)
    _check(lib().orc_i8t2_mm_at(_ptr(A), _ptr(Wp), M, N, K, ms.size, _ptr(ms), _ptr(ns),
                                _ptr(C)), "i8t2_mm_at")
    return C


def t2_tile_locate(N, K, k, n):
    b, sh = ctypes.c_size_t(), ctypes.c_int()
    _check(lib().orc_t2_tile_locate(N, K, k, n, ctypes.byref(b), ctypes.byref(sh)),
           "t2_tile_locate")
    return b.value, sh.value


def t2_tile_pack(Wp, N, K):
    Wp = _c(Wp, np.uint8)
    out = np.zeros(lib().orc_t2_tile_bytes(N, K), np.uint8)
    _check(lib().orc_t2_tile_pack(_ptr(Wp), _ptr(out), N, K), "t2_tile_pack")
    return out


# --------------------------------------------- round-to-nearest quantizer
def f32_to_f16(values):
    """fp16 bit patterns of fp32 values, round to nearest even."""
    L = lib()
    v = np.asarray(values, np.float32).ravel()
    return np.array([L.orc_f32_to_f16(float(a)) for a in v], np.uint16)


def rtn_quantize(W, N, K, w_bit, group_size, symmetric):
    """W (K, N) fp32 -> (qw (K/pack, N) int32, scales (G, N) fp16 bits,
    qzeros (ceil(G/pack), N) int32 or None)."""
    W = _c(W, np.float32)
    pack = 32 // w_bit
    G = 1 if group_size == -1 else K // group_size
    qw = np.zeros((K // pack, N), np.int32)
    sc = np.zeros((G, N), np.uint16)
    qz = None if symmetric else np.zeros(((G + pack - 1) // pack, N), np.int32)
    _check(lib().orc_rtn_quantize(_ptr(W), N, K, w_bit, group_size, int(symmetric), _ptr(qw),
                                  _ptr(sc), _ptr(qz)), "rtn_quantize")
    return qw, sc, qz
