"""Python binding of libqmm.so -- weight-only quantized matmul for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/qmm.h).  torch supplies device memory and
the current stream.  Functions carry the C names; a non-OK status raises
``QmmError`` (a ValueError) with the library's message.

There is no fallback: importing this package without a built libqmm.so
raises ImportError.  Build it with ``python gemv_only_quant_amd/build.py``.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

QMM_OK, QMM_ERR_ARG, QMM_ERR_UNSUPPORTED, QMM_ERR_DEVICE = 0, 1, 2, 3
QMM_F16, QMM_BF16, QMM_F32 = 0, 1, 2
QMM_PER_COLUMN = -1  # group_size for per-column scales (one group spanning K)
QMM_LAYOUT_CANON, QMM_LAYOUT_MFMA = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python gemv_only_quant_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.qmm_version.restype = _I
_lib.qmm_last_error.restype = ctypes.c_char_p
_lib.qmm_packed_bytes.argtypes = [_I, _I, _I, _I]
_lib.qmm_packed_bytes.restype = _S
_lib.qmm_pack.argtypes = [_P, _P, _I, _I, _I, _P]
_lib.qmm_unpack_layout.argtypes = [_P, _P, _I, _I, _I, _P]
_lib.qmm_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.qmm_workspace_bytes.restype = _S
_MATMUL = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _S, _P]
_MATMUL_EX = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]
_lib.qmm_gemv.argtypes = _MATMUL
_lib.qmm_gemm.argtypes = _MATMUL
_lib.qmm_gemv_ex.argtypes = _MATMUL_EX
_lib.qmm_gemm_ex.argtypes = _MATMUL_EX
_lib.qmm_dequant.argtypes = [_P, _I, _P, _P, _P, _I, _I, _I, _I, _P]
_lib.qmm_t2_pack.argtypes = [_P, _P, _I, _I, _P]
_lib.qmm_t2_unpack_layout.argtypes = [_P, _P, _I, _I, _P]
_lib.qmm_i8t2_gemm.argtypes = [_P, _P, _P, _I, _I, _I, _P]
_lib.qmm_quantize.argtypes = [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P]
for _f in ("qmm_pack", "qmm_unpack_layout", "qmm_gemv", "qmm_gemm", "qmm_gemv_ex", "qmm_gemm_ex",
           "qmm_dequant", "qmm_t2_pack", "qmm_t2_unpack_layout", "qmm_i8t2_gemm", "qmm_quantize"):
    getattr(_lib, _f).restype = _I

EXPORTS = ("qmm_version", "qmm_last_error", "qmm_packed_bytes", "qmm_pack",
           "qmm_unpack_layout", "qmm_workspace_bytes", "qmm_gemv", "qmm_gemm", "qmm_gemv_ex",
           "qmm_gemm_ex", "qmm_dequant", "qmm_t2_pack", "qmm_t2_unpack_layout", "qmm_i8t2_gemm",
           "qmm_quantize")


class QmmError(ValueError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != QMM_OK:
        raise QmmError(status, qmm_last_error())


def _dtype_code(x):
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.float16:
            return QMM_F16
        if x.dtype == torch.bfloat16:
            return QMM_BF16
        raise QmmError(QMM_ERR_ARG, f"x must be float16 or bfloat16, got {x.dtype}")
    raise QmmError(QMM_ERR_ARG, "x_dtype must be given when x is a raw pointer")


# ------------------------------------------------------------ C functions
def qmm_version():
    return _lib.qmm_version()


def qmm_last_error():
    return _lib.qmm_last_error().decode()


def qmm_packed_bytes(N, K, w_bit, layout):
    return _lib.qmm_packed_bytes(N, K, w_bit, layout)


def qmm_workspace_bytes(M, N, K, w_bit, group_size):
    return _lib.qmm_workspace_bytes(M, N, K, w_bit, group_size)


def qmm_pack(Q_canon, Q_mfma, N, K, w_bit, stream=None):
    _check(_lib.qmm_pack(_ptr(Q_canon), _ptr(Q_mfma), N, K, w_bit, _stream(stream)))


def qmm_unpack_layout(Q_mfma, Q_canon, N, K, w_bit, stream=None):
    _check(_lib.qmm_unpack_layout(_ptr(Q_mfma), _ptr(Q_canon), N, K, w_bit, _stream(stream)))


def _matmul(fn, x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype, workspace,
            workspace_bytes, stream):
    if x_dtype is None:
        x_dtype = _dtype_code(x)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(x), _ptr(Q), _ptr(scales), _ptr(zeros), _ptr(y), M, N, K, w_bit, group_size,
              x_dtype, _ptr(workspace), workspace_bytes, _stream(stream)))


def qmm_gemv(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype=None,
             workspace=None, workspace_bytes=None, stream=None):
    _matmul(_lib.qmm_gemv, x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype,
            workspace, workspace_bytes, stream)


def qmm_gemm(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype=None,
             workspace=None, workspace_bytes=None, stream=None):
    _matmul(_lib.qmm_gemm, x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype,
            workspace, workspace_bytes, stream)


def _y_code(y):
    if isinstance(y, torch.Tensor):
        codes = {torch.float32: QMM_F32, torch.float16: QMM_F16, torch.bfloat16: QMM_BF16}
        if y.dtype not in codes:
            raise QmmError(QMM_ERR_ARG, f"y must be float32, float16 or bfloat16, got {y.dtype}")
        return codes[y.dtype]
    raise QmmError(QMM_ERR_ARG, "y_dtype must be given when y is a raw pointer")


def _matmul_ex(fn, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size, x_dtype,
               workspace, workspace_bytes, stream):
    if x_dtype is None:
        x_dtype = _dtype_code(x)
    if y_dtype is None:
        y_dtype = _y_code(y)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(x), _ptr(Q), _ptr(scales), _ptr(zeros), _ptr(y), y_dtype, M, N, K, w_bit,
              group_size, x_dtype, _ptr(workspace), workspace_bytes, _stream(stream)))


def qmm_gemv_ex(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, y_dtype=None, x_dtype=None,
                workspace=None, workspace_bytes=None, stream=None):
    _matmul_ex(_lib.qmm_gemv_ex, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
               x_dtype, workspace, workspace_bytes, stream)


def qmm_gemm_ex(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, y_dtype=None, x_dtype=None,
                workspace=None, workspace_bytes=None, stream=None):
    _matmul_ex(_lib.qmm_gemm_ex, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
               x_dtype, workspace, workspace_bytes, stream)


def qmm_dequant(Q, layout, scales, zeros, w_out, N, K, w_bit, group_size, stream=None):
    _check(_lib.qmm_dequant(_ptr(Q), layout, _ptr(scales), _ptr(zeros), _ptr(w_out), N, K,
                            w_bit, group_size, _stream(stream)))


# ------------------------------------------------ tensor-level conveniences
_workspaces = {}


def workspace_for(M, N, K, w_bit, group_size, device):
    """A zero-filled workspace large enough for (M, N, K), cached per device and
    stream (the kernels leave it re-armed after every call)."""
    need = qmm_workspace_bytes(M, N, K, w_bit, group_size)
    if need == 0:
        return None
    key = (torch.device(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _dims(x, Q, w_bit, canonical):
    M, K = x.shape
    if w_bit == 8:
        N = Q.shape[0]
    elif canonical:
        N = Q.shape[1]
    else:
        raise QmmError(QMM_ERR_ARG, "pass N for weights in the MFMA layout")
    return M, N, K


def gemv(x, Q, scales, zeros, w_bit, group_size, out=None, out_dtype=torch.float32):
    """y = x @ dequant(Q) for 1 <= M <= 16, Q in the canonical layout; y is
    `out`, else a new (M, N) tensor of out_dtype (float32, float16, bfloat16)."""
    M, N, K = _dims(x, Q, w_bit, True)
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    ws = workspace_for(M, N, K, w_bit, group_size, x.device)
    qmm_gemv_ex(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, workspace=ws)
    return y


def pack(Q, N, K, w_bit):
    """Canonical weight -> new tensor in the MFMA tile layout."""
    out = torch.empty_like(Q.reshape(-1)).reshape(Q.shape) if w_bit == 8 else \
        torch.empty(Q.numel(), dtype=torch.int32, device=Q.device)
    qmm_pack(Q, out, N, K, w_bit)
    return out


def gemm(x, Q_mfma, scales, zeros, N, w_bit, group_size, out=None, out_dtype=torch.float32):
    """y = x @ dequant(Q) for any M >= 1, Q in the MFMA layout; y as in gemv."""
    M, K = x.shape
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    ws = workspace_for(M, N, K, w_bit, group_size, x.device)
    qmm_gemm_ex(x, Q_mfma, scales, zeros, y, M, N, K, w_bit, group_size, workspace=ws)
    return y


def dequant(Q, layout, scales, zeros, N, K, w_bit, group_size):
    w = torch.empty((K, N), dtype=torch.float32, device=Q.device)
    qmm_dequant(Q, layout, scales, zeros, w, N, K, w_bit, group_size)
    return w


# ---------------------------------------- int8 x ternary (liger-kernel product)
def qmm_t2_pack(W_page, W_tile, N, K, stream=None):
    _check(_lib.qmm_t2_pack(_ptr(W_page), _ptr(W_tile), N, K, _stream(stream)))


def qmm_t2_unpack_layout(W_tile, W_page, N, K, stream=None):
    _check(_lib.qmm_t2_unpack_layout(_ptr(W_tile), _ptr(W_page), N, K, _stream(stream)))


def qmm_i8t2_gemm(x, W_tile, y, M, N, K, stream=None):
    _check(_lib.qmm_i8t2_gemm(_ptr(x), _ptr(W_tile), _ptr(y), M, N, K, _stream(stream)))


def t2_pack(W_page, N, K):
    """(K/4, N) uint8 in the page's layout -> new tensor in the tile layout."""
    out = torch.empty(N * K // 4, dtype=torch.uint8, device=W_page.device)
    qmm_t2_pack(W_page, out, N, K)
    return out


def i8t2_gemm(x, W_tile, N, out=None):
    """y (M, N) int32 = x (M, K) int8 times the ternary weight (tile layout)."""
    M, K = x.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.int32, device=x.device)
    qmm_i8t2_gemm(x, W_tile, y, M, N, K)
    return y


# ------------------------------------------------ round-to-nearest quantizer
def qmm_quantize(W, w_dtype, qw, scales, qzeros, N, K, w_bit, group_size, symmetric, stream=None):
    _check(_lib.qmm_quantize(_ptr(W), w_dtype, _ptr(qw), _ptr(scales), _ptr(qzeros), N, K, w_bit,
                             group_size, int(symmetric), _stream(stream)))


def quantize(W, w_bit, group_size, symmetric=False):
    """W (K, N) float32 / float16 / bfloat16 -> (qw, scales, qzeros or None),
    the canonical operands of gemv / pack + gemm."""
    K, N = W.shape
    codes = {torch.float32: QMM_F32, torch.float16: QMM_F16, torch.bfloat16: QMM_BF16}
    if W.dtype not in codes:
        raise QmmError(QMM_ERR_ARG, f"W must be float32, float16 or bfloat16, got {W.dtype}")
    pack = 32 // w_bit
    G = 1 if group_size == QMM_PER_COLUMN else K // max(group_size, 1)
    qw = torch.empty((K // pack, N), dtype=torch.int32, device=W.device)
    sc = torch.empty((G, N), dtype=torch.float16, device=W.device)
    qz = None if symmetric else torch.empty(((G + pack - 1) // pack, N), dtype=torch.int32,
                                            device=W.device)
    qmm_quantize(W, codes[W.dtype], qw, sc, qz, N, K, w_bit, group_size, symmetric)
    return qw, sc, qz
