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
QMM_NOALLOC_SCRATCH_BYTES = 8 << 20  # scratch held per GPU for qmm_gemm_noalloc

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
_lib.qmm_gemm_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]
_lib.qmm_dequant.argtypes = [_P, _I, _P, _P, _P, _I, _I, _I, _I, _P]
_lib.qmm_t2_pack.argtypes = [_P, _P, _I, _I, _P]
_lib.qmm_t2_unpack_layout.argtypes = [_P, _P, _I, _I, _P]
_lib.qmm_i8t2_gemm.argtypes = [_P, _P, _P, _I, _I, _I, _P]
_lib.qmm_quantize.argtypes = [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P]
for _f in ("qmm_pack", "qmm_unpack_layout", "qmm_gemv", "qmm_gemm", "qmm_gemv_ex", "qmm_gemm_ex",
           "qmm_gemm_noalloc", "qmm_dequant", "qmm_t2_pack", "qmm_t2_unpack_layout", "qmm_i8t2_gemm", "qmm_quantize"):
    getattr(_lib, _f).restype = _I

EXPORTS = ("qmm_version", "qmm_last_error", "qmm_packed_bytes", "qmm_pack",
           "qmm_unpack_layout", "qmm_workspace_bytes", "qmm_gemv", "qmm_gemm", "qmm_gemv_ex",
           "qmm_gemm_ex", "qmm_gemm_noalloc", "qmm_dequant", "qmm_t2_pack", "qmm_t2_unpack_layout",
           "qmm_i8t2_gemm", "qmm_quantize")


class QmmError(ValueError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _stream(stream, device=None):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class _Args:
    """Pointer extraction with the checks the kernels rely on: each tensor is
    of an allowed dtype, contiguous and holds at least the bytes the sizes call
    for (checked as it is taken), and all of them sit on one GPU (checked by
    stream(), the last step before the call).  So a bad tensor raises QmmError
    and the library is never called.  None and raw integer pointers pass
    through unchecked."""

    def __init__(self, fn):
        self.fn = fn
        self.tensors = []

    def __call__(self, t, name, nbytes=0, dtypes=None):
        if t is None or isinstance(t, int):
            return t
        if not isinstance(t, torch.Tensor):
            raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} must be a tensor, an int or None")
        if dtypes is not None and t.dtype not in dtypes:
            want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
            raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} must be {want}, got {t.dtype}")
        if not t.is_contiguous():
            raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} must be contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} holds {have} bytes, "
                                        f"{nbytes} needed")
        self.tensors.append((name, t))
        return t.data_ptr()

    def stream(self, stream):
        """The device checks, then the stream to launch on (by default the
        current stream of the operands' device)."""
        device = None
        for name, t in self.tensors:
            if not t.is_cuda:
                raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} must be a GPU tensor "
                                            f"(got {t.device})")
            if device is None:
                device = t.device
            elif t.device != device:
                raise QmmError(QMM_ERR_ARG, f"{self.fn}: {name} is on {t.device}, other "
                                            f"operands on {device}")
        return _stream(stream, device)


_F16S = (torch.float16, torch.bfloat16)
_I8S = (torch.int8, torch.uint8)
_YS = (torch.float32, torch.float16, torch.bfloat16)


def _operand_bytes(M, N, K, w_bit, group_size):
    """Bytes of x, Q, scales and zeros for the sizes (0 where the sizes are
    themselves invalid: the library reports those)."""
    if min(M, N, K) <= 0 or w_bit not in (2, 4, 8):
        return 0, 0, 0, 0
    if w_bit == 8:
        return M * K * 2, N * K, N * 4, 0
    pack = 32 // w_bit
    if group_size == QMM_PER_COLUMN:
        G = 1
    elif group_size > 0 and K % group_size == 0:
        G = K // group_size
    else:
        G = 0
    return M * K * 2, N * K * w_bit // 8, G * N * 2, -(-G // pack) * N * 4


def _weight_dtypes(w_bit):
    return _I8S if w_bit == 8 else (torch.int32,)


def _scale_dtypes(w_bit):
    return (torch.float32,) if w_bit == 8 else (torch.float16,)


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


def _layout_call(fn, name, src, dst, N, K, w_bit, stream):
    a = _Args(name)
    nb = max(N, 0) * max(K, 0) * w_bit // 8 if w_bit in (2, 4, 8) else 0
    ps = a(src, "source", nb, _weight_dtypes(w_bit))
    pd = a(dst, "destination", nb, _weight_dtypes(w_bit))
    _check(fn(ps, pd, N, K, w_bit, a.stream(stream)))


def qmm_pack(Q_canon, Q_mfma, N, K, w_bit, stream=None):
    _layout_call(_lib.qmm_pack, "qmm_pack", Q_canon, Q_mfma, N, K, w_bit, stream)


def qmm_unpack_layout(Q_mfma, Q_canon, N, K, w_bit, stream=None):
    _layout_call(_lib.qmm_unpack_layout, "qmm_unpack_layout", Q_mfma, Q_canon, N, K, w_bit, stream)


def _matmul_ptrs(name, x, Q, scales, zeros, y, y_size, y_dtypes, M, N, K, w_bit, group_size,
                 workspace, workspace_bytes):
    a = _Args(name)
    xb, qb, sb, zb = _operand_bytes(M, N, K, w_bit, group_size)
    yb = max(M, 0) * max(N, 0) * y_size
    ptrs = (a(x, "x", xb, _F16S), a(Q, "Q", qb, _weight_dtypes(w_bit)),
            a(scales, "scales", sb, _scale_dtypes(w_bit)), a(zeros, "zeros", zb, (torch.int32,)),
            a(y, "y", yb, y_dtypes), a(workspace, "workspace", workspace_bytes))
    return a, ptrs


def _matmul(fn, name, x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype, workspace,
            workspace_bytes, stream):
    if x_dtype is None:
        x_dtype = _dtype_code(x)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a, (px, pq, ps, pz, py, pw) = _matmul_ptrs(name, x, Q, scales, zeros, y, 4,
                                               (torch.float32,), M, N, K, w_bit, group_size,
                                               workspace, workspace_bytes)
    _check(fn(px, pq, ps, pz, py, M, N, K, w_bit, group_size, x_dtype, pw, workspace_bytes,
              a.stream(stream)))


def qmm_gemv(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype=None,
             workspace=None, workspace_bytes=None, stream=None):
    _matmul(_lib.qmm_gemv, "qmm_gemv", x, Q, scales, zeros, y, M, N, K, w_bit, group_size,
            x_dtype, workspace, workspace_bytes, stream)


def qmm_gemm(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, x_dtype=None,
             workspace=None, workspace_bytes=None, stream=None):
    _matmul(_lib.qmm_gemm, "qmm_gemm", x, Q, scales, zeros, y, M, N, K, w_bit, group_size,
            x_dtype, workspace, workspace_bytes, stream)


def _y_code(y):
    if isinstance(y, torch.Tensor):
        codes = {torch.float32: QMM_F32, torch.float16: QMM_F16, torch.bfloat16: QMM_BF16}
        if y.dtype not in codes:
            raise QmmError(QMM_ERR_ARG, f"y must be float32, float16 or bfloat16, got {y.dtype}")
        return codes[y.dtype]
    raise QmmError(QMM_ERR_ARG, "y_dtype must be given when y is a raw pointer")


_Y_SIZE = {QMM_F32: 4, QMM_F16: 2, QMM_BF16: 2}


def _matmul_ex(fn, name, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size, x_dtype,
               workspace, workspace_bytes, stream):
    if x_dtype is None:
        x_dtype = _dtype_code(x)
    if y_dtype is None:
        y_dtype = _y_code(y)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    y_dtypes = ({QMM_F32: (torch.float32,), QMM_F16: (torch.float16,),
                 QMM_BF16: (torch.bfloat16,)}.get(y_dtype, _YS))
    a, (px, pq, ps, pz, py, pw) = _matmul_ptrs(name, x, Q, scales, zeros, y,
                                               _Y_SIZE.get(y_dtype, 0), y_dtypes, M, N, K,
                                               w_bit, group_size, workspace, workspace_bytes)
    _check(fn(px, pq, ps, pz, py, y_dtype, M, N, K, w_bit, group_size, x_dtype, pw,
              workspace_bytes, a.stream(stream)))


def qmm_gemv_ex(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, y_dtype=None, x_dtype=None,
                workspace=None, workspace_bytes=None, stream=None):
    _matmul_ex(_lib.qmm_gemv_ex, "qmm_gemv_ex", x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit,
               group_size, x_dtype, workspace, workspace_bytes, stream)


def qmm_gemm_ex(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, y_dtype=None, x_dtype=None,
                workspace=None, workspace_bytes=None, stream=None):
    _matmul_ex(_lib.qmm_gemm_ex, "qmm_gemm_ex", x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit,
               group_size, x_dtype, workspace, workspace_bytes, stream)


def qmm_gemm_noalloc(x, Q, scales, zeros, y, M, N, K, w_bit, group_size, y_dtype=None,
                     x_dtype=None, stream=None):
    """qmm_gemm_ex with no workspace and no allocation: the library's own
    per-GPU scratch holds what a split of K needs (calls overlapping on one
    GPU race; the stream must be on the current device)."""
    if x_dtype is None:
        x_dtype = _dtype_code(x)
    if y_dtype is None:
        y_dtype = _y_code(y)
    y_dtypes = ({QMM_F32: (torch.float32,), QMM_F16: (torch.float16,),
                 QMM_BF16: (torch.bfloat16,)}.get(y_dtype, _YS))
    a, (px, pq, ps, pz, py, _) = _matmul_ptrs("qmm_gemm_noalloc", x, Q, scales, zeros, y,
                                              _Y_SIZE.get(y_dtype, 0), y_dtypes, M, N, K, w_bit,
                                              group_size, None, 0)
    _check(_lib.qmm_gemm_noalloc(px, pq, ps, pz, py, y_dtype, M, N, K, w_bit, group_size,
                                 x_dtype, a.stream(stream)))


def qmm_dequant(Q, layout, scales, zeros, w_out, N, K, w_bit, group_size, stream=None):
    a = _Args("qmm_dequant")
    _, qb, sb, zb = _operand_bytes(1, N, K, w_bit, group_size)
    ptrs = (a(Q, "Q", qb, _weight_dtypes(w_bit)), a(scales, "scales", sb, _scale_dtypes(w_bit)),
            a(zeros, "zeros", zb, (torch.int32,)),
            a(w_out, "w_out", max(N, 0) * max(K, 0) * 4, (torch.float32,)))
    _check(_lib.qmm_dequant(ptrs[0], layout, ptrs[1], ptrs[2], ptrs[3], N, K, w_bit, group_size,
                            a.stream(stream)))


# ------------------------------------------------ tensor-level conveniences
_workspaces = {}


def workspace_for(M, N, K, w_bit, group_size, device):
    """A zero-filled workspace large enough for (M, N, K), cached per device and
    stream, or None when the shape needs none."""
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
def _t2_layout(fn, name, src, dst, N, K, stream):
    a = _Args(name)
    nb = max(N, 0) * max(K, 0) // 4
    ps, pd = a(src, "source", nb, _I8S), a(dst, "destination", nb, _I8S)
    _check(fn(ps, pd, N, K, a.stream(stream)))


def qmm_t2_pack(W_page, W_tile, N, K, stream=None):
    _t2_layout(_lib.qmm_t2_pack, "qmm_t2_pack", W_page, W_tile, N, K, stream)


def qmm_t2_unpack_layout(W_tile, W_page, N, K, stream=None):
    _t2_layout(_lib.qmm_t2_unpack_layout, "qmm_t2_unpack_layout", W_tile, W_page, N, K, stream)


def qmm_i8t2_gemm(x, W_tile, y, M, N, K, stream=None):
    a = _Args("qmm_i8t2_gemm")
    M0, N0, K0 = max(M, 0), max(N, 0), max(K, 0)
    ptrs = (a(x, "x", M0 * K0, _I8S), a(W_tile, "W_tile", N0 * K0 // 4, _I8S),
            a(y, "y", M0 * N0 * 4, (torch.int32,)))
    _check(_lib.qmm_i8t2_gemm(*ptrs, M, N, K, a.stream(stream)))


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
    a = _Args("qmm_quantize")
    wdt = {QMM_F32: (torch.float32,), QMM_F16: (torch.float16,), QMM_BF16: (torch.bfloat16,)}
    wsz = {QMM_F32: 4, QMM_F16: 2, QMM_BF16: 2}.get(w_dtype, 0)
    _, qb, sb, zb = _operand_bytes(1, N, K, w_bit, group_size) if w_bit in (2, 4) else (0,) * 4
    ptrs = (a(W, "W", max(N, 0) * max(K, 0) * wsz, wdt.get(w_dtype)),
            a(qw, "qw", qb, (torch.int32,)), a(scales, "scales", sb, (torch.float16,)),
            a(qzeros, "qzeros", 0 if symmetric else zb, (torch.int32,)))
    _check(_lib.qmm_quantize(ptrs[0], w_dtype, ptrs[1], ptrs[2], ptrs[3], N, K, w_bit,
                             group_size, int(symmetric), a.stream(stream)))


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
