"""The C-ABI library loads, exports every entry point include/qmm.h declares,
and rejects bad arguments before any HIP call.  CPU only: every call below
fails validation, so nothing is launched (fake pointers never reach a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

qmm = pytest.importorskip("gemv_only_quant_amd")

A = 0x10000  # a 16-byte aligned fake address: only ever used in calls that must fail
MIS = 0x10004  # misaligned fake address


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"QMM_API\s+[\w\s\*]+?\b(qmm_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared()
    assert len(names) == 16, names
    lib = ctypes.CDLL(qmm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(qmm.EXPORTS)


def test_version_and_sizes():
    assert qmm.qmm_version() >= 1
    assert qmm.qmm_packed_bytes(4096, 4096, 4, qmm.QMM_LAYOUT_CANON) == 4096 * 4096 // 2
    assert qmm.qmm_packed_bytes(11008, 4096, 2, qmm.QMM_LAYOUT_MFMA) == 11008 * 4096 // 4
    assert qmm.qmm_packed_bytes(100, 4096, 4, qmm.QMM_LAYOUT_MFMA) == 0   # N % 16
    assert qmm.qmm_packed_bytes(64, 100, 4, qmm.QMM_LAYOUT_CANON) == 0    # K % 8
    assert qmm.qmm_packed_bytes(64, 64, 3, qmm.QMM_LAYOUT_CANON) == 0
    assert qmm.qmm_workspace_bytes(0, 64, 64, 8, 0) == 0
    assert qmm.qmm_workspace_bytes(1, 64, 100, 4, 128) == 0  # invalid: K % group
    assert qmm.qmm_workspace_bytes(16, 4096, 4096, 4, qmm.QMM_PER_COLUMN) == 0
    assert qmm.qmm_workspace_bytes(1, 64, 40, 4, qmm.QMM_PER_COLUMN) == 0  # K % 32
    # grids with enough column tiles, and the prefill kernel, keep every
    # partial sum inside a workgroup: no workspace
    for M, N, K, wb, g in [(16, 8192, 8192, 4, 128), (4096, 11008, 4096, 2, 64),
                           (4096, 64, 4096, 4, 128)]:
        assert qmm.qmm_workspace_bytes(M, N, K, wb, g) == 0
    # few column tiles over a long K: K split over workgroups, tickets + partials
    M, N, K = 16, 1024, 14336
    need = qmm.qmm_workspace_bytes(M, N, K, 4, 128)
    tiles = N // 16
    assert need > tiles * 16 * 16 * 4 and need % 16 == 0


def call_gemv(**kw):
    args = dict(x=A, Q=A, scales=A, zeros=None, y=A, M=1, N=64, K=128, w_bit=4,
                group_size=128, x_dtype=qmm.QMM_F16, workspace=None, workspace_bytes=0,
                stream=0)
    args.update(kw)
    return qmm._lib.qmm_gemv(args["x"], args["Q"], args["scales"], args["zeros"], args["y"],
                             args["M"], args["N"], args["K"], args["w_bit"],
                             args["group_size"], args["x_dtype"], args["workspace"],
                             args["workspace_bytes"], args["stream"])


def call_gemm(**kw):
    args = dict(x=A, Q=A, scales=A, zeros=None, y=A, M=1, N=64, K=128, w_bit=4,
                group_size=128, x_dtype=qmm.QMM_F16, workspace=None, workspace_bytes=0,
                stream=0)
    args.update(kw)
    return qmm._lib.qmm_gemm(args["x"], args["Q"], args["scales"], args["zeros"], args["y"],
                             args["M"], args["N"], args["K"], args["w_bit"],
                             args["group_size"], args["x_dtype"], args["workspace"],
                             args["workspace_bytes"], args["stream"])


E_ARG, E_UNS = qmm.QMM_ERR_ARG, qmm.QMM_ERR_UNSUPPORTED

GEMV_BAD = [
    (dict(M=-1), E_ARG, "negative"),
    (dict(N=-5), E_ARG, "negative"),
    (dict(w_bit=3), E_ARG, "w_bit"),
    (dict(x_dtype=7), E_ARG, "x_dtype"),
    (dict(group_size=0), E_ARG, "group_size"),
    (dict(group_size=-2), E_ARG, "QMM_PER_COLUMN"),
    (dict(group_size=-1, K=100), E_ARG, "multiple of 8"),
    (dict(group_size=-1, K=40), E_UNS, "per-column"),
    (dict(w_bit=8, group_size=-1), E_ARG, "per-row"),
    (dict(K=192), E_ARG, "multiple of group_size"),
    (dict(group_size=96, K=192), E_UNS, "not built"),
    (dict(w_bit=8, group_size=128), E_ARG, "per-row"),
    (dict(w_bit=8, group_size=0, zeros=A), E_ARG, "zero points"),
    (dict(x=None), E_ARG, "NULL"),
    (dict(Q=None), E_ARG, "NULL"),
    (dict(scales=None), E_ARG, "NULL"),
    (dict(y=None), E_ARG, "NULL"),
    (dict(x=MIS), E_ARG, "aligned"),
    (dict(Q=MIS), E_ARG, "aligned"),
    (dict(zeros=MIS), E_ARG, "aligned"),
    (dict(M=17), E_UNS, "M=17"),
    (dict(N=66), E_UNS, "N % 4"),
    (dict(w_bit=8, group_size=0, K=24), E_UNS, "K % 16"),
]


@pytest.mark.parametrize("kw,status,msg", GEMV_BAD)
def test_gemv_rejects(kw, status, msg):
    assert call_gemv(**kw) == status
    assert msg in qmm.qmm_last_error()


GEMM_BAD = [
    (dict(N=72), E_UNS, "N % 16"),
    (dict(K=64), E_ARG, "multiple of group_size"),
    (dict(K=192, group_size=64), E_UNS, "K % 128"),
    (dict(w_bit=2, K=128, group_size=64), E_UNS, "K % 256"),
    (dict(w_bit=8, group_size=0, K=96), E_UNS, "K % 64"),
    (dict(y=MIS), E_ARG, "aligned"),
    # skinny kernel: 32-bit byte offsets into the scale table (2^14 groups x 2^16 columns)
    (dict(M=16, N=65536, K=524288, group_size=32), E_UNS, "too large"),
    # skinny kernel: 32-bit byte offsets into x (64 rows of K)
    (dict(M=16, N=64, K=1 << 24, group_size=128), E_UNS, "K=16777216 too large"),
    # large-M kernel: 32-bit byte offsets into a workgroup's x rows (256 rows of K)
    (dict(M=128, N=64, K=1 << 22, group_size=128), E_UNS, "K=4194304 too large for M > 64"),
    # ... and into the scale table
    (dict(M=128, N=65536, K=524288, group_size=32), E_UNS, "scale table"),
]


@pytest.mark.parametrize("kw,status,msg", GEMM_BAD)
def test_gemm_rejects(kw, status, msg):
    assert call_gemm(**kw) == status
    assert msg in qmm.qmm_last_error()


@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(K=0), dict(M=0, x=None, y=None)])
def test_zero_size_is_noop(kw):
    # zero sizes return OK before touching pointers or the device
    assert call_gemv(**kw) == qmm.QMM_OK
    assert call_gemm(**kw) == qmm.QMM_OK
    assert qmm.qmm_last_error() == ""


def call_ex(fn, y_dtype, **kw):
    args = dict(x=A, Q=A, scales=A, zeros=None, y=A, M=1, N=64, K=128, w_bit=4,
                group_size=128, x_dtype=qmm.QMM_F16)
    args.update(kw)
    return fn(args["x"], args["Q"], args["scales"], args["zeros"], args["y"], y_dtype,
              args["M"], args["N"], args["K"], args["w_bit"], args["group_size"],
              args["x_dtype"], None, 0, 0)


@pytest.mark.parametrize("name", ["qmm_gemv_ex", "qmm_gemm_ex"])
def test_ex_entry_points_reject(name):
    fn = getattr(qmm._lib, name)
    assert call_ex(fn, 3) == E_ARG and "y_dtype" in qmm.qmm_last_error()
    assert call_ex(fn, -1) == E_ARG and name in qmm.qmm_last_error()
    assert call_ex(fn, qmm.QMM_F16, x_dtype=qmm.QMM_F32) == E_ARG
    assert "x_dtype" in qmm.qmm_last_error()
    assert call_ex(fn, qmm.QMM_BF16, y=MIS) == E_ARG and "aligned" in qmm.qmm_last_error()
    assert call_ex(fn, qmm.QMM_F16, M=0, x=None, y=None) == qmm.QMM_OK  # no-op
    assert call_ex(fn, qmm.QMM_F16, group_size=-1, K=40) == E_UNS


def test_ternary_calls_reject():
    L = qmm._lib
    assert L.qmm_t2_pack(A, A + 64, 64, 256, 0) == E_ARG and "overlap" in qmm.qmm_last_error()
    assert L.qmm_t2_pack(A, None, 64, 256, 0) == E_ARG
    assert L.qmm_t2_pack(A, 0x100000, 24, 256, 0) == E_UNS and "N % 16" in qmm.qmm_last_error()
    assert L.qmm_t2_unpack_layout(A, 0x100000, 64, 128, 0) == E_UNS          # K % 256
    assert L.qmm_t2_pack(A, A, 0, 256, 0) == qmm.QMM_OK                      # empty
    assert L.qmm_t2_pack(MIS, 0x100000, 64, 256, 0) == E_ARG
    assert L.qmm_i8t2_gemm(A, A, A, -1, 64, 256, 0) == E_ARG
    assert L.qmm_i8t2_gemm(A, A, None, 4, 64, 256, 0) == E_ARG
    assert L.qmm_i8t2_gemm(A, A, MIS, 4, 64, 256, 0) == E_ARG
    assert L.qmm_i8t2_gemm(A, A, A, 4, 64, 320, 0) == E_UNS
    assert L.qmm_i8t2_gemm(A, A, A, 65, 64, 1 << 23, 0) == E_UNS and "M > 64" in qmm.qmm_last_error()
    assert L.qmm_i8t2_gemm(None, None, None, 0, 64, 256, 0) == qmm.QMM_OK   # M = 0


def test_quantize_rejects():
    L = qmm._lib
    assert L.qmm_quantize(A, 9, A, A, A, 64, 128, 4, 128, 0, 0) == E_ARG
    assert "w_dtype" in qmm.qmm_last_error()
    assert L.qmm_quantize(A, qmm.QMM_F32, A, A, A, 64, 128, 8, 0, 0, 0) == E_ARG
    assert L.qmm_quantize(A, qmm.QMM_F32, A, A, A, 64, 128, 4, 128, 1, 0) == E_ARG
    assert "NULL" in qmm.qmm_last_error()
    assert L.qmm_quantize(A, qmm.QMM_F32, A, A, None, 64, 128, 4, 128, 0, 0) == E_ARG
    assert L.qmm_quantize(A, qmm.QMM_F32, A, A, A, 64, 192, 4, 128, 0, 0) == E_ARG  # K % g
    assert L.qmm_quantize(A, qmm.QMM_F32, A, A, A, 64, 40, 4, -1, 0, 0) == E_UNS    # K % 32
    assert L.qmm_quantize(None, qmm.QMM_F32, A, A, A, 64, 128, 4, 128, 0, 0) == E_ARG
    assert L.qmm_quantize(A, qmm.QMM_F16, A, A, None, 0, 128, 4, 128, 1, 0) == qmm.QMM_OK


def test_layout_calls_reject():
    L = qmm._lib
    assert L.qmm_pack(A, A + 64, 64, 128, 4, 0) == E_ARG            # overlap
    assert "overlap" in qmm.qmm_last_error()
    assert L.qmm_pack(A, None, 64, 128, 4, 0) == E_ARG
    assert L.qmm_pack(A, 0x100000, 24, 128, 4, 0) == E_UNS           # N % 16
    assert L.qmm_pack(A, 0x100000, 64, 128, 5, 0) == E_ARG
    assert L.qmm_unpack_layout(A, 0x100000, 64, 100, 8, 0) == E_UNS  # K % 64
    assert L.qmm_pack(A, A, 0, 128, 4, 0) == qmm.QMM_OK              # empty
    assert L.qmm_dequant(A, 9, A, None, A, 64, 128, 4, 128, 0) == E_ARG
    assert L.qmm_dequant(A, 1, A, None, A, 24, 128, 4, 128, 0) == E_UNS
    assert L.qmm_dequant(A, 0, A, None, None, 64, 128, 4, 128, 0) == E_ARG


def test_python_wrapper_raises_valueerror():
    with pytest.raises(ValueError) as ei:
        qmm.qmm_gemv(A, A, A, None, A, 17, 64, 128, 4, 128, x_dtype=0, stream=0)
    assert ei.value.status == E_UNS
