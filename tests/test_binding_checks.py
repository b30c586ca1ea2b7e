"""The Python binding refuses tensors the kernels could not use -- a wrong
dtype, a non-contiguous view, too few bytes for the sizes, operands on
different devices, a tensor in host memory -- with QmmError, before the
library is called.  CPU only: the checks run in order dtype, contiguity,
size, device, so host tensors reach each of them without a GPU."""
import pytest
import torch

qmm = pytest.importorskip("gemv_only_quant_amd")

M, N, K = 2, 64, 256


def lowbit(dtype_x=torch.float16):
    x = torch.zeros((M, K), dtype=dtype_x)
    Q = torch.zeros((K // 8, N), dtype=torch.int32)
    s = torch.zeros((K // 128, N), dtype=torch.float16)
    z = torch.zeros((1, N), dtype=torch.int32)
    y = torch.zeros((M, N), dtype=torch.float32)
    return x, Q, s, z, y


def call(x, Q, s, z, y, entry="qmm_gemv", **kw):
    getattr(qmm, entry)(x, Q, s, z, y, M, N, K, 4, 128, **kw)


def raises(fn, text):
    with pytest.raises(qmm.QmmError) as e:
        fn()
    assert text in str(e.value), str(e.value)
    assert e.value.status == qmm.QMM_ERR_ARG


@pytest.mark.parametrize("entry", ["qmm_gemv", "qmm_gemm", "qmm_gemv_ex", "qmm_gemm_ex"])
def test_host_tensors_refused(entry):
    raises(lambda: call(*lowbit(), entry=entry), "must be a GPU tensor")


def test_non_contiguous_x_refused():
    x, Q, s, z, y = lowbit()
    wide = torch.zeros((M, 2 * K), dtype=torch.float16)
    raises(lambda: call(wide[:, :K], Q, s, z, y), "x must be contiguous")


def test_wrong_dtypes_refused():
    x, Q, s, z, y = lowbit()
    raises(lambda: call(x.float(), Q, s, z, y), "x must be float16 or bfloat16")
    raises(lambda: call(x, Q.to(torch.int64), s, z, y), "Q must be int32")
    raises(lambda: call(x, Q, s.float(), z, y), "scales must be float16")
    raises(lambda: call(x, Q, s, z.to(torch.int16), y), "zeros must be int32")
    raises(lambda: call(x, Q, s, z, y.half()), "y must be float32")
    # the output type of the _ex entries follows y unless given, and must match it
    raises(lambda: call(x, Q, s, z, y, entry="qmm_gemv_ex", y_dtype=qmm.QMM_BF16),
           "y must be bfloat16")


def test_short_operands_refused():
    x, Q, s, z, y = lowbit()
    raises(lambda: call(x[:1], Q, s, z, y), "x holds")
    raises(lambda: call(x, Q[:-1], s, z, y), "Q holds")
    raises(lambda: call(x, Q, s[:, :N // 2].contiguous(), z, y), "scales holds")
    raises(lambda: call(x, Q, s, z[:, :8].contiguous(), y), "zeros holds")
    raises(lambda: call(x, Q, s, z, y[:1]), "y holds")
    ws = torch.zeros(16, dtype=torch.uint8)
    raises(lambda: call(x, Q, s, z, y, workspace=ws, workspace_bytes=1024), "workspace holds")


def test_int8_operands_checked():
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    Q = torch.zeros((N, K), dtype=torch.int8)
    s = torch.zeros((N,), dtype=torch.float32)
    y = torch.zeros((M, N), dtype=torch.float32)
    go = lambda **o: qmm.qmm_gemv(o.get("x", x), o.get("Q", Q), o.get("s", s), None, y, M, N,
                                  K, 8, 0)
    raises(lambda: go(s=s.half()), "scales must be float32")
    raises(lambda: go(Q=Q[:, :K // 2].contiguous()), "Q holds")
    raises(lambda: go(), "must be a GPU tensor")


def test_layout_ternary_and_quantizer_entries_checked():
    Q = torch.zeros((K // 8, N), dtype=torch.int32)
    raises(lambda: qmm.qmm_pack(Q, torch.zeros(4, dtype=torch.int32), N, K, 4), "destination holds")
    Wp = torch.zeros((K // 4, N), dtype=torch.uint8)
    raises(lambda: qmm.qmm_t2_pack(Wp, Wp.clone(), N, K), "must be a GPU tensor")
    raises(lambda: qmm.qmm_i8t2_gemm(torch.zeros((M, K), dtype=torch.int8), Wp,
                                     torch.zeros((M, N), dtype=torch.float32), M, N, K),
           "y must be int32")
    W = torch.zeros((K, N), dtype=torch.float16)
    raises(lambda: qmm.qmm_quantize(W, qmm.QMM_F32, Q, torch.zeros((2, N), dtype=torch.float16),
                                    None, N, K, 4, 128, True), "W must be float32")
    raises(lambda: qmm.qmm_dequant(Q, qmm.QMM_LAYOUT_CANON, torch.zeros((2, N), dtype=torch.float16),
                                   None, torch.zeros((K, N // 2), dtype=torch.float32), N, K, 4,
                                   128), "w_out holds")


def test_raw_pointers_pass_through_to_the_library():
    """Integer pointers are the caller's responsibility; the library's own
    checks still run (here: M > 16 on the GEMV path, refused before launch)."""
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_gemv(0x10000, 0x10000, 0x10000, None, 0x10000, 17, N, K, 4, 128,
                     x_dtype=qmm.QMM_F16, stream=0)
    assert e.value.status == qmm.QMM_ERR_UNSUPPORTED
