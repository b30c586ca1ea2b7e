// qmm_api.cpp -- the C ABI (include/qmm.h): argument checks, launch plans,
// dispatch onto the caller's stream.  Every check runs before the first HIP
// call, so invalid calls are diagnosable on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/qmm.h"
#include "qmm_internal.h"

// ---- scratch of the allocation-free entry point (qmm_gemm_noalloc) --------
// One copy of this array exists on every GPU the library runs on, for the
// life of the process.  In host code its name is only a stand-in for the
// device address: that address is taken once per device with
// hipGetSymbolAddress (scratch_of_current_device) and only it is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

qmm_status fail(qmm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

qmm_status ok() {
  g_err[0] = '\0';
  return QMM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool group_supported(int g) { return g == 32 || g == 64 || g == 128 || g == 256; }

// Checks shared by qmm_gemv, qmm_gemm and qmm_dequant on the operand table.
// Sets *noop when a size is zero (after the enum / dtype checks).
qmm_status check_operands(const char* fn, const void* Q, const void* scales, const void* zeros,
                          int N, int K, int w_bit, int group_size, bool* noop) {
  *noop = false;
  if (N < 0 || K < 0) return fail(QMM_ERR_ARG, "%s: negative size N=%d K=%d", fn, N, K);
  if (w_bit != 2 && w_bit != 4 && w_bit != 8)
    return fail(QMM_ERR_ARG, "%s: w_bit must be 2, 4 or 8 (got %d)", fn, w_bit);
  if (w_bit == 8) {
    if (group_size != 0)
      return fail(QMM_ERR_ARG, "%s: int8 uses a per-row scale; group_size must be 0 (got %d)",
                  fn, group_size);
    if (zeros != nullptr) return fail(QMM_ERR_ARG, "%s: int8 takes no zero points", fn);
  } else if (group_size == QMM_PER_COLUMN) {
    if (K % (32 / w_bit) != 0)
      return fail(QMM_ERR_ARG, "%s: K=%d is not a multiple of %d", fn, K, 32 / w_bit);
    if (K % 32 != 0)
      return fail(QMM_ERR_UNSUPPORTED, "%s: per-column scales need K %% 32 == 0 (K=%d)", fn, K);
  } else {
    if (group_size <= 0)
      return fail(QMM_ERR_ARG, "%s: group_size must be positive or QMM_PER_COLUMN (got %d)", fn,
                  group_size);
    if (K % group_size != 0)
      return fail(QMM_ERR_ARG, "%s: K=%d is not a multiple of group_size=%d", fn, K, group_size);
    if (!group_supported(group_size))
      return fail(QMM_ERR_UNSUPPORTED, "%s: group_size %d not built (32, 64, 128, 256)", fn,
                  group_size);
  }
  if (N == 0 || K == 0) {
    *noop = true;
    return QMM_OK;
  }
  if (Q == nullptr || scales == nullptr)
    return fail(QMM_ERR_ARG, "%s: NULL Q or scales", fn);
  if (!aligned16(Q) || !aligned16(scales) || !aligned16(zeros))
    return fail(QMM_ERR_ARG, "%s: Q, scales and zeros must be 16-byte aligned", fn);
  return QMM_OK;
}

qmm_status check_matmul(const char* fn, const void* x, const void* Q, const void* scales,
                        const void* zeros, const void* y, int y_dtype, int M, int N, int K,
                        int w_bit, int group_size, int x_dtype, bool* noop) {
  if (M < 0) return fail(QMM_ERR_ARG, "%s: negative M=%d", fn, M);
  if (x_dtype != QMM_F16 && x_dtype != QMM_BF16)
    return fail(QMM_ERR_ARG, "%s: x_dtype must be QMM_F16 or QMM_BF16 (got %d)", fn, x_dtype);
  if (y_dtype != QMM_F32 && y_dtype != QMM_F16 && y_dtype != QMM_BF16)
    return fail(QMM_ERR_ARG, "%s: y_dtype must be QMM_F32, QMM_F16 or QMM_BF16 (got %d)", fn,
                y_dtype);
  qmm_status st = check_operands(fn, Q, scales, zeros, N, K, w_bit, group_size, noop);
  if (st != QMM_OK || *noop) return st;
  if (M == 0) {
    *noop = true;
    return QMM_OK;
  }
  if (x == nullptr || y == nullptr) return fail(QMM_ERR_ARG, "%s: NULL x or y", fn);
  if (!aligned16(x) || !aligned16(y))
    return fail(QMM_ERR_ARG, "%s: x and y must be 16-byte aligned", fn);
  return QMM_OK;
}

qmm_status check_workspace(const char* fn, size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return QMM_OK;
  if (ws == nullptr || ws_bytes < need)
    return fail(QMM_ERR_ARG, "%s: workspace of %zu bytes needed (got %zu%s)", fn, need, ws_bytes,
                ws ? "" : ", NULL");
  if (!aligned16(ws)) return fail(QMM_ERR_ARG, "%s: workspace must be 16-byte aligned", fn);
  return QMM_OK;
}

qmm_status device_status(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(QMM_ERR_DEVICE, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return ok();
}

bool gemv_shape_ok(int N, int K, int w_bit) {
  return w_bit == 8 ? (K % 16 == 0) : (N % 4 == 0);
}

bool gemm_shape_ok(int N, int K, int w_bit) {
  return N % 16 == 0 && K % qmm::mfma_kblock(w_bit) == 0;
}

// Per-column scales are one group spanning K.  The GEMV and dequant kernels
// take the group size at run time, so there it is K itself; the GEMM
// kernels are built for fixed group sizes, so they run the largest built
// size dividing K with every group index masked to 0.
int gemv_group(int K, int group_size) { return group_size == QMM_PER_COLUMN ? K : group_size; }
int gemm_group(int K, int group_size) {
  if (group_size != QMM_PER_COLUMN) return group_size;
  return K % 256 == 0 ? 256 : (K % 128 == 0 ? 128 : (K % 64 == 0 ? 64 : 32));
}
int group_mask(int group_size) { return group_size == QMM_PER_COLUMN ? 0 : -1; }

// Zeroes the tickets at the head of the scratch before a call that uses it
// (a kernel, not a memset, so the call can be captured in a HIP graph).
__global__ void clear_tickets_kernel(uint32_t* t, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) t[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first call on that device (with it current) and kept.
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace qmm {
int env_int(const char* name) {
  const char* v = getenv(name);
  if (v == nullptr || *v == '\0') return -1;
  return atoi(v);
}
}  // namespace qmm

extern "C" {

int qmm_version(void) { return (0 << 16) | 1; }

const char* qmm_last_error(void) { return g_err; }

size_t qmm_packed_bytes(int N, int K, int w_bit, int layout) {
  if (N < 0 || K < 0) return 0;
  if (w_bit != 2 && w_bit != 4 && w_bit != 8) return 0;
  if (layout == QMM_LAYOUT_CANON) {
    if (w_bit != 8 && K % (32 / w_bit) != 0) return 0;
  } else if (layout == QMM_LAYOUT_MFMA) {
    if (!gemm_shape_ok(N, K, w_bit)) return 0;
  } else {
    return 0;
  }
  return (size_t)N * K * w_bit / 8;
}

static qmm_status layout_call(const char* fn, const void* src, void* dst, int N, int K,
                              int w_bit, void* stream, bool to_mfma) {
  if (N < 0 || K < 0) return fail(QMM_ERR_ARG, "%s: negative size N=%d K=%d", fn, N, K);
  if (w_bit != 2 && w_bit != 4 && w_bit != 8)
    return fail(QMM_ERR_ARG, "%s: w_bit must be 2, 4 or 8 (got %d)", fn, w_bit);
  if (N == 0 || K == 0) return ok();
  if (!gemm_shape_ok(N, K, w_bit))
    return fail(QMM_ERR_UNSUPPORTED, "%s: tile layout needs N %% 16 == 0 and K %% %d == 0", fn,
                qmm::mfma_kblock(w_bit));
  if (src == nullptr || dst == nullptr) return fail(QMM_ERR_ARG, "%s: NULL buffer", fn);
  if (!aligned16(src) || !aligned16(dst))
    return fail(QMM_ERR_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t bytes = (size_t)N * K * w_bit / 8;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return fail(QMM_ERR_ARG, "%s: buffers overlap", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = to_mfma ? qmm::launch_pack(src, dst, N, K, w_bit, s)
                         : qmm::launch_unpack_layout(src, dst, N, K, w_bit, s);
  return device_status(fn, e);
}

qmm_status qmm_pack(const void* Q_canon, void* Q_mfma, int N, int K, int w_bit, void* stream) {
  return layout_call("qmm_pack", Q_canon, Q_mfma, N, K, w_bit, stream, true);
}

qmm_status qmm_unpack_layout(const void* Q_mfma, void* Q_canon, int N, int K, int w_bit,
                             void* stream) {
  return layout_call("qmm_unpack_layout", Q_mfma, Q_canon, N, K, w_bit, stream, false);
}

size_t qmm_workspace_bytes(int M, int N, int K, int w_bit, int group_size) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (w_bit != 2 && w_bit != 4 && w_bit != 8) return 0;
  if (w_bit != 8) {
    if (group_size == QMM_PER_COLUMN) {
      if (K % 32 != 0) return 0;
    } else if (group_size <= 0 || K % group_size != 0 || !group_supported(group_size)) {
      return 0;
    }
  }
  size_t need = 0;
  if (M <= 16 && w_bit != 8 && gemv_shape_ok(N, K, w_bit)) {
    const size_t g =
        qmm::plan_gemv_lowbit(M, N, K, w_bit, gemv_group(K, group_size)).workspace_bytes;
    if (g > need) need = g;
  }
  if (gemm_shape_ok(N, K, w_bit)) {
    const size_t g = qmm::plan_gemm(M, N, K, w_bit, gemm_group(K, group_size)).workspace_bytes;
    if (g > need) need = g;
  }
  return need;
}

static qmm_status gemv_impl(const char* fn, const void* x, const void* Q, const void* scales,
                            const void* zeros, void* y, int y_dtype, int M, int N, int K,
                            int w_bit, int group_size, int x_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bool noop = false;
  qmm_status st = check_matmul(fn, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
                               x_dtype, &noop);
  if (st != QMM_OK) return st;
  if (noop) return ok();
  if (M > 16)
    return fail(QMM_ERR_UNSUPPORTED, "%s: M=%d > 16; use qmm_gemm for larger batches", fn, M);
  if (!gemv_shape_ok(N, K, w_bit))
    return fail(QMM_ERR_UNSUPPORTED, "%s: needs %s", fn,
                w_bit == 8 ? "K % 16 == 0 for int8" : "N % 4 == 0 for low-bit weights");
  const int gs = gemv_group(K, group_size);
  qmm::MatmulArgs a{x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, gs, -1, x_dtype, workspace,
                    reinterpret_cast<hipStream_t>(stream)};
  if (w_bit == 8) {
    const qmm::GemvInt8Plan p = qmm::plan_gemv_int8(M, N, K);
    return device_status(fn, qmm::launch_gemv_int8(a, p));
  }
  const qmm::GemvLowbitPlan p = qmm::plan_gemv_lowbit(M, N, K, w_bit, gs);
  st = check_workspace(fn, p.workspace_bytes, workspace, workspace_bytes);
  if (st != QMM_OK) return st;
  return device_status(fn, qmm::launch_gemv_lowbit(a, p));
}

// noalloc: the allocation-free entry point -- the workspace is the current
// device's scratch array, its tickets cleared first on `stream`.
static qmm_status gemm_impl(const char* fn, const void* x, const void* Q, const void* scales,
                            const void* zeros, void* y, int y_dtype, int M, int N, int K,
                            int w_bit, int group_size, int x_dtype, void* workspace,
                            size_t workspace_bytes, void* stream, bool noalloc = false) {
  bool noop = false;
  qmm_status st = check_matmul(fn, x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
                               x_dtype, &noop);
  if (st != QMM_OK) return st;
  if (noop) return ok();
  if (!gemm_shape_ok(N, K, w_bit))
    return fail(QMM_ERR_UNSUPPORTED, "%s: tile layout needs N %% 16 == 0 and K %% %d == 0", fn,
                qmm::mfma_kblock(w_bit));
  // the kernels carry their column-tile count in 24 bits (N / 16 < 2^24)
  if (N >= (1 << 28))
    return fail(QMM_ERR_UNSUPPORTED, "%s: N=%d too large (N < 2^28)", fn, N);
  const int gs = gemm_group(K, group_size);
  // without a workspace the plan keeps every partial sum inside a workgroup
  const qmm::GemmPlan p = qmm::plan_gemm(M, N, K, w_bit, gs, noalloc || workspace != nullptr);
  if (p.kind < 0) return fail(QMM_ERR_UNSUPPORTED, "%s: no MFMA kernel for this shape", fn);
  // the kernels address a workgroup's x rows (up to 64 rows of K; 256 for
  // M > 64) and weight strips with 32-bit byte offsets
  if (p.kind != 1 && (int64_t)K * 128 >= (int64_t(1) << 31))
    return fail(QMM_ERR_UNSUPPORTED, "%s: K=%d too large for M <= 64 (K < 2^24)", fn, K);
  if (p.kind == 1 && (int64_t)K * 512 >= (int64_t(1) << 31))
    return fail(QMM_ERR_UNSUPPORTED, "%s: K=%d too large for M > 64 (K < 2^22)", fn, K);
  // ... and their scale and zero rows too: the scale table must stay below 2 GiB
  if (w_bit != 8) {
    const int64_t G = group_size == QMM_PER_COLUMN ? 1 : K / group_size;
    if (G * (int64_t)N >= (int64_t(1) << 30))
      return fail(QMM_ERR_UNSUPPORTED, "%s: scale table of %lld x %d too large (< 2^30 entries)",
                  fn, (long long)G, N);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (noalloc) {
    if (p.workspace_bytes > QMM_NOALLOC_SCRATCH_BYTES)
      return fail(QMM_ERR_UNSUPPORTED,
                  "%s: this shape needs %zu bytes of scratch, more than the %zu the "
                  "allocation-free entry point holds (use qmm_gemm_ex with a workspace)",
                  fn, p.workspace_bytes, (size_t)QMM_NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    if (p.workspace_bytes > 0) {
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return device_status(fn, e);
      if (s != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(s, &sd);
        if (e != hipSuccess) return device_status(fn, e);
        if ((int)sd != cur)
          return fail(QMM_ERR_ARG, "%s: stream belongs to device %d, the current device is %d",
                      fn, (int)sd, cur);
      }
      e = scratch_of_current_device(&workspace);
      if (e != hipSuccess) return device_status(fn, e);
      const int tickets = (int)(((long)p.n_tiles * p.m_tiles + 63) & ~63L);
      e = qmm::launch_kernel(clear_tickets_kernel, dim3((tickets + 255) / 256), dim3(256), s,
                             workspace, tickets);
      if (e != hipSuccess) return device_status(fn, e);
    }
  } else {
    st = check_workspace(fn, p.workspace_bytes, workspace, workspace_bytes);
    if (st != QMM_OK) return st;
  }
  qmm::MatmulArgs a{x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, gs, group_mask(group_size),
                    x_dtype, workspace, s};
  return device_status(fn, qmm::launch_gemm(a, p));
}

qmm_status qmm_gemv(const void* x, const void* Q, const void* scales, const void* zeros, float* y,
                    int M, int N, int K, int w_bit, int group_size, int x_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return gemv_impl("qmm_gemv", x, Q, scales, zeros, y, QMM_F32, M, N, K, w_bit, group_size,
                   x_dtype, workspace, workspace_bytes, stream);
}

qmm_status qmm_gemv_ex(const void* x, const void* Q, const void* scales, const void* zeros,
                       void* y, int y_dtype, int M, int N, int K, int w_bit, int group_size,
                       int x_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return gemv_impl("qmm_gemv_ex", x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
                   x_dtype, workspace, workspace_bytes, stream);
}

qmm_status qmm_gemm(const void* x, const void* Q, const void* scales, const void* zeros, float* y,
                    int M, int N, int K, int w_bit, int group_size, int x_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return gemm_impl("qmm_gemm", x, Q, scales, zeros, y, QMM_F32, M, N, K, w_bit, group_size,
                   x_dtype, workspace, workspace_bytes, stream);
}

qmm_status qmm_gemm_ex(const void* x, const void* Q, const void* scales, const void* zeros,
                       void* y, int y_dtype, int M, int N, int K, int w_bit, int group_size,
                       int x_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl("qmm_gemm_ex", x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit, group_size,
                   x_dtype, workspace, workspace_bytes, stream);
}

qmm_status qmm_gemm_noalloc(const void* x, const void* Q, const void* scales, const void* zeros,
                            void* y, int y_dtype, int M, int N, int K, int w_bit, int group_size,
                            int x_dtype, void* stream) {
  return gemm_impl("qmm_gemm_noalloc", x, Q, scales, zeros, y, y_dtype, M, N, K, w_bit,
                   group_size, x_dtype, nullptr, 0, stream, true);
}

qmm_status qmm_dequant(const void* Q, int layout, const void* scales, const void* zeros,
                       float* w_out, int N, int K, int w_bit, int group_size, void* stream) {
  const char* fn = "qmm_dequant";
  if (layout != QMM_LAYOUT_CANON && layout != QMM_LAYOUT_MFMA)
    return fail(QMM_ERR_ARG, "%s: unknown layout %d", fn, layout);
  bool noop = false;
  qmm_status st = check_operands(fn, Q, scales, zeros, N, K, w_bit, group_size, &noop);
  if (st != QMM_OK) return st;
  if (noop) return ok();
  if (w_out == nullptr) return fail(QMM_ERR_ARG, "%s: NULL w_out", fn);
  if (layout == QMM_LAYOUT_MFMA && !gemm_shape_ok(N, K, w_bit))
    return fail(QMM_ERR_UNSUPPORTED, "%s: tile layout needs N %% 16 == 0 and K %% %d == 0", fn,
                qmm::mfma_kblock(w_bit));
  if (layout == QMM_LAYOUT_CANON && w_bit != 8 && K % (32 / w_bit) != 0)
    return fail(QMM_ERR_ARG, "%s: K must be a multiple of %d", fn, 32 / w_bit);
  return device_status(fn, qmm::launch_dequant(Q, layout, scales, zeros, w_out, N, K, w_bit,
                                               gemv_group(K, group_size),
                                               reinterpret_cast<hipStream_t>(stream)));
}

static qmm_status t2_shape(const char* fn, int N, int K, bool* noop) {
  *noop = false;
  if (N < 0 || K < 0) return fail(QMM_ERR_ARG, "%s: negative size N=%d K=%d", fn, N, K);
  if (N == 0 || K == 0) {
    *noop = true;
    return QMM_OK;
  }
  if (N % 16 != 0 || K % 256 != 0)
    return fail(QMM_ERR_UNSUPPORTED, "%s: needs N %% 16 == 0 and K %% 256 == 0 (N=%d K=%d)", fn,
                N, K);
  return QMM_OK;
}

static qmm_status t2_layout_call(const char* fn, const void* src, void* dst, int N, int K,
                                 void* stream, bool to_tile) {
  bool noop = false;
  qmm_status st = t2_shape(fn, N, K, &noop);
  if (st != QMM_OK) return st;
  if (noop) return ok();
  if (src == nullptr || dst == nullptr) return fail(QMM_ERR_ARG, "%s: NULL buffer", fn);
  if (!aligned16(src) || !aligned16(dst))
    return fail(QMM_ERR_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t bytes = (size_t)N * K / 4;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return fail(QMM_ERR_ARG, "%s: buffers overlap", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return device_status(fn, to_tile ? qmm::launch_t2_pack(src, dst, N, K, s)
                                   : qmm::launch_t2_unpack(src, dst, N, K, s));
}

qmm_status qmm_t2_pack(const void* W_page, void* W_tile, int N, int K, void* stream) {
  return t2_layout_call("qmm_t2_pack", W_page, W_tile, N, K, stream, true);
}

qmm_status qmm_t2_unpack_layout(const void* W_tile, void* W_page, int N, int K, void* stream) {
  return t2_layout_call("qmm_t2_unpack_layout", W_tile, W_page, N, K, stream, false);
}

qmm_status qmm_i8t2_gemm(const void* x, const void* W_tile, int32_t* y, int M, int N, int K,
                         void* stream) {
  const char* fn = "qmm_i8t2_gemm";
  if (M < 0) return fail(QMM_ERR_ARG, "%s: negative M=%d", fn, M);
  bool noop = false;
  qmm_status st = t2_shape(fn, N, K, &noop);
  if (st != QMM_OK) return st;
  if (noop || M == 0) return ok();
  // large M: 32-bit buffer offsets span a 256-row tile of x (256 K bytes)
  if (M > 64 && K >= (1 << 23))
    return fail(QMM_ERR_UNSUPPORTED, "%s: K=%d too large for M > 64 (K < 2^23)", fn, K);
  if (x == nullptr || W_tile == nullptr || y == nullptr)
    return fail(QMM_ERR_ARG, "%s: NULL x, W_tile or y", fn);
  if (!aligned16(x) || !aligned16(W_tile) || !aligned16(y))
    return fail(QMM_ERR_ARG, "%s: x, W_tile and y must be 16-byte aligned", fn);
  return device_status(fn, qmm::launch_i8t2_gemm(x, W_tile, y, M, N, K,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

qmm_status qmm_quantize(const void* W, int w_dtype, void* qw, void* scales, void* qzeros, int N,
                        int K, int w_bit, int group_size, int symmetric, void* stream) {
  const char* fn = "qmm_quantize";
  if (w_dtype != QMM_F32 && w_dtype != QMM_F16 && w_dtype != QMM_BF16)
    return fail(QMM_ERR_ARG, "%s: w_dtype must be QMM_F32, QMM_F16 or QMM_BF16 (got %d)", fn,
                w_dtype);
  if (w_bit == 8) return fail(QMM_ERR_ARG, "%s: w_bit must be 2 or 4 (got 8)", fn);
  if (symmetric != 0 && symmetric != 1)
    return fail(QMM_ERR_ARG, "%s: symmetric must be 0 or 1 (got %d)", fn, symmetric);
  if (symmetric && qzeros != nullptr)
    return fail(QMM_ERR_ARG, "%s: symmetric quantization writes no zero points (qzeros must be "
                "NULL)", fn);
  bool noop = false;
  // the operand checks of the matmul (sizes, w_bit, group_size, alignment)
  qmm_status st = check_operands(fn, qw, scales, qzeros, N, K, w_bit, group_size, &noop);
  if (st != QMM_OK || noop) return noop ? ok() : st;
  if (W == nullptr || (!symmetric && qzeros == nullptr))
    return fail(QMM_ERR_ARG, "%s: NULL W%s", fn, symmetric ? "" : " or qzeros");
  if (!aligned16(W)) return fail(QMM_ERR_ARG, "%s: W must be 16-byte aligned", fn);
  return device_status(fn, qmm::launch_quantize(W, w_dtype, qw, scales, qzeros, N, K, w_bit,
                                                gemv_group(K, group_size), symmetric,
                                                reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
