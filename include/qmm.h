/*
 * qmm.h -- weight-only quantized matmul for AMD Instinct MI355X (gfx950).
 *
 *     y[m][n] = sum_k x[m][k] * W[k][n],     W = dequant(Q)
 *
 * x is fp16 or bf16, Q holds int4 / int2 codes with per-group fp16 scales
 * and integer zero points, or int8 codes with a per-output-row fp32 scale;
 * accumulation is fp32 and y is fp32.
 *
 * Where the operation is defined:
 *  - operands and the canonical packed layout: BitDistiller,
 *    quantization/triton_kernels.py, quant_matmul_kernel (docstring shapes
 *    a (M,K), qw (K/pack_num, N), scales (K/group_size, N),
 *    qzeros (K/group_size/pack_num, N); the unpack shifts the word right by
 *    (k mod pack_num) * w_bit and masks with offset; group index
 *    floor(k / group_size));
 *  - the symmetric int4 zero point 8: aphrodite-engine marlin_cuda_kernel.cu,
 *    dequant() (the zero point 8 folded into its int4 conversion constants);
 *  - int8 weights (N, K) with the fp32 row scale applied after an fp32 sum:
 *    tiny-llm src/tinyllm/kernels/int8_gemv.py (module and int8_matmul
 *    docstrings);
 *  - the zero-size early return: marlin_cuda_kernel.cu, marlin_cuda();
 *  - per-column scales (one scale row, group size -1) and a 16-bit output:
 *    marlin_cuda_kernel.cu, marlin_cuda() (groupsize -1 when the scales
 *    have a single row) and the kernel's write-out step (the per-column
 *    scale applied to the accumulated result as it is written in fp16).
 *
 * Conventions for every entry point
 *  - Data pointers are DEVICE pointers owned by the caller, contiguous,
 *    row-major and 16-byte aligned.  `stream` is a hipStream_t passed as
 *    void* (NULL = the null stream).  Calls are asynchronous on `stream`,
 *    never synchronise and never allocate.
 *  - Every argument is checked before any HIP call; a failing call returns a
 *    status, launches nothing and sets a thread-local message read with
 *    qmm_last_error().
 *  - M == 0, N == 0 or K == 0 (with otherwise valid arguments) is a no-op
 *    returning QMM_OK.
 *
 * Operand table (pack = 32 / w_bit, G = K / group_size, Zr = ceil(G / pack))
 *   w_bit 4 or 2:
 *     Q       canonical: (K/pack, N) int32; code k of column n at bit
 *             (k % pack) * w_bit of word [k / pack][n], low field first.
 *             MFMA layout: see qmm_pack.
 *     scales  (G, N) fp16
 *     zeros   NULL (symmetric, z = 2^(w_bit-1): 8 for int4, 2 for int2) or
 *             (Zr, N) int32, zero of group g at bit (g % pack) * w_bit of
 *             word [g / pack][n] (fields past G are ignored)
 *     group_size in {32, 64, 128, 256}, K % group_size == 0, or
 *     QMM_PER_COLUMN (-1): one group spanning K -- scales (1, N), zeros
 *     NULL or (1, N) with the zero in field 0 -- and K % 32 == 0
 *     W[k][n] = (q - z) * s[k / group_size][n]   (per column: s[0][n])
 *   w_bit 8:
 *     Q       (N, K) int8 (two's complement), same in both layouts' inputs
 *     scales  (N,) fp32; zeros must be NULL; group_size must be 0
 *     y[m][n] = scales[n] * sum_k x[m][k] * Q[n][k]
 *   x (M, K) fp16 or bf16 (x_dtype), y (M, N) fp32, fully overwritten
 *   (qmm_gemv_ex / qmm_gemm_ex: fp32, fp16 or bf16, the fp32 result
 *   rounded once to nearest even).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QMM_API __attribute__((visibility("default")))
#else
#define QMM_API
#endif

typedef enum {
    QMM_OK = 0,
    QMM_ERR_ARG = 1,          /* invalid argument (NULL, negative, bad enum, misaligned,
                                 K % group_size, workspace too small, ...) */
    QMM_ERR_UNSUPPORTED = 2,  /* valid but not built: shape or group size outside
                                 the supported set, M > 16 on qmm_gemv */
    QMM_ERR_DEVICE = 3        /* a HIP call or kernel launch failed */
} qmm_status;

typedef enum { QMM_F16 = 0, QMM_BF16 = 1, QMM_F32 = 2 } qmm_dtype;  /* x: F16 / BF16 only */

/* group_size value for per-column scales and zeros (one group spanning K) */
#define QMM_PER_COLUMN (-1)
typedef enum { QMM_LAYOUT_CANON = 0, QMM_LAYOUT_MFMA = 1 } qmm_layout;

/* Library version, (major << 16) | minor. */
QMM_API int qmm_version(void);

/* Message describing the last failing call on this thread ("" if none). */
QMM_API const char* qmm_last_error(void);

/* Bytes of Q for an (N, K) weight in `layout`; 0 if the combination is
 * invalid.  Both layouts hold N*K*w_bit/8 bytes: the canonical low-bit
 * weight is BitDistiller quant_matmul_kernel's qw, (K/pack_num, N) int32
 * (its docstring shapes); int8 is tiny-llm int8_gemv.py's q, (N, K) int8
 * (int8_matmul docstring); the tile layout (qmm_pack) is a permutation of
 * the same bits. */
QMM_API size_t qmm_packed_bytes(int N, int K, int w_bit, int layout);

/*
 * qmm_pack: canonical Q -> MFMA tile layout (offline, integer bijection).
 * The pages print no repack routine (Marlin consumes a pre-permuted B but
 * its permutation is not shown), so this layout is this library's own:
 *   columns in strips of 16, K in blocks of KB = 128 (int4), 256 (int2)
 *   or 64 (int8); block (strip s, K-block kb) is 1024 contiguous bytes at
 *   offset 1024 * (s * (K/KB) + kb).  Bytes [16 L, 16 L + 16) of a block
 *   ("lane" L in 0..63) serve column 16 s + L % 16 and k-octet c = L / 16:
 *     int4: int32 word j (0..3) holds k = 128 kb + 32 j + 8 c + i (i 0..7),
 *           code i in nibble i/2 for even i, 4 + i/2 for odd i;
 *     int2: word j holds k = 256 kb + 64 j + 32 h + 8 c + i (h 0..1),
 *           code in 2-bit field 4 h + i/2 (even i) or 8 + 4 h + i/2 (odd i);
 *     int8: byte 8 h + i holds k = 64 kb + 32 h + 8 c + i.
 * Requires N % 16 == 0 and K % KB == 0.  Q_canon and Q_mfma must not
 * overlap.  qmm_unpack_layout is the exact inverse.
 */
QMM_API qmm_status qmm_pack(const void* Q_canon, void* Q_mfma, int N, int K, int w_bit, void* stream);
QMM_API qmm_status qmm_unpack_layout(const void* Q_mfma, void* Q_canon, int N, int K, int w_bit,
                             void* stream);

/*
 * Scratch device memory a qmm_gemm / qmm_gemm_ex call can use for the given
 * shape beyond its inputs and outputs (cf. the lock workspace Marlin's
 * marlin_cuda() takes from its caller, and its striped partition of K over
 * thread blocks with a global reduction).  Nonzero for shapes whose column
 * tiles alone leave most compute units idle: K is then split over several
 * workgroups per tile, which leave partial tiles and an arrival ticket per
 * tile in the workspace; the last workgroup of a tile to arrive adds the
 * partials in a fixed order and writes y.
 *   - Caller-owned device memory of at least this many bytes, 16-byte
 *     aligned, ZERO-FILLED before its first use.  Every call leaves it
 *     re-armed (all tickets back at zero), so one workspace serves any
 *     sequence of calls on one stream; calls that may run concurrently need
 *     distinct workspaces.
 *   - A NULL workspace is always accepted: the call then runs a plan that
 *     keeps every partial sum inside a workgroup (slower on such shapes).
 *     A non-NULL one smaller than this size is QMM_ERR_ARG.
 *   - qmm_gemv and the ternary product never use one.
 * Returns 0 for shapes that need none and for invalid arguments.
 */
QMM_API size_t qmm_workspace_bytes(int M, int N, int K, int w_bit, int group_size);

/*
 * qmm_gemv: decode / skinny path, 1 <= M <= 16, Q in the CANONICAL layout.
 * Streams each packed weight byte once per call.  Low-bit: N % 4 == 0.
 * int8: K % 16 == 0.  M > 16 returns QMM_ERR_UNSUPPORTED (cf. the int8
 * decode kernel's MAX_M row limit in tiny-llm int8_gemv.py).
 */
QMM_API qmm_status qmm_gemv(const void* x, const void* Q, const void* scales, const void* zeros,
                    float* y, int M, int N, int K, int w_bit, int group_size, int x_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmm_gemm: the same product as qmm_gemv for any M >= 1, Q in the MFMA
 * layout produced by qmm_pack (N % 16 == 0, K % KB == 0), contracted on the
 * matrix cores.  The operation is BitDistiller quant_matmul_kernel's
 * a (M,K) times dequant(qw) accumulated in fp32 (int8: tiny-llm's
 * y = scale * (x . q) with the scale after the sum); that larger batches are
 * a dense contraction for the matrix units is tiny-llm int8_gemv.py's note
 * on MAX_M (past a few rows the product is a plain GEMM) and the premise of Marlin's
 * tensor-core kernel (aphrodite-engine marlin_cuda_kernel.cu, Marlin<...>).
 * Output and errors as qmm_gemv; M > 16 is allowed.
 */
QMM_API qmm_status qmm_gemm(const void* x, const void* Q, const void* scales, const void* zeros,
                    float* y, int M, int N, int K, int w_bit, int group_size, int x_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmm_gemv_ex / qmm_gemm_ex: the same operations with y of type y_dtype
 * (QMM_F32, QMM_F16 or QMM_BF16; cf. Marlin's fp16 output).  The sum is
 * formed in fp32 exactly as in qmm_gemv / qmm_gemm and rounded once, to
 * nearest even, as it is stored; fp16 overflows to +-inf.  An unknown
 * y_dtype is QMM_ERR_ARG.  qmm_gemv / qmm_gemm are these with QMM_F32.
 */
QMM_API qmm_status qmm_gemv_ex(const void* x, const void* Q, const void* scales,
                               const void* zeros, void* y, int y_dtype, int M, int N, int K,
                               int w_bit, int group_size, int x_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);
QMM_API qmm_status qmm_gemm_ex(const void* x, const void* Q, const void* scales,
                               const void* zeros, void* y, int y_dtype, int M, int N, int K,
                               int w_bit, int group_size, int x_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * qmm_gemm_noalloc: qmm_gemm_ex for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing and takes no workspace:
 * where the plan splits K over workgroups (see qmm_workspace_bytes), the
 * tickets and partial tiles live in a scratch array the library holds on
 * each GPU it runs on (QMM_NOALLOC_SCRATCH_BYTES, kept until the process
 * ends), and a small kernel clears the tickets on `stream` before the
 * product.  Every call on a GPU shares that GPU's array, so calls that may
 * overlap on one GPU (on different streams) race: the caller serialises
 * them.  `stream` must belong to the current device (else QMM_ERR_ARG).  A
 * shape whose plan needs more scratch than the array holds is
 * QMM_ERR_UNSUPPORTED (qmm_gemm_ex with a workspace takes any size).
 * Operands, results and all other errors as qmm_gemm_ex.
 */
#define QMM_NOALLOC_SCRATCH_BYTES (8u << 20)
QMM_API qmm_status qmm_gemm_noalloc(const void* x, const void* Q, const void* scales,
                                    const void* zeros, void* y, int y_dtype, int M, int N,
                                    int K, int w_bit, int group_size, int x_dtype, void* stream);

/*
 * qmm_dequant: W (K, N) fp32 from Q in either layout, bit-exact:
 * W[k][n] = float(q - z) * float(s) for low-bit (exact in fp32), and
 * W[k][n] = float(Q[n][k]) for int8 (row scale NOT applied).  For tests.
 * The codes, group index and zero unpacking are BitDistiller
 * quant_matmul_kernel's ((qw >> shift) & offset, group floor(k/group_size));
 * (q - z) * s with an integer zero in code space is aphrodite-engine
 * marlin_cuda_kernel.cu dequant()'s symmetric (q - 8) * s with z read from
 * qzeros (the BitDistiller page is cut off before its own dequant line).
 * w_out is (K, N) fp32, fully overwritten; errors as qmm_gemv.
 */
QMM_API qmm_status qmm_dequant(const void* Q, int layout, const void* scales, const void* zeros,
                       float* w_out, int N, int K, int w_bit, int group_size, void* stream);

/*
 * int8 activations x ternary weights (liger-kernel ops/experimental/
 * mm_int8int2.py): y (M, N) int32 = x (M, K) int8 times W (K, N) with
 * values in {-1, 0, +1}, exact.  The page stores W as pack_weights does:
 * (K/4, N) uint8, K split into four consecutive quarters of R = K/4 rows,
 * quarter i in bits 2i..2i+1, each field the value + 1 (code 3 reads as +2,
 * as unpack_weights gives: it masks the field, shifts it down and subtracts 1).
 *
 * qmm_t2_pack rewrites that once into the tile layout qmm_i8t2_gemm reads:
 * 1 KiB blocks, one per (16-column strip s, 256-deep K block kb),
 * strip-major; bytes [16 L, 16 L + 16) of a block are lane L: column
 * 16 s + L % 16, lane group g = L / 16; dword j (0..3) of the lane holds
 * the codes of k = 256 kb + 64 j + 16 g + e, e = 0..15, code e at bit
 * 2 (4 (e % 4) + e / 4).  Both layouts take N * K / 4 bytes.  Requires
 * N % 16 == 0 and K % 256 == 0 (else QMM_ERR_UNSUPPORTED); buffers must
 * not overlap.  qmm_t2_unpack_layout is the exact inverse.
 */
QMM_API qmm_status qmm_t2_pack(const void* W_page, void* W_tile, int N, int K, void* stream);
QMM_API qmm_status qmm_t2_unpack_layout(const void* W_tile, void* W_page, int N, int K,
                                        void* stream);
/*
 * qmm_i8t2_gemm: y = x * W on the int8 matrix cores, W in the tile layout;
 * any M >= 1, N % 16 == 0, K % 256 == 0; y fully overwritten.  The sums are
 * exact for K < 2^23 (|x w| <= 256); larger K wraps as the page's int32
 * accumulator would.  For M > 64, K must be below 2^23 (QMM_ERR_UNSUPPORTED
 * otherwise).
 */
QMM_API qmm_status qmm_i8t2_gemm(const void* x, const void* W_tile, int32_t* y, int M, int N,
                                 int K, void* stream);

/*
 * qmm_quantize: the step before the matmul -- round-to-nearest quantization
 * of W (K, N) (w_dtype QMM_F32, QMM_F16 or QMM_BF16) into the canonical
 * operands above: qw (K/pack, N) int32, scales (G, N) fp16, and qzeros
 * (ceil(G/pack), N) int32 (asymmetric; must be NULL when symmetric != 0).
 * The pages give only those operand shapes (BitDistiller
 * quant_matmul_kernel); the rule is this library's: per group and column,
 * over [min(0, min w), max(0, max w)],
 *   asymmetric: s = (max - min) / (2^b - 1), z = clamp(rint(-min/s), 0, 2^b - 1)
 *   symmetric:  s = max(|max|, |min|) / (2^(b-1) - 1), z = 2^(b-1)
 *   q = clamp(rint(w / s) + z, 0, 2^b - 1),
 * s stored as fp16 (nearest even; 1.0 if that is 0), the codes taken from
 * the stored scale, every step in fp32 with correctly rounded division and
 * ties-to-even rint.  w_bit 2 or 4; group_size as for the matmul (including
 * QMM_PER_COLUMN).
 */
QMM_API qmm_status qmm_quantize(const void* W, int w_dtype, void* qw, void* scales, void* qzeros,
                                int N, int K, int w_bit, int group_size, int symmetric,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
