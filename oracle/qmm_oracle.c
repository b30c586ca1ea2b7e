/*
 * qmm_oracle.c -- plain CPU oracle for the weight-only quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY (see qmm_oracle.h): used by the tests, the smoke
 * check and the benchmark's CPU baseline, never by the product path.
 *
 * Sources of each step (pages are cited by project, file and passage):
 *  - canonical packing and unpack rule: BitDistiller, quantization/
 *    triton_kernels.py, quant_matmul_kernel -- operand shapes in its
 *    docstring, the per-element shifter (k mod pack_num) * w_bit and the
 *    "(packed >> shifter) & offset" unpack;
 *  - group index floor(k / group_size): same kernel, scale-loading step
 *    (k_iters_per_quant_group / grp_idx);
 *  - dequant w = (q - z) * s with an integer zero point, and the symmetric
 *    zero 8 for int4: aphrodite-engine marlin_cuda_kernel.cu, dequant()
 *    (the "-8 symmetric zero point" fused into its SUB/ADD constants);
 *  - int8 per-row scale applied after the sum over k, fp32 accumulation:
 *    tiny-llm src/tinyllm/kernels/int8_gemv.py, module docstring and
 *    int8_matmul() docstring;
 *  - per-column scales, group_size -1 (one scale row, one group spanning
 *    K): aphrodite-engine marlin_cuda_kernel.cu, marlin_cuda() (groupsize
 *    -1 when the scales have a single row).
 *
 * Readings where the pages are silent (the zero-point packing rule, the
 * symmetric zero for int2) are listed in the project design notes.
 */
#include "qmm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* c1: 16-bit float decodes, from the format definitions              */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 encodes zero and subnormals (fraction * 2^-24),
 * field 31 encodes infinities (fraction 0) and NaNs. */
float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v);
}

/* bfloat16 is by definition the upper 16 bits of an IEEE binary32 word. */
float orc_bf16_to_f32(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float v;
    memcpy(&v, &bits, sizeof v);
    return v;
}

void orc_f16_to_f32_n(const uint16_t* h, float* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

void orc_bf16_to_f32_n(const uint16_t* h, float* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(h[i]);
}

static double x_at(const uint16_t* x, int x_dtype, int K, int m, int k) {
    uint16_t h = x[(size_t)m * K + k];
    return (double)(x_dtype == 0 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h));
}

/* ------------------------------------------------------------------ */
/* argument checks                                                     */
/* ------------------------------------------------------------------ */

static int check_lowbit(int N, int K, int w_bit, int group_size) {
    if (N < 0 || K < 0) return -1;
    if (w_bit != 2 && w_bit != 4) return -1;
    if (group_size != -1 && group_size <= 0) return -1;
    if (group_size != -1 && K % group_size != 0) return -1;
    if (K % (32 / w_bit) != 0) return -1;
    return 0;
}

static int check_args(int N, int K, int w_bit, int group_size, const int32_t* zeros) {
    if (w_bit == 8) {
        if (N < 0 || K < 0 || group_size != 0 || zeros != NULL) return -1;
        return 0;
    }
    return check_lowbit(N, K, w_bit, group_size);
}

/* ------------------------------------------------------------------ */
/* c2/c3: unpack                                                       */
/* ------------------------------------------------------------------ */

/* Element k of column n sits in word k / pack of that column, at bit
 * (k mod pack) * w_bit, least significant first; the mask is 2^w_bit - 1
 * (BitDistiller quant_matmul_kernel: weight-load and unpack step). */
uint32_t orc_q_at(const int32_t* qw, int N, int w_bit, int k, int n) {
    int pack = 32 / w_bit;
    uint32_t word = (uint32_t)qw[(size_t)(k / pack) * N + n];
    return (word >> ((k % pack) * w_bit)) & ((1u << w_bit) - 1u);
}

/* Zero points are packed the same way along the group axis; without zeros
 * the symmetric midpoint 2^(w_bit-1) is used (8 for int4, as in Marlin's
 * dequant()). */
uint32_t orc_z_at(const int32_t* qz, int N, int w_bit, int g, int n) {
    if (qz == NULL) return 1u << (w_bit - 1);
    int pack = 32 / w_bit;
    uint32_t word = (uint32_t)qz[(size_t)(g / pack) * N + n];
    return (word >> ((g % pack) * w_bit)) & ((1u << w_bit) - 1u);
}

int orc_unpack_q(const int32_t* qw, int N, int K, int w_bit, uint8_t* q_out) {
    if (N < 0 || K < 0 || (w_bit != 2 && w_bit != 4) || K % (32 / w_bit)) return -1;
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            q_out[(size_t)k * N + n] = (uint8_t)orc_q_at(qw, N, w_bit, k, n);
    return 0;
}

int orc_unpack_z(const int32_t* qz, int N, int G, int w_bit, uint8_t* z_out) {
    if (N < 0 || G < 0 || (w_bit != 2 && w_bit != 4)) return -1;
    for (int g = 0; g < G; ++g)
        for (int n = 0; n < N; ++n)
            z_out[(size_t)g * N + n] = (uint8_t)orc_z_at(qz, N, w_bit, g, n);
    return 0;
}

/* ------------------------------------------------------------------ */
/* c4: dequant                                                         */
/* ------------------------------------------------------------------ */

/* w = (q - z) * s, s the fp16 scale of group floor(k / group_size), or of
 * the single group when group_size is -1 (per-column).
 * |q - z| <= 15 needs 4 bits and s has an 11-bit significand, so the fp32
 * product is exact.  int8: w = q exactly (|q| <= 128); the fp32 row scale
 * is applied after the sum (tiny-llm int8_gemv.py docstring). */
float orc_w_at(const void* Q, const void* scales, const int32_t* zeros,
               int N, int K, int w_bit, int group_size, int k, int n) {
    if (w_bit == 8) {
        const int8_t* q8 = (const int8_t*)Q;
        return (float)q8[(size_t)n * K + k];
    }
    int g = group_size == -1 ? 0 : k / group_size;
    int q = (int)orc_q_at((const int32_t*)Q, N, w_bit, k, n);
    int z = (int)orc_z_at(zeros, N, w_bit, g, n);
    float s = orc_f16_to_f32(((const uint16_t*)scales)[(size_t)g * N + n]);
    return (float)(q - z) * s;
}

int orc_dequant(const void* Q, const void* scales, const int32_t* zeros,
                int N, int K, int w_bit, int group_size, float* w_out) {
    if (check_args(N, K, w_bit, group_size, zeros)) return -1;
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            w_out[(size_t)k * N + n] =
                orc_w_at(Q, scales, zeros, N, K, w_bit, group_size, k, n);
    return 0;
}

/* ------------------------------------------------------------------ */
/* c5: the product, fp64 accumulation, k ascending                     */
/* ------------------------------------------------------------------ */

static double row_scale(const void* scales, int w_bit, int n) {
    return w_bit == 8 ? (double)((const float*)scales)[n] : 1.0;
}

/* Outputs (m, n) for every row m and the columns n0 <= n < n1.  xd is x
 * decoded to double, (M, K).  The columns are dequantized once into
 * column-major storage wt[n][k] (storage order only); each output is then
 * the fp64 sum over k ascending, with the int8 row scale applied after it. */
static int qmm_columns(const double* xd, const void* Q, const void* scales,
                       const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
                       int n0, int n1, double* y_ref, double* abs_ref) {
    float* wt = (float*)malloc(sizeof(float) * ((size_t)(n1 - n0) * K + 1));
    if (!wt) return -1;
    for (int n = n0; n < n1; ++n)
        for (int k = 0; k < K; ++k)
            wt[(size_t)(n - n0) * K + k] =
                orc_w_at(Q, scales, zeros, N, K, w_bit, group_size, k, n);
    for (int m = 0; m < M; ++m) {
        const double* xr = xd + (size_t)m * K;
        for (int n = n0; n < n1; ++n) {
            const float* w = wt + (size_t)(n - n0) * K;
            double s = row_scale(scales, w_bit, n);
            double acc = 0.0, ab = 0.0;
            for (int k = 0; k < K; ++k) {
                double p = xr[k] * (double)w[k];
                acc += p;
                ab += fabs(p * s);
            }
            y_ref[(size_t)m * N + n] = s * acc;
            abs_ref[(size_t)m * N + n] = ab;
        }
    }
    free(wt);
    return 0;
}

static double* decode_x(const uint16_t* x, int x_dtype, int M, int K) {
    double* xd = (double*)malloc(sizeof(double) * ((size_t)M * K + 1));
    if (!xd) return NULL;
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) xd[(size_t)m * K + k] = x_at(x, x_dtype, K, m, k);
    return xd;
}

int orc_qmm(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
            const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
            double* y_ref, double* abs_ref) {
    if (M < 0 || (x_dtype != 0 && x_dtype != 1)) return -1;
    if (check_args(N, K, w_bit, group_size, zeros)) return -1;
    double* xd = decode_x(x, x_dtype, M, K);
    if (!xd) return -1;
    int rc = qmm_columns(xd, Q, scales, zeros, M, N, K, w_bit, group_size, 0, N, y_ref, abs_ref);
    free(xd);
    return rc;
}

int orc_qmm_at(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
               const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
               int count, const int* ms, const int* ns, double* y_ref, double* abs_ref) {
    if (M < 0 || count < 0 || (x_dtype != 0 && x_dtype != 1)) return -1;
    if (check_args(N, K, w_bit, group_size, zeros)) return -1;
    for (int i = 0; i < count; ++i) {
        int m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double s = row_scale(scales, w_bit, n);
        double acc = 0.0, ab = 0.0;
        for (int k = 0; k < K; ++k) {
            double p = x_at(x, x_dtype, K, m, k) *
                       (double)orc_w_at(Q, scales, zeros, N, K, w_bit, group_size, k, n);
            acc += p;
            ab += fabs(p * s);
        }
        y_ref[i] = s * acc;
        abs_ref[i] = ab;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* MFMA tile layout: reference permutation from the layout spec        */
/* ------------------------------------------------------------------ */
/*
 * The layout is this project's own (the pages print no repack routine).
 * Columns are taken in strips of 16; K in blocks of KB = 128 (int4),
 * 256 (int2) or 64 (int8).  Each (strip s, K-block kb) is one contiguous
 * 1024-byte block, blocks ordered strip-major: b = s * (K / KB) + kb.
 * Inside a block, "lane" L in [0, 64) owns bytes [16 L, 16 L + 16); it
 * serves column n = 16 s + (L mod 16) and k-octet c = L / 16.
 *   int4: word j (0..3) of lane L holds k = 128 kb + 32 j + 8 c + i,
 *         i = 0..7, in nibble slot i/2 (i even) or 4 + i/2 (i odd).
 *   int2: word j of lane L holds k = 256 kb + 64 j + 32 h + 8 c + i,
 *         h = 0..1, i = 0..7, in 2-bit slot 4 h + i/2 (i even) or
 *         8 + 4 h + i/2 (i odd).
 *   int8: byte 8 h + i of lane L holds k = 64 kb + 32 h + 8 c + i.
 */
static int mfma_kb(int w_bit) { return w_bit == 4 ? 128 : (w_bit == 2 ? 256 : 64); }

size_t orc_mfma_bytes(int N, int K, int w_bit) {
    if (w_bit != 2 && w_bit != 4 && w_bit != 8) return 0;
    if (N < 0 || K < 0 || N % 16 || K % mfma_kb(w_bit)) return 0;
    return (size_t)N * K * w_bit / 8;
}

int orc_mfma_locate(int N, int K, int w_bit, int k, int n, size_t* where, int* shift) {
    if (orc_mfma_bytes(N, K, w_bit) == 0 && (N * (size_t)K) != 0) return -1;
    if (k < 0 || k >= K || n < 0 || n >= N) return -1;
    int KB = mfma_kb(w_bit);
    int s = n / 16, kb = k / KB, r = k % KB;
    size_t block = (size_t)s * (K / KB) + kb;
    int col = n % 16;
    if (w_bit == 4) {
        int j = r / 32, c = (r % 32) / 8, i = r % 8;
        int lane = 16 * c + col;
        int slot = (i % 2 == 0) ? i / 2 : 4 + i / 2;
        *where = block * 256 + (size_t)lane * 4 + j; /* int32 word index */
        *shift = 4 * slot;
    } else if (w_bit == 2) {
        int j = r / 64, h = (r % 64) / 32, c = (r % 32) / 8, i = r % 8;
        int lane = 16 * c + col;
        int slot = (i % 2 == 0) ? 4 * h + i / 2 : 8 + 4 * h + i / 2;
        *where = block * 256 + (size_t)lane * 4 + j;
        *shift = 2 * slot;
    } else {
        int h = r / 32, c = (r % 32) / 8, i = r % 8;
        int lane = 16 * c + col;
        *where = block * 1024 + (size_t)lane * 16 + 8 * h + i; /* byte index */
        *shift = 0;
    }
    return 0;
}

int orc_mfma_pack(const void* Q_canon, void* Q_mfma, int N, int K, int w_bit) {
    size_t bytes = orc_mfma_bytes(N, K, w_bit);
    if (bytes == 0 && (size_t)N * K != 0) return -1;
    memset(Q_mfma, 0, bytes);
    for (int k = 0; k < K; ++k) {
        for (int n = 0; n < N; ++n) {
            size_t where;
            int shift;
            orc_mfma_locate(N, K, w_bit, k, n, &where, &shift);
            if (w_bit == 8) {
                ((int8_t*)Q_mfma)[where] = ((const int8_t*)Q_canon)[(size_t)n * K + k];
            } else {
                uint32_t q = orc_q_at((const int32_t*)Q_canon, N, w_bit, k, n);
                ((uint32_t*)Q_mfma)[where] |= q << shift;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* int8 activations x ternary weights (liger-kernel, ops/experimental/  */
/* mm_int8int2.py: pack_weights / unpack_weights / matmul)             */
/* ------------------------------------------------------------------ */

/* The packed weight has ceil(K/4) rows of N bytes.  pack_weights splits K
 * into four consecutive quarters of R = K/4 rows (K % 4 == 0 here) and ORs
 * quarter i into bits 2i..2i+1, so element k of column n sits in row k mod R
 * at bit 2 * (k div R); unpack_weights masks that field and subtracts 1
 * (codes 0, 1, 2 are the values -1, 0, +1; code 3 reads as +2). */
int orc_t2_at(const uint8_t* Wp, int N, int K, int k, int n) {
    int R = K / 4;
    int code = (Wp[(size_t)(k % R) * N + n] >> (2 * (k / R))) & 3;
    return code - 1;
}

/* C (M, N) int32 = A (M, K) int8 times the ternary W (K, N): the sum of
 * integer products, exact (int64 accumulation, k ascending).  Returns -1 on
 * bad sizes, -2 if a sum leaves the int32 range (the page accumulates in
 * int32; no valid input with K < 2^23 gets there). */
static int i8t2_columns(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int n0,
                        int n1, int32_t* C) {
    /* each column's values decoded once (storage order only) */
    int8_t* wc = (int8_t*)malloc((size_t)(n1 - n0) * K + 1);
    if (!wc) return -1;
    for (int n = n0; n < n1; ++n)
        for (int k = 0; k < K; ++k) wc[(size_t)(n - n0) * K + k] = (int8_t)orc_t2_at(Wp, N, K, k, n);
    int rc = 0;
    for (int m = 0; m < M; ++m)
        for (int n = n0; n < n1; ++n) {
            const int8_t* w = wc + (size_t)(n - n0) * K;
            int64_t acc = 0;
            for (int k = 0; k < K; ++k) acc += (int64_t)A[(size_t)m * K + k] * w[k];
            if (acc > INT32_MAX || acc < INT32_MIN) rc = -2;
            C[(size_t)m * N + n] = (int32_t)acc;
        }
    free(wc);
    return rc;
}

int orc_i8t2_mm(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int32_t* C) {
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return -1;
    return i8t2_columns(A, Wp, M, N, K, 0, N, C);
}

/* The same for `count` chosen outputs (ms[i], ns[i]). */
int orc_i8t2_mm_at(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int count,
                   const int* ms, const int* ns, int32_t* C) {
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return -1;
    for (int i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
        int64_t acc = 0;
        for (int k = 0; k < K; ++k)
            acc += (int64_t)A[(size_t)ms[i] * K + k] * orc_t2_at(Wp, N, K, k, ns[i]);
        C[i] = (int32_t)acc;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Threaded driver: the products above over column slices on several   */
/* host threads.  Each output is computed by the same column function   */
/* with the same arithmetic as the single-threaded call, so the results */
/* are bit-identical; only the work is divided (64-column chunks dealt  */
/* round-robin to the threads).                                          */
/* ------------------------------------------------------------------ */
enum { ORC_CHUNK = 64 };

struct orc_job {
    int ternary;
    const double* xd;                 /* low-bit / int8: x decoded to double */
    const int8_t* A;                  /* ternary: int8 activations */
    const void* Q;
    const void* scales;
    const int32_t* zeros;
    int M, N, K, w_bit, group_size;
    double* y_ref;
    double* abs_ref;
    int32_t* C;
    int tid, threads, rc;
};

static void* orc_worker(void* arg) {
    struct orc_job* j = (struct orc_job*)arg;
    int chunks = (j->N + ORC_CHUNK - 1) / ORC_CHUNK;
    for (int c = j->tid; c < chunks; c += j->threads) {
        int n0 = c * ORC_CHUNK, n1 = n0 + ORC_CHUNK < j->N ? n0 + ORC_CHUNK : j->N;
        int rc = j->ternary
                     ? i8t2_columns(j->A, (const uint8_t*)j->Q, j->M, j->N, j->K, n0, n1, j->C)
                     : qmm_columns(j->xd, j->Q, j->scales, j->zeros, j->M, j->N, j->K, j->w_bit,
                                   j->group_size, n0, n1, j->y_ref, j->abs_ref);
        if (rc == -1 || (rc != 0 && j->rc == 0)) j->rc = rc;
    }
    return NULL;
}

/* Runs `threads` workers on copies of *proto; the first failure wins
 * (-1 allocation, -2 int32 range). */
static int orc_run(const struct orc_job* proto, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    struct orc_job jobs[256];
    pthread_t tids[256];
    int started = 0, rc = 0;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].threads = threads;
        jobs[t].rc = 0;
    }
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tids[t], NULL, orc_worker, &jobs[t]) != 0) break;
        started = t;
    }
    /* chunks of workers that could not be started are done here */
    for (int t = started + 1; t < threads; ++t) {
        jobs[t].threads = threads;
        orc_worker(&jobs[t]);
    }
    orc_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    for (int t = 0; t < threads; ++t)
        if (jobs[t].rc == -1 || (jobs[t].rc != 0 && rc == 0)) rc = jobs[t].rc;
    return rc;
}

int orc_qmm_mt(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
               const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
               double* y_ref, double* abs_ref, int threads) {
    if (M < 0 || (x_dtype != 0 && x_dtype != 1)) return -1;
    if (check_args(N, K, w_bit, group_size, zeros)) return -1;
    double* xd = decode_x(x, x_dtype, M, K);
    if (!xd) return -1;
    struct orc_job j;
    memset(&j, 0, sizeof j);
    j.xd = xd;
    j.Q = Q;
    j.scales = scales;
    j.zeros = zeros;
    j.M = M;
    j.N = N;
    j.K = K;
    j.w_bit = w_bit;
    j.group_size = group_size;
    j.y_ref = y_ref;
    j.abs_ref = abs_ref;
    int rc = orc_run(&j, threads);
    free(xd);
    return rc;
}

int orc_i8t2_mm_mt(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int32_t* C,
                   int threads) {
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return -1;
    struct orc_job j;
    memset(&j, 0, sizeof j);
    j.ternary = 1;
    j.A = A;
    j.Q = Wp;
    j.M = M;
    j.N = N;
    j.K = K;
    j.C = C;
    return orc_run(&j, threads);
}

/* Reference permutation of the ternary weight into this library's tile
 * layout (the HIP path's qmm_t2_pack), written from its specification:
 *   1 KiB blocks, one per (16-column strip s, 256-deep K block kb), strip-
 *   major; bytes [16 L, 16 L + 16) of a block belong to lane L: column
 *   16 s + L % 16, lane group g = L / 16; dword j (0..3) of the lane holds
 *   the 16 codes of k = 256 kb + 64 j + 16 g + e, e = 0..15, code e at bit
 *   2 * (4 * (e % 4) + e / 4).  Codes are stored as the page stores them. */
size_t orc_t2_tile_bytes(int N, int K) {
    if (N < 0 || K < 0 || N % 16 || K % 256) return 0;
    return (size_t)N * K / 4;
}

int orc_t2_tile_locate(int N, int K, int k, int n, size_t* byte, int* shift) {
    if (orc_t2_tile_bytes(N, K) == 0 && (size_t)N * K != 0) return -1;
    if (k < 0 || k >= K || n < 0 || n >= N) return -1;
    int s = n / 16, kb = k / 256, r = k % 256;
    int j = r / 64, g = (r % 64) / 16, e = r % 16;
    int lane = 16 * g + n % 16;
    int bit = 2 * (4 * (e % 4) + e / 4);
    *byte = ((size_t)s * (K / 256) + kb) * 1024 + (size_t)lane * 16 + 4 * j + bit / 8;
    *shift = bit % 8;
    return 0;
}

int orc_t2_tile_pack(const uint8_t* Wp, uint8_t* Wt, int N, int K) {
    size_t bytes = orc_t2_tile_bytes(N, K);
    if (bytes == 0 && (size_t)N * K != 0) return -1;
    memset(Wt, 0, bytes);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            size_t byte;
            int shift;
            orc_t2_tile_locate(N, K, k, n, &byte, &shift);
            Wt[byte] |= (uint8_t)((orc_t2_at(Wp, N, K, k, n) + 1) << shift);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Round-to-nearest quantizer (the step before the path: fp weights ->  */
/* qw, scales, qzeros in the operand contract of BitDistiller's         */
/* quant_matmul_kernel; the page gives only those shapes)               */
/* ------------------------------------------------------------------ */

/* fp32 -> fp16 bit pattern, round to nearest even, from the binary16
 * definition: normals 2^(e-15) (1 + m/1024), e in 1..30; subnormals
 * 2^-14 (m/1024); magnitudes that round past 65504 become infinity. */
uint16_t orc_f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = fr * 2^e, fr in [0.5, 1) */
    int ue = e - 1;               /* a in [2^ue, 2^(ue+1)) */
    if (ue < -14) ue = -14;       /* subnormal range: spacing 2^-24 */
    double ulp = ldexp(1.0, ue - 10);
    double n = rint(a / ulp);     /* exact quotient (power-of-two divisor), ties to even */
    double v = n * ulp;           /* the rounded magnitude */
    if (v >= 65536.0) return (uint16_t)(sign | 0x7C00u);  /* rounds past the largest finite */
    if (v < ldexp(1.0, -14))      /* subnormal (or rounded up to the smallest normal below) */
        return (uint16_t)(sign | (uint16_t)rint(v / ldexp(1.0, -24)));
    int ve;
    double vf = frexp(v, &ve);    /* v = vf * 2^ve, vf in [0.5, 1) */
    int exp16 = ve - 1 + 15;
    uint16_t mant = (uint16_t)rint((vf * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)(exp16 << 10) | mant);
}

/* Quantize W (K, N) fp32, group by group along k, column by column, with
 * min = min(0, min w) and max = max(0, max w) (the range holds 0, so zero is
 * exactly representable and a constant group keeps its value to half a
 * step):
 *   asymmetric: s = (max - min) / (2^b - 1), z = clamp(rint(-min / s), 0, 2^b - 1)
 *   symmetric:  s = max(|max|, |min|) / (2^(b-1) - 1), z = 2^(b-1)
 *   q = clamp(rint(w / s) + z, 0, 2^b - 1)
 * with s stored as fp16 (round to nearest even; if that is 0 -- an all-zero
 * group -- s = 1) and the codes computed from the stored scale, every step
 * in fp32 (division correctly rounded, rint ties to even).
 * group_size -1: one group spanning K.  Outputs in the canonical layout:
 * qw (K/pack, N), scales (G, N), qzeros (ceil(G/pack), N) (not written when
 * symmetric). */
int orc_rtn_quantize(const float* W, int N, int K, int w_bit, int group_size, int symmetric,
                     int32_t* qw, uint16_t* scales, int32_t* qzeros) {
    if (check_lowbit(N, K, w_bit, group_size)) return -1;
    int gs = group_size == -1 ? K : group_size;
    int G = gs ? K / gs : 0, pack = 32 / w_bit;
    float qmax = (float)((1 << w_bit) - 1);
    memset(qw, 0, (size_t)(K / pack) * N * sizeof(int32_t));
    if (!symmetric) memset(qzeros, 0, (size_t)((G + pack - 1) / pack) * N * sizeof(int32_t));
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            float mn = 0.0f, mx = 0.0f;
            for (int i = 0; i < gs; ++i) {
                float v = W[((size_t)g * gs + i) * N + n];
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float s32;
            if (symmetric) {
                float amax = fabsf(mx) > fabsf(mn) ? fabsf(mx) : fabsf(mn);
                s32 = amax / (float)((1 << (w_bit - 1)) - 1);
            } else {
                s32 = (mx - mn) / qmax;
            }
            uint16_t sb = orc_f32_to_f16(s32);
            if ((sb & 0x7FFFu) == 0) sb = 0x3C00u; /* 1.0 */
            scales[(size_t)g * N + n] = sb;
            float s = orc_f16_to_f32(sb);
            float z;
            if (symmetric) {
                z = (float)(1 << (w_bit - 1));
            } else {
                z = rintf(-mn / s);
                z = z < 0.0f ? 0.0f : (z > qmax ? qmax : z);
                qzeros[(size_t)(g / pack) * N + n] |= (int32_t)((uint32_t)z << ((g % pack) * w_bit));
            }
            for (int i = 0; i < gs; ++i) {
                int k = g * gs + i;
                float q = rintf(W[(size_t)k * N + n] / s) + z;
                q = q < 0.0f ? 0.0f : (q > qmax ? qmax : q);
                qw[(size_t)(k / pack) * N + n] |= (int32_t)((uint32_t)q << ((k % pack) * w_bit));
            }
        }
    }
    return 0;
}
