/*
 * qmm_oracle.h -- CPU oracle for the weight-only quantized matmul
 *
 *     y[m][n] = sum_k x[m][k] * W[k][n],   W = dequant(Q)
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this library: only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Plain, slow C99.  Every decode is written from its definition; the matmul
 * accumulates in fp64 with k ascending.  Single-threaded, except that the
 * *_mt calls hand the same per-output work to several host threads.
 *
 * Operand conventions (all arrays contiguous, row-major):
 *   x       (M, K) 16-bit words, fp16 (x_dtype 0) or bf16 (x_dtype 1)
 *   w_bit 2|4: Q = qw (K/pack, N) int32, pack = 32/w_bit;
 *              scales (K/group_size, N) fp16 bit patterns;
 *              zeros  NULL (symmetric, z = 2^(w_bit-1)) or
 *                     (ceil(G/pack), N) int32 packed along the group axis;
 *              group_size -1: per column, one group spanning K (G = 1)
 *   w_bit 8:   Q (N, K) int8; scales (N,) fp32; zeros NULL; group_size 0
 * and, for the int8 x ternary product (orc_i8t2_*), A (M, K) int8 and the
 * packed ternary weight (K/4, N) uint8.
 * Return codes: 0 ok, -1 bad argument.
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t h);
void orc_f16_to_f32_n(const uint16_t* h, float* out, size_t n);
void orc_bf16_to_f32_n(const uint16_t* h, float* out, size_t n);

/* Integer code of element (k, n) of a canonical low-bit weight. */
uint32_t orc_q_at(const int32_t* qw, int N, int w_bit, int k, int n);
/* Zero point of group g, column n (symmetric when qz == NULL). */
uint32_t orc_z_at(const int32_t* qz, int N, int w_bit, int g, int n);

/* Dequantized weight W[k][n] (fp32, exact).  int8: the raw code, scale not
 * applied (it is applied after the sum). */
float orc_w_at(const void* Q, const void* scales, const int32_t* zeros,
               int N, int K, int w_bit, int group_size, int k, int n);

/* Bulk unpack / dequant. */
int orc_unpack_q(const int32_t* qw, int N, int K, int w_bit, uint8_t* q_out /*(K,N)*/);
int orc_unpack_z(const int32_t* qz, int N, int G, int w_bit, uint8_t* z_out /*(G,N)*/);
int orc_dequant(const void* Q, const void* scales, const int32_t* zeros,
                int N, int K, int w_bit, int group_size, float* w_out /*(K,N)*/);

/* Full product: y_ref and abs_ref = sum_k |x * w_eff| (M, N) in fp64. */
int orc_qmm(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
            const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
            double* y_ref, double* abs_ref);

/* The same, for `count` chosen outputs (ms[i], ns[i]) only. */
int orc_qmm_at(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
               const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
               int count, const int* ms, const int* ns, double* y_ref, double* abs_ref);

/* The same two products over column slices on `threads` host threads:
 * identical per-output arithmetic, so bit-identical results.  orc_i8t2_mm_mt
 * returns -2 if a sum leaves the int32 range. */
int orc_qmm_mt(const uint16_t* x, int x_dtype, const void* Q, const void* scales,
               const int32_t* zeros, int M, int N, int K, int w_bit, int group_size,
               double* y_ref, double* abs_ref, int threads);

/* Reference permutation into the MFMA tile layout, written element by
 * element from the layout specification (see orc_mfma_locate). */
int orc_mfma_locate(int N, int K, int w_bit, int k, int n, size_t* byte_or_word, int* shift);
size_t orc_mfma_bytes(int N, int K, int w_bit);
int orc_mfma_pack(const void* Q_canon, void* Q_mfma, int N, int K, int w_bit);

/* int8 activations x ternary weights (liger-kernel mm_int8int2): packed
 * weight (K/4, N) uint8, element k at row k mod (K/4), bits 2 * (k div
 * (K/4)), value code - 1; C (M, N) int32 exact.  K % 4 == 0. */
int orc_t2_at(const uint8_t* Wp, int N, int K, int k, int n);
int orc_i8t2_mm(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int32_t* C);
int orc_i8t2_mm_at(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int count,
                   const int* ms, const int* ns, int32_t* C);
int orc_i8t2_mm_mt(const int8_t* A, const uint8_t* Wp, int M, int N, int K, int32_t* C,
                   int threads);
/* Reference permutation into the ternary tile layout (see the .c file). */
size_t orc_t2_tile_bytes(int N, int K);
int orc_t2_tile_locate(int N, int K, int k, int n, size_t* byte, int* shift);
int orc_t2_tile_pack(const uint8_t* Wp, uint8_t* Wt, int N, int K);

/* fp32 -> fp16 bits, round to nearest even (from the binary16 definition). */
uint16_t orc_f32_to_f16(float f);
/* Round-to-nearest quantizer into the canonical operands (see the .c file). */
int orc_rtn_quantize(const float* W /*(K,N)*/, int N, int K, int w_bit, int group_size,
                     int symmetric, int32_t* qw, uint16_t* scales, int32_t* qzeros);

#ifdef __cplusplus
}
#endif
#endif
