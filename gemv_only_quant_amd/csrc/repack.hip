// repack.hip -- canonical packed weights <-> MFMA tile layout, and the
// bit-exact fp32 dequant export used by the tests.
//
// Tile layout (the pages print no repack routine; Marlin only shows that its
// B operand arrives pre-permuted so that each thread's 16-byte load feeds its
// own MMA fragments -- this is the gfx950 counterpart of that idea):
//   1 KiB block per (16-column strip s, K-block kb), KB = 128 / 256 / 64 for
//   int4 / int2 / int8, blocks strip-major.  "Lane" L of a block owns bytes
//   [16 L, 16 L + 16): column 16 s + L % 16, k-octet c = L / 16.  That is the
//   B-operand lane map of v_mfma_f32_16x16x32_{f16,bf16} (lane L holds
//   k = 8 (L / 16) .. + 7 of column L % 16 for one 32-deep k step), so one
//   128-bit load per lane feeds 4 (int4), 8 (int2) or 2 (int8) MFMA steps.
//   Inside an int4 word the codes of k-octet positions i = 0..7 sit in
//   nibbles [0,2,4,6 | 1,3,5,7] order, so (w >> 4 t) & 0x000F000F is the
//   pair (i = 2t, i = 2t + 1) -- exactly one MFMA operand register.  int2
//   words hold two k steps (h = 0, 1) the same way in 2-bit fields.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "../../include/qmm.h"

namespace qmm {

int mfma_kblock(int w_bit) { return w_bit == 4 ? 128 : (w_bit == 2 ? 256 : 64); }

// Code slot of octet position i (0..7) in a word: int4 nibble index.
__device__ __forceinline__ int slot4(int i) { return (i & 1) ? 4 + (i >> 1) : (i >> 1); }
// int2: 2-bit field index for k step h and octet position i.
__device__ __forceinline__ int slot2(int h, int i) { return (i & 1) ? 8 + 4 * h + (i >> 1) : 4 * h + (i >> 1); }

// --- int4 ------------------------------------------------------------------
// One thread per layout word: block b, lane L, word j.  The eight codes come
// from canonical word [16 kb + 4 j + c][n] (k = 128 kb + 32 j + 8 c + i).
__global__ void pack4_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                             int N, int K) {
  const size_t total = (size_t)N * K / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int kblocks = K / 128;
  const size_t b = idx / 256;
  const int L = (int)(idx % 256) / 4, j = (int)(idx % 4);
  const int s = (int)(b / kblocks), kb = (int)(b % kblocks);
  const int n = 16 * s + (L & 15), c = L >> 4;
  const uint32_t wsrc = src[(size_t)(16 * kb + 4 * j + c) * N + n];
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out |= ((wsrc >> (4 * i)) & 0xFu) << (4 * slot4(i));
  dst[idx] = out;
}

__global__ void unpack4_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                               int N, int K) {
  const size_t total = (size_t)N * K / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // canonical word
  if (idx >= total) return;
  const int r = (int)(idx / N), n = (int)(idx % N);
  const int kb = r / 16, j = (r % 16) / 4, c = r % 4;
  const int s = n / 16, L = 16 * c + (n & 15);
  const size_t b = (size_t)s * (K / 128) + kb;
  const uint32_t w = src[b * 256 + 4 * L + j];
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out |= ((w >> (4 * slot4(i))) & 0xFu) << (4 * i);
  dst[idx] = out;
}

// --- int2 ------------------------------------------------------------------
// Layout word (b, L, j) holds k = 256 kb + 64 j + 32 h + 8 c + i; canonical
// word of that k is [16 kb + 4 j + 2 h + c / 2], field 8 (c % 2) + i.
__global__ void pack2_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                             int N, int K) {
  const size_t total = (size_t)N * K / 16;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int kblocks = K / 256;
  const size_t b = idx / 256;
  const int L = (int)(idx % 256) / 4, j = (int)(idx % 4);
  const int s = (int)(b / kblocks), kb = (int)(b % kblocks);
  const int n = 16 * s + (L & 15), c = L >> 4;
  uint32_t out = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t wsrc = src[(size_t)(16 * kb + 4 * j + 2 * h + c / 2) * N + n];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out |= ((wsrc >> (2 * (8 * (c & 1) + i))) & 3u) << (2 * slot2(h, i));
  }
  dst[idx] = out;
}

__global__ void unpack2_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                               int N, int K) {
  const size_t total = (size_t)N * K / 16;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // canonical word
  if (idx >= total) return;
  const int r = (int)(idx / N), n = (int)(idx % N);
  // canonical word r holds k = 16 r + t, t = 0..15
  const int kb = r / 16, j = (r % 16) / 4, h = (r % 4) / 2, chalf = r % 2;
  const int s = n / 16;
  const size_t b = (size_t)s * (K / 256) + kb;
  uint32_t out = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int c = 2 * chalf + t / 8, i = t % 8;
    const int L = 16 * c + (n & 15);
    const uint32_t w = src[b * 256 + 4 * L + j];
    out |= ((w >> (2 * slot2(h, i))) & 3u) << (2 * t);
  }
  dst[idx] = out;
}

// --- int8 ------------------------------------------------------------------
// Layout lane (b, L): bytes 8 h + i = Q[n][64 kb + 32 h + 8 c + i].
__global__ void pack8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int N,
                             int K) {
  const size_t total = (size_t)N * K / 16;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte lane slot
  if (idx >= total) return;
  const int kblocks = K / 64;
  const size_t b = idx / 64;
  const int L = (int)(idx % 64);
  const int s = (int)(b / kblocks), kb = (int)(b % kblocks);
  const int n = 16 * s + (L & 15), c = L >> 4;
  const uint8_t* row = src + (size_t)n * K + 64 * kb + 8 * c;
  const uint2 lo = *reinterpret_cast<const uint2*>(row);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + 32);
  *reinterpret_cast<u32x4_t*>(dst + idx * 16) = u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

__global__ void unpack8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int N,
                               int K) {
  const size_t total = (size_t)N * K / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-byte canonical run
  if (idx >= total) return;
  const int n = (int)(idx / (K / 8)), k = (int)(idx % (K / 8)) * 8;
  const int kb = k / 64, h = (k % 64) / 32, c = (k % 32) / 8;
  const int s = n / 16, L = 16 * c + (n & 15);
  const size_t b = (size_t)s * (K / 64) + kb;
  *reinterpret_cast<uint2*>(dst + (size_t)n * K + k) =
      *reinterpret_cast<const uint2*>(src + b * 1024 + 16 * L + 8 * h);
}

static unsigned blocks_for(size_t n, int t) { return (unsigned)((n + t - 1) / t); }

hipError_t launch_pack(const void* q_canon, void* q_mfma, int N, int K, int w_bit,
                       hipStream_t st) {
  const int T = 256;
  if (w_bit == 4)
    return launch_kernel(pack4_kernel, dim3(blocks_for((size_t)N * K / 8, T)), dim3(T), st, q_canon,
                         q_mfma, N, K);
  if (w_bit == 2)
    return launch_kernel(pack2_kernel, dim3(blocks_for((size_t)N * K / 16, T)), dim3(T), st, q_canon,
                         q_mfma, N, K);
  return launch_kernel(pack8_kernel, dim3(blocks_for((size_t)N * K / 16, T)), dim3(T), st, q_canon,
                       q_mfma, N, K);
}

hipError_t launch_unpack_layout(const void* q_mfma, void* q_canon, int N, int K, int w_bit,
                                hipStream_t st) {
  const int T = 256;
  if (w_bit == 4)
    return launch_kernel(unpack4_kernel, dim3(blocks_for((size_t)N * K / 8, T)), dim3(T), st, q_mfma,
                         q_canon, N, K);
  if (w_bit == 2)
    return launch_kernel(unpack2_kernel, dim3(blocks_for((size_t)N * K / 16, T)), dim3(T), st, q_mfma,
                         q_canon, N, K);
  return launch_kernel(unpack8_kernel, dim3(blocks_for((size_t)N * K / 8, T)), dim3(T), st, q_mfma,
                       q_canon, N, K);
}

// --- dequant export ----------------------------------------------------------
// One thread per output W[k][n]: locate the code in the given layout, then
// W = float(q - z) * float(s) (exact: at most 4 + 11 significant bits), or
// float(q) for int8.
__device__ __forceinline__ uint32_t code_at(const void* Q, int layout, int N, int K, int w_bit,
                                            int k, int n) {
  if (w_bit == 8) {
    const int8_t* q8 = (const int8_t*)Q;
    if (layout == QMM_LAYOUT_CANON) return (uint32_t)(int32_t)q8[(size_t)n * K + k];
    const int kb = k / 64, r = k % 64, h = r / 32, c = (r % 32) / 8, i = r % 8;
    const size_t b = (size_t)(n / 16) * (K / 64) + kb;
    return (uint32_t)(int32_t)q8[b * 1024 + 16 * (16 * c + (n & 15)) + 8 * h + i];
  }
  const uint32_t* qw = (const uint32_t*)Q;
  const uint32_t mask = (1u << w_bit) - 1u;
  if (layout == QMM_LAYOUT_CANON) {
    const int pack = 32 / w_bit;
    return (qw[(size_t)(k / pack) * N + n] >> ((k % pack) * w_bit)) & mask;
  }
  const int KB = w_bit == 4 ? 128 : 256;
  const int kb = k / KB, r = k % KB;
  const size_t b = (size_t)(n / 16) * (K / KB) + kb;
  int j, c, i, field;
  if (w_bit == 4) {
    j = r / 32; c = (r % 32) / 8; i = r % 8; field = slot4(i);
  } else {
    j = r / 64; const int h = (r % 64) / 32; c = (r % 32) / 8; i = r % 8; field = slot2(h, i);
  }
  const int L = 16 * c + (n & 15);
  return (qw[b * 256 + 4 * L + j] >> (w_bit * field)) & mask;
}

__global__ void dequant_kernel(const void* __restrict__ Q, int layout,
                               const uint16_t* __restrict__ scales,
                               const uint32_t* __restrict__ zeros, float* __restrict__ w,
                               int N, int K, int w_bit, int group_size) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)N * K) return;
  const int k = (int)(idx / N), n = (int)(idx % N);
  const uint32_t q = code_at(Q, layout, N, K, w_bit, k, n);
  if (w_bit == 8) {
    w[idx] = (float)(int32_t)q;
    return;
  }
  const int g = k / group_size, pack = 32 / w_bit;
  const uint32_t z = zeros ? (zeros[(size_t)(g / pack) * N + n] >> ((g % pack) * w_bit)) &
                                 ((1u << w_bit) - 1u)
                           : (1u << (w_bit - 1));
  const float s = f16_bits_to_f32(scales[(size_t)g * N + n]);
  w[idx] = (float)((int)q - (int)z) * s;
}

hipError_t launch_dequant(const void* Q, int layout, const void* scales, const void* zeros,
                          float* w, int N, int K, int w_bit, int group_size, hipStream_t st) {
  const int T = 256;
  return launch_kernel(dequant_kernel, dim3(blocks_for((size_t)N * K, T)), dim3(T), st, Q, layout,
                       scales, zeros, w, N, K, w_bit, group_size);
}

}  // namespace qmm
