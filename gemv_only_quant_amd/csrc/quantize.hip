// quantize.hip -- round-to-nearest quantizer: fp weights W (K, N) into the
// operands the matmul reads (BitDistiller quant_matmul_kernel's shapes:
// qw (K/pack, N) int32, scales (G, N) fp16, qzeros (ceil(G/pack), N) int32).
//
// Per group of group_size consecutive k and per column n, with the range
// [min(0, min w), max(0, max w)] (zero stays exactly representable):
//   asymmetric: s = (max - min) / (2^b - 1), z = clamp(rint(-min / s), 0, 2^b - 1)
//   symmetric:  s = max(|max|, |min|) / (2^(b-1) - 1), z = 2^(b-1)
//   q = clamp(rint(w / s) + z, 0, 2^b - 1)
// s is stored as fp16 (round to nearest even; 1.0 if that is 0) and the
// codes come from the stored scale.  Every decision is taken in fp32 with
// correctly rounded division and ties-to-even rint, so the codes are a
// deterministic function of the inputs.
//
// One thread per (zero-word row, column): it walks the `pack` groups that
// share a zero word, so every output word has one writer; a wave's 64
// columns make every load and store a contiguous row segment.
#include <hip/hip_runtime.h>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int W_BIT>
__global__ __launch_bounds__(256) void rtn_quantize_kernel(const void* __restrict__ W, int w_dtype,
                                                           uint32_t* __restrict__ qw,
                                                           uint16_t* __restrict__ sc,
                                                           uint32_t* __restrict__ qz, int N, int K,
                                                           int gs, int symmetric) {
  constexpr int PACK = 32 / W_BIT;
  constexpr float QMAX = (float)((1 << W_BIT) - 1);
  const int G = K / gs;
  const int ZR = (G + PACK - 1) / PACK;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (size_t)ZR * N) return;
  const int zr = (int)(t / N), n = (int)(t % N);
  auto load = [&](int k) -> float {
    const size_t i = (size_t)k * N + n;
    if (w_dtype == YF32) return reinterpret_cast<const float*>(W)[i];
    if (w_dtype == XF16) return (float)reinterpret_cast<const _Float16*>(W)[i];
    return (float)reinterpret_cast<const __bf16*>(W)[i];
  };

  uint32_t zword = 0;
  const int g1 = min(G, zr * PACK + PACK);
  for (int g = zr * PACK; g < g1; ++g) {
    float mn = 0.0f, mx = 0.0f;
    for (int i = 0; i < gs; ++i) {
      const float v = load(g * gs + i);
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    float s32;
    if (symmetric) {
      const float amax = fabsf(mx) > fabsf(mn) ? fabsf(mx) : fabsf(mn);
      s32 = __fdiv_rn(amax, (float)((1 << (W_BIT - 1)) - 1));
    } else {
      s32 = __fdiv_rn(mx - mn, QMAX);
    }
    uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)s32);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // 1.0
    sc[(size_t)g * N + n] = sb;
    const float s = (float)__builtin_bit_cast(_Float16, sb);
    float z;
    if (symmetric) {
      z = (float)(1 << (W_BIT - 1));
    } else {
      z = __builtin_rintf(__fdiv_rn(-mn, s));
      z = z < 0.0f ? 0.0f : (z > QMAX ? QMAX : z);
      zword |= (uint32_t)z << ((g % PACK) * W_BIT);
    }
    for (int k0 = g * gs; k0 < (g + 1) * gs; k0 += PACK) {
      uint32_t word = 0;
#pragma unroll
      for (int p = 0; p < PACK; ++p) {
        float q = __builtin_rintf(__fdiv_rn(load(k0 + p), s)) + z;
        q = q < 0.0f ? 0.0f : (q > QMAX ? QMAX : q);
        word |= (uint32_t)q << (p * W_BIT);
      }
      qw[(size_t)(k0 / PACK) * N + n] = word;
    }
  }
  if (!symmetric) qz[(size_t)zr * N + n] = zword;
}

hipError_t launch_quantize(const void* W, int w_dtype, void* qw, void* scales, void* qzeros,
                           int N, int K, int w_bit, int group_size, int symmetric,
                           hipStream_t st) {
  const int pack = 32 / w_bit;
  const int G = K / group_size, ZR = (G + pack - 1) / pack;
  const size_t threads = (size_t)ZR * N;
  const dim3 grid((unsigned)((threads + 255) / 256));
  auto* q = reinterpret_cast<uint32_t*>(qw);
  auto* s = reinterpret_cast<uint16_t*>(scales);
  auto* z = reinterpret_cast<uint32_t*>(qzeros);
  if (w_bit == 4)
    hipLaunchKernelGGL(rtn_quantize_kernel<4>, grid, dim3(256), 0, st, W, w_dtype, q, s, z, N, K,
                       group_size, symmetric);
  else
    hipLaunchKernelGGL(rtn_quantize_kernel<2>, grid, dim3(256), 0, st, W, w_dtype, q, s, z, N, K,
                       group_size, symmetric);
  return hipGetLastError();
}

}  // namespace qmm
