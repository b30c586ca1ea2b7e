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
// Two kernels.  rtn_scales_kernel: a workgroup owns one zero-word row (the
// `pack` groups that share a zero word) for 64 columns; wave w takes the
// range of group pack * row + w, one column per lane, so every load of a
// wave is one contiguous 64-column row segment; it stores the fp16 scale,
// and the waves' zero fields meet in LDS, where wave 0 assembles each zero
// word (one writer per word).  rtn_codes_kernel: one lane per packed word
// (pack consecutive k of one column) -- far more lanes in flight than one
// per group -- reading the scale and zero just stored.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// The input type is a template parameter: with a run-time switch inside the
// load, every load sat in its own branch and waited for itself.
template <int WDT> __device__ __forceinline__ float load_w(const void* W, size_t i) {
  if constexpr (WDT == YF32) return reinterpret_cast<const float*>(W)[i];
  if constexpr (WDT == XF16) return (float)reinterpret_cast<const _Float16*>(W)[i];
  if constexpr (WDT == XBF16) return (float)reinterpret_cast<const __bf16*>(W)[i];
}

template <int W_BIT, int WDT>
__global__ __launch_bounds__(64 * (32 / W_BIT)) void rtn_scales_kernel(
    const void* __restrict__ W, uint16_t* __restrict__ sc, uint32_t* __restrict__ qz, int N,
    int K, int gs, int symmetric) {
  constexpr int PACK = 32 / W_BIT;
  constexpr float QMAX = (float)((1 << W_BIT) - 1);
  __shared__ uint32_t zfield[PACK][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cblocks = (int)(((unsigned)N + 63u) / 64u);
  const int zr = (int)(blockIdx.x / cblocks);
  const int n = (int)(blockIdx.x % cblocks) * 64 + lane;
  const int g = zr * PACK + wv;

  uint32_t zbits = 0;
  if (g < K / gs && n < N) {
    float mn = 0.0f, mx = 0.0f;
#pragma unroll 32
    for (int i = 0; i < gs; ++i) {
      const float v = load_w<WDT>(W, (size_t)(g * gs + i) * N + n);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    const float s32 = symmetric
                          ? __fdiv_rn(fmaxf(fabsf(mx), fabsf(mn)), (float)((1 << (W_BIT - 1)) - 1))
                          : __fdiv_rn(mx - mn, QMAX);
    uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)s32);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // 1.0
    sc[(size_t)g * N + n] = sb;
    if (!symmetric) {
      const float s = (float)__builtin_bit_cast(_Float16, sb);
      const float z = __builtin_amdgcn_fmed3f(__builtin_rintf(__fdiv_rn(-mn, s)), 0.0f, QMAX);
      zbits = (uint32_t)z << (wv * W_BIT);
    }
  }
  if (!symmetric) {  // uniform: every wave of the workgroup reaches the barrier
    zfield[wv][lane] = zbits;
    __syncthreads();
    if (wv == 0 && n < N) {
      uint32_t zw = 0;
#pragma unroll
      for (int p = 0; p < PACK; ++p) zw |= zfield[p][lane];
      qz[(size_t)zr * N + n] = zw;
    }
  }
}

// rint(w / s) with the division correctly rounded, as the definition has it,
// at the cost of a multiply in almost every case: f = w * fl(1/s) is within
// |w/s| 2^-22 of fl(w/s) (two roundings of 2^-24 each, and fl(w/s)'s own),
// so when f is farther than |f| 2^-20 from every half-integer, f and fl(w/s)
// lie strictly inside the same rounding interval and rint gives the same
// integer.  A word with any element that close (about 1 in 10^4 for random
// data, and every exact tie) is redone with the correctly rounded division.
template <int W_BIT, int WDT>
__global__ __launch_bounds__(256) void rtn_codes_kernel(const void* __restrict__ W,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint32_t* __restrict__ qz,
                                                        uint32_t* __restrict__ qw, int N, int K,
                                                        int gs, int symmetric) {
  constexpr int PACK = 32 / W_BIT;
  constexpr float QMAX = (float)((1 << W_BIT) - 1);
  // block = (word row kw, 256-column block); the division is the block's
  const unsigned cblocks = ((unsigned)N + 255u) / 256u;
  const int kw = (int)(blockIdx.x / cblocks);
  const int n = (int)(blockIdx.x % cblocks) * 256 + (int)threadIdx.x;
  if (n >= N) return;
  const int g = kw * PACK / gs;
  const float s = (float)__builtin_bit_cast(_Float16, sc[(size_t)g * N + n]);
  const float z = symmetric ? (float)(1 << (W_BIT - 1))
                            : (float)((qz[(size_t)(g / PACK) * N + n] >> ((g % PACK) * W_BIT)) &
                                      ((1u << W_BIT) - 1));
  const float r = __fdiv_rn(1.0f, s);
  float v[PACK], q[PACK];
  bool near = false;
#pragma unroll
  for (int p = 0; p < PACK; ++p) v[p] = load_w<WDT>(W, (size_t)(kw * PACK + p) * N + n);
#pragma unroll
  for (int p = 0; p < PACK; ++p) {
    const float f = v[p] * r;
    q[p] = __builtin_rintf(f);
    near |= fabsf(f - __builtin_floorf(f) - 0.5f) <= fabsf(f) * 0x1p-20f;
  }
  if (near) {
#pragma unroll
    for (int p = 0; p < PACK; ++p) q[p] = __builtin_rintf(__fdiv_rn(v[p], s));
  }
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < PACK; ++p)
    word |= (uint32_t)__builtin_amdgcn_fmed3f(q[p] + z, 0.0f, QMAX) << (p * W_BIT);
  qw[(size_t)kw * N + n] = word;
}

hipError_t launch_quantize(const void* W, int w_dtype, void* qw, void* scales, void* qzeros,
                           int N, int K, int w_bit, int group_size, int symmetric,
                           hipStream_t st) {
  const int pack = 32 / w_bit;
  const int G = K / group_size, ZR = (G + pack - 1) / pack;
  const size_t blocks1 = (size_t)ZR * (((size_t)N + 63) / 64);
  const size_t blocks2 = (size_t)(K / pack) * (((size_t)N + 255) / 256);
  if (blocks1 > 0x7FFFFFFFu || blocks2 > 0x7FFFFFFFu) return hipErrorInvalidValue;
  auto* q = reinterpret_cast<uint32_t*>(qw);
  auto* s = reinterpret_cast<uint16_t*>(scales);
  auto* z = reinterpret_cast<uint32_t*>(qzeros);
  auto go = [&](auto bits, auto wdt) {
    constexpr int B = decltype(bits)::value, D = decltype(wdt)::value;
    const hipError_t e = launch_kernel(rtn_scales_kernel<B, D>, dim3((unsigned)blocks1),
                                       dim3(64 * (32 / B)), st, W, s, z, N, K, group_size,
                                       symmetric);
    if (e != hipSuccess) return e;
    return launch_kernel(rtn_codes_kernel<B, D>, dim3((unsigned)blocks2), dim3(256), st, W, s, z,
                         q, N, K, group_size, symmetric);
  };
  auto by_dtype = [&](auto bits) {
    if (w_dtype == YF32) return go(bits, std::integral_constant<int, YF32>{});
    if (w_dtype == XF16) return go(bits, std::integral_constant<int, XF16>{});
    return go(bits, std::integral_constant<int, XBF16>{});
  };
  if (w_bit == 4) return by_dtype(std::integral_constant<int, 4>{});
  return by_dtype(std::integral_constant<int, 2>{});
}

}  // namespace qmm
