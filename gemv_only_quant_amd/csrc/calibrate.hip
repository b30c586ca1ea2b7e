// calibrate.hip -- measurement-only kernel of the stamp build
// (libqmm_phases.so, gemv_only_quant_amd/build.py --phases; never part of the
// product library): the rate the matrix cores sustain on this chip with
// register-resident operands (bf16 and int8), the ceilings the prefill
// kernels are read against (bench.py --phases).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// One MFMA of the loop: bf16 16x16x32 (fp32 sums) or int8 16x16x64 (int32
// sums), both 16 cycles per instruction at the matrix cores' rated rate.
template <bool I8> struct LoopMfma;
template <> struct LoopMfma<false> {
  typedef f32x4_t acc_t;
  static __device__ __forceinline__ void run(acc_t& c, const u32x4_t& a, const u32x4_t& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ float value(const acc_t& c) { return c[0] + c[1] + c[2] + c[3]; }
};
template <> struct LoopMfma<true> {
  typedef i32x4_t acc_t;
  static __device__ __forceinline__ void run(acc_t& c, const u32x4_t& a, const u32x4_t& b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ float value(const acc_t& c) {
    return (float)(c[0] + c[1] + c[2] + c[3]);
  }
};

// Every wave runs `iters` rounds of 8 independent MFMAs (8 accumulators, so
// no MFMA waits on the previous one's result) on operands loaded once from
// `seed` (128 16-byte rows: A then B per lane).
template <bool I8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(const u32x4_t* __restrict__ seed,
                                                        float* __restrict__ out, int iters) {
  using L = LoopMfma<I8>;
  const int lane = threadIdx.x & 63;
  const u32x4_t a = seed[lane], b = seed[64 + lane];
  typename L::acc_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = typename L::acc_t{0, 0, 0, 0};
  // accumulators pinned to the matrix-core registers (the builtin lets the
  // allocator move them between register files every round)
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) L::run(c[j], a, b);
  }
  // the last MFMAs' results are read below: give them their latency
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(c[j]));
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += L::value(c[j]);
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Read-only probes with the headline GEMV's grid (one 256-thread workgroup
// per 16-column strip, each wave loading 8 consecutive 1 KiB blocks of its
// strip at once), adding the GEMV's steps one at a time, to see which of
// them costs time once graph-replayed: bit 0 the x slice (8 KiB per
// workgroup, to LDS, two barriers); bit 1 the per-block work after each
// load (the GEMV's recipe: per 32-bit word one shift, four mask-ors under
// the fp16 1024 pattern, four v_dot2c_f32_f16 against x from LDS); bit 2
// the GEMV's closing step (every lane's partial to LDS, a barrier, 16
// threads adding 16 values each).  The weight loads carry the GEMV's
// non-temporal hint.  Without bit 2 every thread stores one
// word.  Reads src[0 .. gridDim.x * 32 KiB), x[0 .. 8 KiB); writes dst[0 ..
// gridDim.x * 256) words.
template <int V>
__global__ __launch_bounds__(256) void readonly_probe_kernel(const u32x4_t* __restrict__ src,
                                                             const u32x4_t* __restrict__ x,
                                                             uint32_t* __restrict__ dst) {
  constexpr bool XS = V & 1, DOT = V & 2, EPI = V & 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const buf_t b = make_buf(src + (size_t)blockIdx.x * 2048, 32u * 1024u);
  __shared__ u32x4_t xs[XS ? 768 : 1];
  __shared__ float red[4][4][16];
  u32x4_t xr[2];
  if constexpr (XS) {
    const buf_t xb = make_buf(x, 8192u);
#pragma unroll
    for (int j = 0; j < 2; ++j) xr[j] = buf_load128(xb, (threadIdx.x + 256 * j) * 16);
  }
  u32x4_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = buf_load128_stream(b, ((wave * 8 + i) * 64 + lane) * 16);
  if constexpr (XS) {
    xs[threadIdx.x] = xr[0];
    xs[threadIdx.x + 256] = xr[1];
    __syncthreads();
    xs[512 + threadIdx.x] = xs[(threadIdx.x * 3) & 511];
    __syncthreads();
  }
  uint32_t acc = 0;
  if constexpr (DOT) {
    float f = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t xv = XS ? xs[(threadIdx.x + i) & 511] : u32x4_t{0x3C003C00u, 0x3C003C00u,
                                                                    0x3C003C00u, 0x3C003C00u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = v[i][j], w8 = w >> 8;
        const uint32_t p[4] = {(w & 0x000F000Fu) | 0x64006400u, (w & 0x00F000F0u) | 0x64006400u,
                               (w8 & 0x000F000Fu) | 0x64006400u, (w8 & 0x00F000F0u) | 0x64006400u};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          f = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, xv[t]),
                                     __builtin_bit_cast(half2_t, p[t]), f, false);
      }
    }
    acc = __builtin_bit_cast(uint32_t, f);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if constexpr (XS) acc += xs[(threadIdx.x + 7) & 511][0];
  }
  if constexpr (EPI) {
    red[wave][lane >> 4][lane & 15] = __builtin_bit_cast(float, acc);
    __syncthreads();
    if (threadIdx.x < 16) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int o = 0; o < 4; ++o) sum += red[w][o][threadIdx.x];
      dst[(size_t)blockIdx.x * 256 + threadIdx.x] = __builtin_bit_cast(uint32_t, sum);
    }
  } else {
    dst[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
  }
}

}  // namespace qmm

// variant 0-7 (the bits above); strips workgroups; src strips x 32 KiB, x
// 8 KiB, dst strips x 256 words.
extern "C" __attribute__((visibility("default"))) int qmm_calib_readonly(int variant,
                                                                         const void* src,
                                                                         const void* x, void* dst,
                                                                         int strips,
                                                                         void* stream) {
  if (strips <= 0 || strips > 65536) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 g((unsigned)strips), blk(256);
  auto s = static_cast<const qmm::u32x4_t*>(src);
  auto xv = static_cast<const qmm::u32x4_t*>(x);
  auto d = static_cast<uint32_t*>(dst);
  switch (variant) {
    case 0: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<0>, g, blk, st, s, xv, d);
    case 1: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<1>, g, blk, st, s, xv, d);
    case 2: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<2>, g, blk, st, s, xv, d);
    case 3: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<3>, g, blk, st, s, xv, d);
    case 4: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<4>, g, blk, st, s, xv, d);
    case 5: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<5>, g, blk, st, s, xv, d);
    case 6: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<6>, g, blk, st, s, xv, d);
    case 7: return (int)qmm::launch_kernel(qmm::readonly_probe_kernel<7>, g, blk, st, s, xv, d);
  }
  return -1;
}

// blocks workgroups of 4 waves; `seed` holds 128 x 16 bytes, `out` blocks x
// 256 floats.  int8 != 0 runs v_mfma_i32_16x16x64_i8, else
// v_mfma_f32_16x16x32_bf16.
extern "C" __attribute__((visibility("default"))) int qmm_calib_mfma(const void* seed, void* out,
                                                                     int blocks, int iters,
                                                                     int int8, void* stream) {
  if (blocks <= 0 || iters <= 0) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (int8 != 0)
    return (int)qmm::launch_kernel(qmm::mfma_loop_kernel<true>, dim3((unsigned)blocks),
                                   dim3(256), st, seed, out, iters);
  return (int)qmm::launch_kernel(qmm::mfma_loop_kernel<false>, dim3((unsigned)blocks), dim3(256),
                                 st, seed, out, iters);
}
