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

}  // namespace qmm

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
