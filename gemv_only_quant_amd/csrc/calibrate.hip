// calibrate.hip -- measurement-only kernel of the stamp build
// (libqmm_phases.so, gemv_only_quant_amd/build.py --phases; never part of the
// product library): the rate the matrix cores sustain on this chip with
// register-resident operands, the ceiling the prefill kernels are read
// against (bench.py --phases).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// Every wave runs `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16
// (8 accumulators, so no MFMA waits on the previous one's result) on
// operands loaded once from `seed` (128 16-byte rows: A then B per lane).
__global__ __launch_bounds__(256) void mfma_loop_kernel(const u32x4_t* __restrict__ seed,
                                                        float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const u32x4_t a = seed[lane], b = seed[64 + lane];
  f32x4_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // accumulators pinned to the matrix-core registers (the builtin lets the
  // allocator move them between register files every round)
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c[j]) : "v"(a), "v"(b));
  }
  // the last MFMAs' results are read below: give them their latency
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(c[j]));
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace qmm

// blocks workgroups of 4 waves; `seed` holds 128 x 16 bytes, `out` blocks x 256 floats.
extern "C" __attribute__((visibility("default"))) int qmm_calib_mfma(const void* seed, void* out,
                                                                     int blocks, int iters,
                                                                     void* stream) {
  if (blocks <= 0 || iters <= 0) return -1;
  return (int)qmm::launch_kernel(qmm::mfma_loop_kernel, dim3((unsigned)blocks), dim3(256),
                                 reinterpret_cast<hipStream_t>(stream), seed, out, iters);
}
