// gemv_int8.hip -- decode / skinny GEMV for int8 weights Q (N, K) with a
// per-output-row fp32 scale (tiny-llm src/tinyllm/kernels/int8_gemv.py:
// y[m, n] = scale[n] * sum_k x[m, k] * q[n, k], the int8 -> 16-bit
// conversion exact because |q| <= 128, fp32 accumulation, scale last).
//
// Shape of the work: a wave owns RN consecutive output rows n and sweeps K
// in steps of 1024, each lane taking 16 contiguous bytes of every row (one
// 128-bit load per row and step).  The lane's x slice stays in registers as
// natural 16-bit pairs and is reused across its RN rows.  Codes become
// 16-bit pairs without a multiply:
//   fp16: u = q ^ 0x80 = q + 128 in [0, 255]; perm the bytes of u under the
//         fp16 exponent byte 0x64 -> (1024 + u) exactly;     bias C = 1152
//   bf16: u -> fp32 by v_cvt_f32_ubyte, pairs -> bf16 (exact, u <= 255);
//                                                           bias C = 128
// and the bias leaves once per lane: sum x (C + q) - C sum x.  The 64 lane
// partials of each (m, n) are folded with DPP (qmm_device.h wave_sum).
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int XDT> struct Int8Pairs;
template <> struct Int8Pairs<XF16> {
  static constexpr float bias = 1152.0f;
  // 4 codes (one dword) -> 2 pairs (k0,k1), (k2,k3)
  static __device__ __forceinline__ void cvt(uint32_t q, uint32_t* out) {
    const uint32_t u = q ^ 0x80808080u;
    out[0] = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    out[1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  }
};
template <> struct Int8Pairs<XBF16> {
  static constexpr float bias = 128.0f;
  static __device__ __forceinline__ void cvt(uint32_t q, uint32_t* out) {
    const uint32_t u = q ^ 0x80808080u;
    // byte-to-float conversions (the compiler selects v_cvt_f32_ubyte0..3)
    const float f0 = (float)(u & 0xFFu);
    const float f1 = (float)((u >> 8) & 0xFFu);
    const float f2 = (float)((u >> 16) & 0xFFu);
    const float f3 = (float)(u >> 24);
    bf16x2_t p0 = {(__bf16)f0, (__bf16)f1};
    bf16x2_t p1 = {(__bf16)f2, (__bf16)f3};
    out[0] = __builtin_bit_cast(uint32_t, p0);
    out[1] = __builtin_bit_cast(uint32_t, p1);
  }
};

template <int XDT, int MB, int RN>
__global__ __launch_bounds__(256) void gemv_int8_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ Q,
    const float* __restrict__ scale, void* __restrict__ y, int ydt, int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n0 = (blockIdx.x * 4 + wave) * RN;
  if (n0 >= N) return;
  float sc[RN];
#pragma unroll
  for (int r = 0; r < RN; ++r) sc[r] = 0.f;

  float acc[MB][RN];
  float xs[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    xs[m] = 0.f;
#pragma unroll
    for (int r = 0; r < RN; ++r) acc[m][r] = 0.f;
  }

  for (int kc = 0; kc < K; kc += 1024) {
    const int k = kc + lane * 16;
    const bool kok = k < K;  // K % 16 == 0
    u32x4_t q[RN];
#pragma unroll
    for (int r = 0; r < RN; ++r)
      q[r] = (kok && n0 + r < N)
                 ? __builtin_nontemporal_load(
                       reinterpret_cast<const u32x4_t*>(Q + (size_t)(n0 + r) * K + k))
                 : u32x4_t{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
    // the rows' scales, loaded behind the first weights (loads return in
    // order): their latency overlaps the weights' instead of following the
    // reduction, and no weight waits for them
    // (a vector load: a scalar one would be waited for with the kernel's
    // other scalar loads; rows past N read 0)
    if (kc == 0) {
      const buf_t sb = make_buf(scale, (uint32_t)N * 4u);
#pragma unroll
      for (int r = 0; r < RN; ++r) sc[r] = __builtin_bit_cast(float, buf_load32(sb, (n0 + r) * 4));
    }
    uint32_t wp[RN][8];
#pragma unroll
    for (int r = 0; r < RN; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) Int8Pairs<XDT>::cvt(q[r][v], &wp[r][2 * v]);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < M && kok) {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(x + (size_t)m * K + k);
        const u32x4_t x0 = xp[0], x1 = xp[1];
        const uint32_t xd[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xs[m] = dot2<XDT>(xd[j], Bias<XDT>::one_pair, xs[m]);
#pragma unroll
          for (int r = 0; r < RN; ++r) acc[m][r] = dot2<XDT>(xd[j], wp[r][j], acc[m][r]);
        }
      }
    }
  }

  float v[MB][RN];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < RN; ++r) v[m][r] = m < M ? wave_sum(acc[m][r] - Int8Pairs<XDT>::bias * xs[m]) : 0.f;
  if (lane == 0) {
    with_y(y, ydt, [&](auto* yt) {
      using T = typename std::remove_pointer<decltype(yt)>::type;
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < RN; ++r)
          if (m < M && n0 + r < N) yt[(size_t)m * N + n0 + r] = (T)(sc[r] * v[m][r]);
    });
  }
}

// ---------------------------------------------------------------- host side
static int m_bucket8(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

GemvInt8Plan plan_gemv_int8(int M, int N, int K) {
  GemvInt8Plan p{};
  p.mb = m_bucket8(M);
  // enough waves to cover the chip; more rows per wave once N is large
  int rn = (N >= 8192 && M <= 4) ? 4 : (N >= 4096 ? 2 : 1);
  static const int want = env_int("QMM_GEMV8_RN");
  if (want == 1 || want == 2 || want == 4) rn = want;
  p.rn = rn;
  const int waves = (N + rn - 1) / rn;
  p.blocks = (waves + 3) / 4;
  (void)K;
  return p;
}

template <int XDT, int MB>
static hipError_t launch8(const MatmulArgs& a, const GemvInt8Plan& p) {
  dim3 grid(p.blocks), block(256);
  auto xq = reinterpret_cast<const uint16_t*>(a.x);
  auto Q = reinterpret_cast<const int8_t*>(a.Q);
  auto s = reinterpret_cast<const float*>(a.scales);
  switch (p.rn) {
    case 1: return launch_kernel(gemv_int8_kernel<XDT, MB, 1>, grid, block, a.stream, xq, Q, s, a.y, a.y_dtype, a.M, a.N, a.K);
    case 2: return launch_kernel(gemv_int8_kernel<XDT, MB, 2>, grid, block, a.stream, xq, Q, s, a.y, a.y_dtype, a.M, a.N, a.K);
    case 4: return launch_kernel(gemv_int8_kernel<XDT, MB, 4>, grid, block, a.stream, xq, Q, s, a.y, a.y_dtype, a.M, a.N, a.K);
  }
  return hipErrorInvalidValue;
}

template <int XDT>
static hipError_t launch8_x(const MatmulArgs& a, const GemvInt8Plan& p) {
  switch (p.mb) {
    case 1: return launch8<XDT, 1>(a, p);
    case 2: return launch8<XDT, 2>(a, p);
    case 4: return launch8<XDT, 4>(a, p);
    case 8: return launch8<XDT, 8>(a, p);
    case 16: return launch8<XDT, 16>(a, p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_int8(const MatmulArgs& a, const GemvInt8Plan& p) {
  return a.x_dtype == XF16 ? launch8_x<XF16>(a, p) : launch8_x<XBF16>(a, p);
}

}  // namespace qmm
