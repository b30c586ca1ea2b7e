// gemv_lowbit.hip -- decode / skinny GEMV for int4 and int2 weights in the
// canonical packed layout (BitDistiller quant_matmul_kernel operand
// contract: qw (K/pack, N) int32, scales (G, N) fp16, qzeros (ceil(G/pack), N)).
//
// Shape of the work:
//  * a workgroup owns 16 output columns over the WHOLE of K, so no partial
//    sum ever leaves the workgroup: no workspace, no atomics, no cross-XCD
//    fences (an agent-scope release/acquire writes back and invalidates the
//    XCD's L2, which costs more than the whole decode GEMV);
//  * lane = (cq, rl): column quad n0 = 16 * tile + 4 * cq (one 16-byte load
//    per packed row; the 4 quads of a row read 64 contiguous bytes) and a
//    run of RL consecutive packed rows inside one quantization group.  A
//    workgroup's 64 row-lanes cover 64 * RL rows per pass;
//  * every weight load of a pass is issued before its arithmetic, so the
//    pass is in flight at once and each byte is read exactly once;
//  * the pass's x slice is staged in LDS, pre-paired as (x[t], x[t + P])
//    to match the code fields (loaded before the weights so the in-order
//    load counter lets it go to LDS while the weights stream in);
//  * codes become 16-bit pairs (B + q_a, B + q_b) by masking two fields into
//    the mantissa of a biased constant (B = 1024 fp16, 128 bf16) and meet x
//    in v_dot2c_f32 (fp32 accumulation).  Bias and zero point leave once
//    per lane and pass through
//        sum_k x_k (q_k - z) = sum_k x_k (B + q_k) - (B + z) sum_k x_k,
//    and the group scale multiplies that once: r += s * (...);
//  * the 16 row-lanes of a wave that share a column quad are summed with
//    cross-lane shuffles, then the 4 waves through LDS.
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// Y32: fp32 output; else fp16 / bf16, the type in bits 8+ of m_ydt (M <= 16
// in bits 0-7: the output type rides on M so that the explicit arguments
// stay within 56 bytes, see pack_tiles).
template <int W_BIT, int XDT, int MB, int RL, int CQ, int WAVES, bool Y32>
__global__ __launch_bounds__(64 * WAVES) void gemv_lowbit_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ sc, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int m_ydt, int N, int K, int group_size) {
  const int M = Y32 ? m_ydt : (m_ydt & 0xFF);
  const int ydt = Y32 ? (int)YF32 : (m_ydt >> 8);
  constexpr int PACK = 32 / W_BIT;   // codes per word
  constexpr int PAIRS = PACK / 2;    // 16-bit pairs per word
  constexpr uint32_t FIELD2 = W_BIT == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr uint32_t ZMASK = (1u << W_BIT) - 1u;
  constexpr int NT = 64 * WAVES;             // threads
  constexpr int CW = 4 * CQ;                 // columns per workgroup
  constexpr int GROUPS = WAVES * 64 / CQ;    // row-lanes per workgroup
  constexpr int ROWS_P = RL * GROUPS;        // packed rows per pass
  constexpr int GSTRIDE = RL * PAIRS + 4;    // dwords per row-lane in LDS (+16 B pad)

  const int rows = K / PACK;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cq = lane % CQ;
  const int grp = wave * (64 / CQ) + lane / CQ;
  const int tile = xcd_remap(blockIdx.x, (N + CW - 1) / CW);  // the grid
  const int n0 = tile * CW + cq * 4;
  const bool col_ok = n0 < N;  // N % 4 == 0: the quad is all in or all out

  __shared__ uint32_t xl[MB * GROUPS * GSTRIDE];
  constexpr int ITEMS = MB * ROWS_P;
  constexpr int PER_T = (ITEMS + NT - 1) / NT;

  float r[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) r[m][c] = 0.f;

  const int passes = (rows + ROWS_P - 1) / ROWS_P;
  for (int p = 0; p < passes; ++p) {
    const int r_base = p * ROWS_P;
    const int row0 = r_base + grp * RL;
    const bool live = col_ok && row0 < rows;  // rows % RL == 0: all RL rows or none

    // 1. x slice of this pass (first, see header)
    u32x4_t xr[PER_T][PACK / 8];
#pragma unroll
    for (int j = 0; j < PER_T; ++j) {
      const int it = threadIdx.x + j * NT;
      const int m = min(it / ROWS_P, M - 1);
      const int rr = min(r_base + it % ROWS_P, rows - 1);
#pragma unroll
      for (int v = 0; v < PACK / 8; ++v)
        xr[j][v] = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * K + (size_t)rr * PACK + 8 * v);
    }

    // 2. every weight load of this lane for the pass.  Loads are never
    // predicated: a dead lane reads a clamped, valid address and its result
    // is dropped in step 6.  (Loads under a lane mask leave the compiler
    // unsure how many loads follow the x slice, and it then waits for all of
    // them before x can go to LDS.)
    const int rowc = live ? row0 : 0;
    const int nc = col_ok ? n0 : 0;
    u32x4_t wq[RL];
#pragma unroll
    for (int i = 0; i < RL; ++i)
      wq[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(qw + (size_t)(rowc + i) * N + nc));

    // 3. scale and zero point of the lane's group, for its four columns
    const int g = (rowc * PACK) / group_size;
    uint2 s2 = *reinterpret_cast<const uint2*>(sc + (size_t)g * N + nc);
    u32x4_t zw = u32x4_t{0u, 0u, 0u, 0u};
    if (qz != nullptr)  // uniform: no lane mask
      zw = *reinterpret_cast<const u32x4_t*>(qz + (size_t)(g / PACK) * N + nc);

    // 4. x to LDS as (x[t], x[t + PAIRS]) pairs
    if (p > 0) __syncthreads();  // previous pass done reading xl
#pragma unroll
    for (int j = 0; j < PER_T; ++j) {
      const int it = threadIdx.x + j * NT;
      if (it < ITEMS) {
        const int m = it / ROWS_P, rr = it % ROWS_P;
        const bool ok = m < M && r_base + rr < rows;  // else x is zero
        uint32_t* dst = xl + (m * GROUPS + rr / RL) * GSTRIDE + (rr % RL) * PAIRS;
        uint32_t d[PAIRS];
#pragma unroll
        for (int v = 0; v < PACK / 8; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * v + e] = ok ? xr[j][v][e] : 0u;
#pragma unroll
        for (int t = 0; t < PAIRS; ++t) {
          const uint32_t a = d[t / 2], b = d[t / 2 + PAIRS / 2];
          dst[t] = (t & 1) ? pair_hi(a, b) : pair_lo(a, b);
        }
      }
    }
    __syncthreads();

    // 5. dot products
    float acc[MB][4];
    float xs[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      xs[m] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][c] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      uint32_t wp[4][PAIRS];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < PAIRS; ++t)
          wp[c][t] = ((wq[i][c] >> (W_BIT * t)) & FIELD2) | Bias<XDT>::pair;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const uint32_t* xp = xl + (m * GROUPS + grp) * GSTRIDE + i * PAIRS;
          uint32_t xv[PAIRS];
#pragma unroll
          for (int v = 0; v < PAIRS / 4; ++v) {
            const u32x4_t t4 = *reinterpret_cast<const u32x4_t*>(xp + 4 * v);
            xv[4 * v] = t4[0];
            xv[4 * v + 1] = t4[1];
            xv[4 * v + 2] = t4[2];
            xv[4 * v + 3] = t4[3];
          }
#pragma unroll
          for (int t = 0; t < PAIRS; ++t) {
            xs[m] = dot2<XDT>(xv[t], Bias<XDT>::one_pair, xs[m]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[m][c] = dot2<XDT>(xv[t], wp[c][t], acc[m][c]);
          }
        }
      }
    }

    // 6. this pass's group: scale and (bias + zero) per column
    if (live) {
      const uint32_t sh[4] = {s2.x & 0xFFFFu, s2.x >> 16, s2.y & 0xFFFFu, s2.y >> 16};
      const int zsh = (g % PACK) * W_BIT;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float s = f16_bits_to_f32((uint16_t)sh[c]);
        const uint32_t z = qz != nullptr ? (zw[c] >> zsh) & ZMASK : (1u << (W_BIT - 1));
        const float bz = Bias<XDT>::value + (float)z;
#pragma unroll
        for (int m = 0; m < MB; ++m) r[m][c] += s * (acc[m][c] - bz * xs[m]);
      }
    }
  }

  // 7. sum the row-lanes of each column quad: with 4 quads, two DPP row
  // rotations (by 4 and 8 lanes) sum the 4 row-lanes of a quad inside each
  // 16-lane row, and the rows' and waves' partials meet in LDS (no
  // cross-row shuffle); otherwise cross-lane shuffles sum the whole wave
  constexpr int PARTS = CQ == 4 ? 4 : 1;  // partials per wave left for LDS
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = r[m][c];
      if constexpr (CQ == 4) {
        v = dpp_add<0x124, 0xF>(v);  // row_ror:4
        v = dpp_add<0x128, 0xF>(v);  // row_ror:8
      } else {
#pragma unroll
        for (int b = CQ; b < 64; b *= 2) v += __shfl_xor(v, b);
      }
      r[m][c] = v;
    }
  __syncthreads();
  float* red = reinterpret_cast<float*>(xl);  // [WAVES * PARTS][MB][CW]
  static_assert(WAVES * PARTS * MB * CW <= MB * GROUPS * GSTRIDE, "LDS reuse");
  if ((lane & 15) < CQ && (PARTS == 4 || lane < CQ)) {
    const int part = wave * PARTS + (PARTS == 4 ? lane >> 4 : 0);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[(part * MB + m) * CW + cq * 4 + c] = r[m][c];
  }
  __syncthreads();
  auto store = [&](auto* yt) {
    using T = typename std::remove_pointer<decltype(yt)>::type;
    for (int o = threadIdx.x; o < MB * CW; o += NT) {
      const int m = o / CW, col = o % CW;
      const int n = tile * CW + col;
      if (m < M && n < N) {
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < WAVES * PARTS; ++v) sum += red[(v * MB + m) * CW + col];
        yt[(size_t)m * N + n] = (T)sum;
      }
    }
  };
  if constexpr (Y32) store(reinterpret_cast<float*>(y));
  else with_y(y, ydt, store);
}

// ---------------------------------------------------------------- host side
static int m_bucket(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// LDS of one pass's x slice (64 row-lanes, +16 B pad each), kept within
// 80 KiB so a workgroup always fits the CU.
static constexpr size_t x_lds_bytes(int mb, int rl, int pairs, int groups = 64) {
  return (size_t)mb * groups * (rl * pairs + 4) * 4;
}
static constexpr size_t kXldsMax = 80 * 1024;

GemvLowbitPlan plan_gemv_lowbit(int M, int N, int K, int w_bit, int group_size) {
  GemvLowbitPlan p{};
  const int pack = 32 / w_bit;
  const int pairs = pack / 2;
  const int rows = K / pack;
  const int rpg = group_size / pack;  // packed rows per group
  p.mb = m_bucket(M);
  p.n_tiles = (N + 15) / 16;
  // rows per lane: a power of two dividing the group, no more than the 64
  // row-lanes need to cover K in one pass, and an x slice within 64 KiB
  // (per-column scales: the group is all of K, rpg = K / pack, an even number)
  int rl = 16;
  while (rl > 2 && (rl > rpg || rpg % rl != 0)) rl /= 2;
  while (rl > 2 && rl * 64 / 2 >= rows) rl /= 2;
  while (rl > 2 && x_lds_bytes(p.mb, rl, pairs) > kXldsMax) rl /= 2;
  static const int want = env_int("QMM_GEMV_RL");
  if (want >= 2 && want <= rl && (rl % want) == 0) rl = want;
  p.rl = rl;
  p.workspace_bytes = 0;
  return p;
}

template <int W_BIT, int XDT, int MB, int RL>
static hipError_t launch_rl(const MatmulArgs& a, const GemvLowbitPlan& p) {
  if constexpr (x_lds_bytes(MB, RL, 16 / W_BIT) > kXldsMax && RL > 2) {
    return hipErrorInvalidValue;  // never planned
  } else {
  const auto k = a.y_dtype == YF32 ? gemv_lowbit_kernel<W_BIT, XDT, MB, RL, 4, 4, true>
                                   : gemv_lowbit_kernel<W_BIT, XDT, MB, RL, 4, 4, false>;
  return launch_kernel(k, dim3(p.n_tiles), dim3(256), a.stream, a.x, a.Q, a.scales, a.zeros, a.y,
                       a.y_dtype == YF32 ? a.M : (a.M | (a.y_dtype << 8)), a.N, a.K,
                       a.group_size);
  }
}

template <int W_BIT, int XDT, int MB>
static hipError_t launch_mb(const MatmulArgs& a, const GemvLowbitPlan& p) {
  switch (p.rl) {
    case 2: return launch_rl<W_BIT, XDT, MB, 2>(a, p);
    case 4: return launch_rl<W_BIT, XDT, MB, 4>(a, p);
    case 8: return launch_rl<W_BIT, XDT, MB, 8>(a, p);
    case 16: return launch_rl<W_BIT, XDT, MB, 16>(a, p);
  }
  return hipErrorInvalidValue;
}

template <int W_BIT, int XDT>
static hipError_t launch_xdt(const MatmulArgs& a, const GemvLowbitPlan& p) {
  switch (p.mb) {
    case 1: return launch_mb<W_BIT, XDT, 1>(a, p);
    case 2: return launch_mb<W_BIT, XDT, 2>(a, p);
    case 4: return launch_mb<W_BIT, XDT, 4>(a, p);
    case 8: return launch_mb<W_BIT, XDT, 8>(a, p);
    case 16: return launch_mb<W_BIT, XDT, 16>(a, p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_lowbit(const MatmulArgs& a, const GemvLowbitPlan& p) {
  if (a.w_bit == 4) {
    return a.x_dtype == XF16 ? launch_xdt<4, XF16>(a, p) : launch_xdt<4, XBF16>(a, p);
  }
  return a.x_dtype == XF16 ? launch_xdt<2, XF16>(a, p) : launch_xdt<2, XBF16>(a, p);
}

}  // namespace qmm
