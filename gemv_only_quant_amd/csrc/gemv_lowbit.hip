// gemv_lowbit.hip -- decode / skinny GEMV for int4 and int2 weights in the
// canonical packed layout (BitDistiller quant_matmul_kernel operand
// contract: qw (K/pack, N) int32, scales (G, N) fp16, qzeros (ceil(G/pack), N)).
//
// Shape of the work:
//  * a wave owns 64 columns: lane = 4 * 16 lanes; lane (rl, cq) holds column
//    quad n0 = 64 * tile + 4 * cq (one 16-byte load per packed row, so a row
//    of 16 lanes reads 256 contiguous bytes) and a run of RL consecutive
//    packed rows that never crosses a quantization group;
//  * every weight load of a lane is issued before any arithmetic, so the
//    whole slice is in flight at once (each byte is read exactly once);
//  * codes are turned into 16-bit pairs (B + q_a, B + q_b) by masking two
//    fields into the mantissa of a biased constant (B = 1024 for fp16,
//    128 for bf16), and multiplied against x pairs with v_dot2c_f32, which
//    accumulates in fp32.  The zero point and the bias come out once per
//    lane through the identity
//        sum_k x_k (q_k - z) = sum_k x_k (B + q_k) - (B + z) sum_k x_k,
//    and the group scale is applied once per lane: r = s * (...);
//  * partial sums: lanes of a wave that share columns (xor 16, 32) ->
//    waves of a workgroup through LDS -> workgroups along K through the
//    workspace, where the last workgroup to arrive (atomic ticket) adds the
//    partials in a fixed order and re-arms the ticket counter.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int W_BIT, int XDT, int MB, int RL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_lowbit_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ sc, const uint32_t* __restrict__ qz, float* __restrict__ y,
    float* __restrict__ part, unsigned* __restrict__ ticket, int M, int N, int K,
    int group_size, int ksplit) {
  constexpr int PACK = 32 / W_BIT;   // codes per word
  constexpr int PAIRS = PACK / 2;    // 16-bit pairs per word
  constexpr uint32_t FIELD2 = W_BIT == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr uint32_t ZMASK = (1u << W_BIT) - 1u;
  constexpr int XW = PACK / 2;       // x dwords per packed row (natural pairs)

  const int rows = K / PACK;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cq = lane & 15;
  const int rl = lane >> 4;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = w / ksplit;
  const int ks = w - tile * ksplit;
  const int n0 = tile * 64 + cq * 4;
  const int row0 = ((ks * WAVES + wave) * 4 + rl) * RL;
  const bool live = (n0 < N) && (row0 < rows);  // all RL rows and 4 columns, or none

  // 1. issue every weight load of this lane
  u32x4_t wq[RL];
#pragma unroll
  for (int i = 0; i < RL; ++i) {
    wq[i] = live ? *reinterpret_cast<const u32x4_t*>(qw + (size_t)(row0 + i) * N + n0)
                 : u32x4_t{0u, 0u, 0u, 0u};
  }

  // 2. scale and zero point of this lane's group, for its four columns
  const int g = live ? (row0 * PACK) / group_size : 0;
  float s[4], bz[4];
  {
    uint2 s2 = live ? *reinterpret_cast<const uint2*>(sc + (size_t)g * N + n0) : uint2{0u, 0u};
    s[0] = f16_bits_to_f32(s2.x & 0xFFFFu);
    s[1] = f16_bits_to_f32(s2.x >> 16);
    s[2] = f16_bits_to_f32(s2.y & 0xFFFFu);
    s[3] = f16_bits_to_f32(s2.y >> 16);
    u32x4_t zw = u32x4_t{0u, 0u, 0u, 0u};
    if (qz != nullptr && live)
      zw = *reinterpret_cast<const u32x4_t*>(qz + (size_t)(g / PACK) * N + n0);
    const int zsh = (g % PACK) * W_BIT;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t z = qz != nullptr ? (zw[c] >> zsh) & ZMASK : (1u << (W_BIT - 1));
      bz[c] = Bias<XDT>::value + (float)z;
    }
  }

  // 3. dot products against x
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
    // weight pairs (B + q[t], B + q[t + PAIRS]) for each column
    uint32_t wp[4][PAIRS];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < PAIRS; ++t)
        wp[c][t] = ((wq[i][c] >> (W_BIT * t)) & FIELD2) | Bias<XDT>::pair;

    const size_t kx = (size_t)(row0 + i) * PACK;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < M) {
        // natural x halves k .. k+PACK-1 of row m, regrouped as (x[t], x[t+PAIRS])
        uint32_t xd[XW];
        if (live) {
#pragma unroll
          for (int v = 0; v < XW / 4; ++v) {
            u32x4_t t4 = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * K + kx + 8 * v);
            xd[4 * v + 0] = t4[0];
            xd[4 * v + 1] = t4[1];
            xd[4 * v + 2] = t4[2];
            xd[4 * v + 3] = t4[3];
          }
        } else {
#pragma unroll
          for (int v = 0; v < XW; ++v) xd[v] = 0u;
        }
#pragma unroll
        for (int t = 0; t < PAIRS; ++t) {
          const uint32_t a = xd[t / 2], b = xd[t / 2 + PAIRS / 2];
          const uint32_t xp = (t & 1) ? pair_hi(a, b) : pair_lo(a, b);
          xs[m] = dot2<XDT>(xp, Bias<XDT>::one_pair, xs[m]);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[m][c] = dot2<XDT>(xp, wp[c][t], acc[m][c]);
        }
      }
    }
  }

  // 4. lane result, then sum over the four row-lanes sharing these columns
  float r[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = live ? s[c] * (acc[m][c] - bz[c] * xs[m]) : 0.f;
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      r[m][c] = v;
    }

  // 5. across the waves of the workgroup
  __shared__ float red[WAVES][MB][64];
  __shared__ int last_flag;
  if (rl == 0) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[wave][m][cq * 4 + c] = r[m][c];
  }
  __syncthreads();

  for (int o = threadIdx.x; o < MB * 64; o += 64 * WAVES) {
    const int m = o >> 6, col = o & 63;
    const int n = tile * 64 + col;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) sum += red[v][m][col];
    if (m < M && n < N) {
      if (ksplit == 1) y[(size_t)m * N + n] = sum;
      else part[((size_t)ks * M + m) * N + n] = sum;
    }
  }
  if (ksplit == 1) return;

  // 6. across workgroups: the last arrival adds the partials in ks order
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_flag = (atomicAdd(&ticket[tile], 1u) == (unsigned)(ksplit - 1));
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  for (int o = threadIdx.x; o < MB * 64; o += 64 * WAVES) {
    const int m = o >> 6, col = o & 63;
    const int n = tile * 64 + col;
    if (m < M && n < N) {
      float sum = 0.f;
      for (int j = 0; j < ksplit; ++j) sum += __builtin_nontemporal_load(&part[((size_t)j * M + m) * N + n]);
      y[(size_t)m * N + n] = sum;
    }
  }
  if (threadIdx.x == 0) atomicExch(&ticket[tile], 0u);
}

// ---------------------------------------------------------------- host side
static constexpr int kGemvWaves = 4;

static int m_bucket(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

GemvLowbitPlan plan_gemv_lowbit(int M, int N, int K, int w_bit, int group_size) {
  GemvLowbitPlan p{};
  const int pack = 32 / w_bit;
  const int rows = K / pack;
  const int rpg = group_size / pack;  // packed rows per group (power of two)
  p.mb = m_bucket(M);
  p.waves = kGemvWaves;
  p.n_tiles = (N + 63) / 64;
  int rl = rpg < 16 ? rpg : 16;
  const int want = env_int("QMM_GEMV_RL");
  if (want > 0 && want <= rl && (rl % want) == 0) rl = want;
  p.rl = rl;
  const int rows_per_block = rl * 4 * p.waves;
  p.ksplit = (rows + rows_per_block - 1) / rows_per_block;
  if (p.ksplit < 1) p.ksplit = 1;
  p.workspace_bytes = 0;
  if (p.ksplit > 1) {
    const size_t tickets = ((size_t)p.n_tiles * 4 + 255) / 256 * 256;
    p.workspace_bytes = tickets + (size_t)p.ksplit * M * N * sizeof(float);
  }
  return p;
}

template <int W_BIT, int XDT, int MB, int RL>
static hipError_t launch_rl(const MatmulArgs& a, const GemvLowbitPlan& p) {
  unsigned* ticket = nullptr;
  float* part = nullptr;
  if (p.ksplit > 1) {
    ticket = reinterpret_cast<unsigned*>(a.workspace);
    const size_t tickets = ((size_t)p.n_tiles * 4 + 255) / 256 * 256;
    part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + tickets);
  }
  dim3 grid(p.n_tiles * p.ksplit), block(64 * kGemvWaves);
  hipLaunchKernelGGL((gemv_lowbit_kernel<W_BIT, XDT, MB, RL, kGemvWaves>), grid, block, 0,
                     a.stream, reinterpret_cast<const uint16_t*>(a.x),
                     reinterpret_cast<const uint32_t*>(a.Q),
                     reinterpret_cast<const uint16_t*>(a.scales),
                     reinterpret_cast<const uint32_t*>(a.zeros), a.y, part, ticket, a.M, a.N,
                     a.K, a.group_size, p.ksplit);
  return hipGetLastError();
}

template <int W_BIT, int XDT, int MB>
static hipError_t launch_mb(const MatmulArgs& a, const GemvLowbitPlan& p) {
  switch (p.rl) {
    case 2: if constexpr (W_BIT == 2) return launch_rl<W_BIT, XDT, MB, 2>(a, p); break;
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
