// gemm_mfma.hip -- matrix-core path: y = x * dequant(Q) with Q in the tile
// layout written by qmm_pack (repack.hip), on v_mfma_f32_16x16x32_{f16,bf16}.
//
// Skinny kernel (decode batches, M up to a few 16-row tiles), HBM-bound:
//  * a workgroup = 4 waves on one M-tile and one K-range; each wave owns NT
//    16-column strips.  Per stage (128 k; 256 k for int2) a lane loads ONE
//    16-byte slot of each strip's 1 KiB layout block -- already the MFMA
//    B-operand lane map -- so weights go HBM -> VGPR -> MFMA without LDS;
//  * codes become operand pairs (B + q_a, B + q_b) with one mask-or per pair
//    (fp16 B = 1024, bf16 B = 128; int8: u = q + 128 through a byte perm
//    (fp16) or byte->float->bf16 converts (bf16)), exact in 16 bits;
//  * one extra MFMA per step against an all-ones B gives the row sums of x
//    over the same k, in the accumulator layout; at each group end
//        y += s * (acc - (B + z) * xsum)
//    in fp32 -- so the matrix cores only see exact integers and the group
//    scale is applied once per group (the page's w = (q - z) * s, regrouped);
//  * the x tile of a stage goes through double-buffered LDS (ds_read does
//    not wait on the in-order weight loads); weights, scales and zeros of
//    stage i + 1 are in flight while stage i computes;
//  * K is split over workgroups when the tile grid is small; partial tiles
//    meet in the workspace and the last workgroup to arrive adds them in a
//    fixed order and re-arms the ticket.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int W_BIT> struct Stage;
template <> struct Stage<4> { static constexpr int KB = 128, BLK = 1, PACK = 8; };
template <> struct Stage<2> { static constexpr int KB = 256, BLK = 1, PACK = 16; };
template <> struct Stage<8> { static constexpr int KB = 64, BLK = 2, PACK = 0; };

template <int XDT> __device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b,
                                                            const f32x4_t& c);
template <> __device__ __forceinline__ f32x4_t mfma16<XF16>(const u32x4_t& a, const u32x4_t& b,
                                                           const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma16<XBF16>(const u32x4_t& a, const u32x4_t& b,
                                                            const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Bias removed after the sum: low-bit B, int8 1152 (fp16) / 128 (bf16).
template <int W_BIT, int XDT> struct OpBias {
  static constexpr float value = Bias<XDT>::value;
};
template <> struct OpBias<8, XF16> { static constexpr float value = 1152.0f; };
template <> struct OpBias<8, XBF16> { static constexpr float value = 128.0f; };

// B operand of k step `st` (32 deep) from a lane's slot(s) of one stage.
// int4: word st, pair t = fields (t, t + 4).  int2: word st / 2, k half
// h = st % 2, pair t = fields (4 h + t, 8 + 4 h + t).  int8: bytes
// 8 st' .. 8 st' + 7 of block st / 2 (st' = st % 2), natural pairs.
template <int W_BIT, int XDT>
__device__ __forceinline__ u32x4_t bfrag(const u32x4_t* slot, int st) {
  u32x4_t b;
  if constexpr (W_BIT == 4) {
    const uint32_t w = slot[0][st];
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = ((w >> (4 * t)) & 0x000F000Fu) | Bias<XDT>::pair;
  } else if constexpr (W_BIT == 2) {
    const uint32_t w = slot[0][st >> 1];
    const int h = st & 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = ((w >> (2 * (4 * h + t))) & 0x00030003u) | Bias<XDT>::pair;
  } else {
    const u32x4_t& s = slot[st >> 1];
    const int h = st & 1;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t u = s[2 * h + d] ^ 0x80808080u;
      if constexpr (XDT == XF16) {
        b[2 * d] = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
        b[2 * d + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
      } else {
        bf16x2_t p0 = {(__bf16)(float)(u & 0xFFu), (__bf16)(float)((u >> 8) & 0xFFu)};
        bf16x2_t p1 = {(__bf16)(float)((u >> 16) & 0xFFu), (__bf16)(float)(u >> 24)};
        b[2 * d] = __builtin_bit_cast(uint32_t, p0);
        b[2 * d + 1] = __builtin_bit_cast(uint32_t, p1);
      }
    }
  }
  return b;
}

template <int W_BIT, int XDT, int GS, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const void* __restrict__ scales, const uint32_t* __restrict__ qz, float* __restrict__ y,
    float* __restrict__ part, unsigned* __restrict__ ticket, int M, int N, int K, int ksplit,
    int n_tiles) {
  constexpr int WAVES = 4;
  constexpr int KB = Stage<W_BIT>::KB;
  constexpr int BLK = Stage<W_BIT>::BLK;
  constexpr int KS = KB * BLK;           // k per stage
  constexpr int STEPS = KS / 32;         // MFMA k steps per stage
  constexpr int ROWS = 16 * MT;          // x rows per workgroup
  constexpr int XROW = KS + 8;           // LDS row stride in halves (16 B pad)
  constexpr int CHUNKS = ROWS * KS / 8;  // 16-byte x chunks per stage
  constexpr int XPT = (CHUNKS + 255) / 256;
  constexpr bool LOWBIT = W_BIT != 8;
  constexpr int PACK = LOWBIT ? Stage<W_BIT>::PACK : 1;
  constexpr int GSZ = LOWBIT ? GS : KS;
  constexpr int NGS = GSZ < KS ? KS / GSZ : 1;  // groups touched per stage
  constexpr float CB = OpBias<W_BIT, XDT>::value;

  __shared__ uint16_t xl[2][ROWS * XROW];
  __shared__ int last_flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, quad = lane >> 4;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int ks = w % ksplit;
  const int tile = w / ksplit;
  const int nt = tile % n_tiles, mt_idx = tile / n_tiles;
  const int m0 = mt_idx * ROWS;
  const int strips = N / 16;
  const int s0 = (nt * WAVES + wave) * NT;
  const int nblk = K / KB;
  const int nst = (nblk + BLK - 1) / BLK;  // stages along K
  const int per = (nst + ksplit - 1) / ksplit;
  const int st0 = ks * per;
  const int st1 = min(nst, st0 + per);

  bool sval[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) sval[s] = s0 + s < strips;

  // One stage in registers: weight slots, scales and zero words of the
  // groups it touches, and this thread's share of the x tile.
  struct StageRegs {
    u32x4_t w[NT][BLK];
    uint32_t sc[NT][NGS];
    uint32_t zw[NT];
    u32x4_t xr[XPT];
  };
  auto load_stage = [&](int st, StageRegs& R) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int row = c / (KS / 8), col = st * KS + (c % (KS / 8)) * 8;
      const int m = m0 + row;
      R.xr[j] = (c < CHUNKS && m < M && col < K)
                    ? *reinterpret_cast<const u32x4_t*>(x + (size_t)m * K + col)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < NT; ++s) {
#pragma unroll
      for (int b = 0; b < BLK; ++b) {
        const int kb = st * BLK + b;
        R.w[s][b] = (sval[s] && kb < nblk) ? Qt[((size_t)(s0 + s) * nblk + kb) * 64 + lane]
                                           : u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (LOWBIT) {
        const int n = 16 * (s0 + s) + l16;
        const int g0 = (st * KS) / GS;
        const uint16_t* s16 = reinterpret_cast<const uint16_t*>(scales);
#pragma unroll
        for (int q = 0; q < NGS; ++q)
          R.sc[s][q] = sval[s] ? s16[(size_t)(g0 + q) * N + n] : 0u;
        R.zw[s] = (qz != nullptr && sval[s]) ? qz[(size_t)(g0 / PACK) * N + n] : 0u;
      }
    }
  };
  auto store_x = [&](const StageRegs& R, int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      if (c < CHUNKS) {
        const int row = c / (KS / 8), col = (c % (KS / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(&xl[buf][row * XROW + col]) = R.xr[j];
      }
    }
  };

  f32x4_t acc[MT][NT], yacc[MT][NT], xs[MT];
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    xs[i] = zero4;
#pragma unroll
    for (int s = 0; s < NT; ++s) acc[i][s] = yacc[i][s] = zero4;
  }
  const u32x4_t ones = {Bias<XDT>::one_pair, Bias<XDT>::one_pair, Bias<XDT>::one_pair,
                        Bias<XDT>::one_pair};

  // y += s * (acc - (B + z) * xsum), then restart the group sums
  auto flush = [&](const float (&sc)[NT], const float (&bz)[NT]) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int s = 0; s < NT; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[i][s][r] += sc[s] * (acc[i][s][r] - bz[s] * xs[i][r]);
        acc[i][s] = zero4;
      }
      xs[i] = zero4;
    }
  };
  // scale and (bias + zero) of group q of the current stage
  auto group_consts = [&](const StageRegs& R, int st, int q, float (&sc)[NT], float (&bz)[NT]) {
    const int g = (st * KS) / GS + q;
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      sc[s] = f16_bits_to_f32((uint16_t)R.sc[s][q]);
      const uint32_t z = qz != nullptr ? (R.zw[s] >> ((g % PACK) * W_BIT)) & ((1u << W_BIT) - 1u)
                                       : (1u << (W_BIT - 1));
      bz[s] = CB + (float)z;
    }
  };

  if (st0 < st1) {
    StageRegs cur, nxt;
    load_stage(st0, cur);
    store_x(cur, 0);
    __syncthreads();
    for (int st = st0; st < st1; ++st) {
      const int buf = (st - st0) & 1;
      const bool more = st + 1 < st1;
      if (more) load_stage(st + 1, nxt);
      const uint16_t* xb = xl[buf];
#pragma unroll
      for (int k = 0; k < STEPS; ++k) {
        u32x4_t a[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          a[i] = *reinterpret_cast<const u32x4_t*>(&xb[(16 * i + l16) * XROW + 32 * k + 8 * quad]);
          xs[i] = mfma16<XDT>(a[i], ones, xs[i]);
        }
#pragma unroll
        for (int s = 0; s < NT; ++s) {
          const u32x4_t b = bfrag<W_BIT, XDT>(cur.w[s], k);
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[i][s] = mfma16<XDT>(a[i], b, acc[i][s]);
        }
        if constexpr (LOWBIT) {
          const int kend = st * KS + 32 * (k + 1);  // one past this step
          if (kend % GS == 0 || (k == STEPS - 1 && !more)) {
            float sc[NT], bz[NT];
            group_consts(cur, st, GS < KS ? (32 * k) / GS : 0, sc, bz);
            flush(sc, bz);
          }
        }
      }
      if (more) {
        store_x(nxt, buf ^ 1);
        cur = nxt;
      }
      __syncthreads();
    }
  }
  if constexpr (!LOWBIT) {
    float sc[NT], bz[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      sc[s] = sval[s] ? reinterpret_cast<const float*>(scales)[16 * (s0 + s) + l16] : 0.f;
      bz[s] = CB;
    }
    flush(sc, bz);
  }

  // ---- write the tile (or this K-range's partial) ----------------------
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      if (!sval[s]) continue;
      const int n = 16 * (s0 + s) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * quad + r;
        if (m < M) {
          if (ksplit == 1) y[(size_t)m * N + n] = yacc[i][s][r];
          else part[((size_t)ks * M + m) * N + n] = yacc[i][s][r];
        }
      }
    }
  if (ksplit == 1) return;

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_flag = (atomicAdd(&ticket[tile], 1u) == (unsigned)(ksplit - 1));
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const int ncols = 16 * NT * WAVES;
  const int n_first = 16 * nt * NT * WAVES;
  for (int o = threadIdx.x; o < ROWS * ncols; o += 256) {
    const int m = m0 + o / ncols, n = n_first + o % ncols;
    if (m < M && n < N) {
      float sum = 0.f;
      for (int j = 0; j < ksplit; ++j) sum += part[((size_t)j * M + m) * N + n];
      y[(size_t)m * N + n] = sum;
    }
  }
  if (threadIdx.x == 0) atomicExch(&ticket[tile], 0u);
}

// ---------------------------------------------------------------- host side
static void skinny_shape(int M, int w_bit, int* mt, int* nt) {
  if (M <= 16) { *mt = 1; *nt = 4; }
  else if (M <= 32) { *mt = 2; *nt = 4; }
  else { *mt = 4; *nt = 2; }
  (void)w_bit;
}

GemmPlan plan_gemm(int M, int N, int K, int w_bit, int group_size) {
  GemmPlan p{};
  (void)group_size;
  int mt, nt;
  skinny_shape(M, w_bit, &mt, &nt);
  p.kind = 0;
  p.mtile = 16 * mt;
  const int strips = N / 16;
  p.n_tiles = (strips + 4 * nt - 1) / (4 * nt);
  p.m_tiles = (M + p.mtile - 1) / p.mtile;
  const int ks_ext = w_bit == 2 ? 256 : 128;  // k per pipeline stage
  const int nst = (K + ks_ext - 1) / ks_ext;
  const long tiles = (long)p.n_tiles * p.m_tiles;
  int ksplit = (int)((512 + tiles - 1) / tiles);
  const int want = env_int("QMM_GEMM_KSPLIT");
  if (want > 0) ksplit = want;
  if (ksplit > nst) ksplit = nst;
  if (ksplit < 1) ksplit = 1;
  // every split gets at least one stage
  const int per = (nst + ksplit - 1) / ksplit;
  ksplit = (nst + per - 1) / per;
  p.ksplit = ksplit;
  p.workspace_bytes = 0;
  if (ksplit > 1) {
    const size_t tickets = ((size_t)tiles * 4 + 255) / 256 * 256;
    p.workspace_bytes = tickets + (size_t)ksplit * M * N * sizeof(float);
  }
  return p;
}

template <int W_BIT, int XDT, int GS, int MT, int NT>
static hipError_t launch_skinny(const MatmulArgs& a, const GemmPlan& p) {
  unsigned* ticket = nullptr;
  float* part = nullptr;
  if (p.ksplit > 1) {
    ticket = reinterpret_cast<unsigned*>(a.workspace);
    const size_t tickets = ((size_t)p.n_tiles * p.m_tiles * 4 + 255) / 256 * 256;
    part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + tickets);
  }
  const long blocks = (long)p.n_tiles * p.m_tiles * p.ksplit;
  hipLaunchKernelGGL((gemm_skinny_kernel<W_BIT, XDT, GS, MT, NT>), dim3((unsigned)blocks),
                     dim3(256), 0, a.stream, reinterpret_cast<const uint16_t*>(a.x),
                     reinterpret_cast<const u32x4_t*>(a.Q), a.scales,
                     reinterpret_cast<const uint32_t*>(a.zeros), a.y, part, ticket, a.M, a.N,
                     a.K, p.ksplit, p.n_tiles);
  return hipGetLastError();
}

template <int W_BIT, int XDT, int GS>
static hipError_t launch_mt(const MatmulArgs& a, const GemmPlan& p) {
  switch (p.mtile) {
    case 16: return launch_skinny<W_BIT, XDT, GS, 1, 4>(a, p);
    case 32: return launch_skinny<W_BIT, XDT, GS, 2, 4>(a, p);
    case 64: return launch_skinny<W_BIT, XDT, GS, 4, 2>(a, p);
  }
  return hipErrorInvalidValue;
}

template <int W_BIT, int XDT>
static hipError_t launch_gs(const MatmulArgs& a, const GemmPlan& p) {
  if constexpr (W_BIT == 8) {
    return launch_mt<8, XDT, 0>(a, p);
  } else {
    switch (a.group_size) {
      case 32: return launch_mt<W_BIT, XDT, 32>(a, p);
      case 64: return launch_mt<W_BIT, XDT, 64>(a, p);
      case 128: return launch_mt<W_BIT, XDT, 128>(a, p);
      case 256: return launch_mt<W_BIT, XDT, 256>(a, p);
    }
    return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const MatmulArgs& a, const GemmPlan& p) {
  const bool f16 = a.x_dtype == XF16;
  switch (a.w_bit) {
    case 4: return f16 ? launch_gs<4, XF16>(a, p) : launch_gs<4, XBF16>(a, p);
    case 2: return f16 ? launch_gs<2, XF16>(a, p) : launch_gs<2, XBF16>(a, p);
    case 8: return f16 ? launch_gs<8, XF16>(a, p) : launch_gs<8, XBF16>(a, p);
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
