// gemm_mfma.hip -- matrix-core path: y = x * dequant(Q) with Q in the tile
// layout written by qmm_pack (repack.hip), on v_mfma_f32_16x16x32_{f16,bf16}.
//
// Skinny kernel (decode batches, M up to a few 16-row tiles), HBM-bound:
//  * a workgroup = 4 waves on one M-tile (MT 16-row tiles) and NT 16-column
//    strips; the 4 waves split K into quarters, and their partial tiles meet
//    in LDS at the end, so no partial sum leaves the workgroup;
//  * per stage (128 k; 256 k for int2; two 64-deep blocks for int8) a lane
//    loads ONE 16-byte slot of each strip's 1 KiB layout block -- already
//    the MFMA B-operand lane map -- so weights go HBM -> VGPR -> MFMA
//    without LDS; x arrives as whole rows and becomes operand fragments
//    through a small per-wave LDS tile; a DEPTH-deep ring of stages in
//    registers (buffer loads, issued in ring order) keeps the loads in flight;
//  * codes become operand pairs (B + q_a, B + q_b) with one mask-or per pair
//    (fp16 B = 1024, bf16 B = 128; int8: u = q + 128 through a byte perm
//    (fp16) or byte->float->bf16 converts (bf16)), exact in 16 bits;
//  * one extra MFMA per step against an all-ones B gives the row sums of x
//    over the same k, in the accumulator layout; at each group end
//        y += s * (acc - (B + z) * xsum)
//    in fp32 -- so the matrix cores only see exact integers and the group
//    scale is applied once per group (the page's w = (q - z) * s, regrouped).
#include <algorithm>
#include <type_traits>

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

// SPLIT: K is also divided over S = splits_of(tile_opts) workgroups per tile
// (consecutive work ids, so one XCD); each writes its partial tile to the
// workspace and takes a ticket, and the last of the S to arrive adds the S
// partials in split order and writes y (see the end of the body).
template <int W_BIT, int XDT, int GS, int MT, int NT, int DEPTH, int WAVES, bool SPLIT>
__device__ __forceinline__ void skinny_body(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const void* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    uint32_t* __restrict__ ws, int M, int N, int K, int tile_opts) {
  const int n_tiles = tiles_of(tile_opts), ydt = ydt_of(tile_opts), gmask = gmask_of(tile_opts);
  constexpr int KB = Stage<W_BIT>::KB;
  constexpr int BLK = Stage<W_BIT>::BLK;
  constexpr int KS = KB * BLK;           // k per stage
  constexpr int STEPS = KS / 32;         // MFMA k steps per stage
  constexpr bool LOWBIT = W_BIT != 8;
  constexpr int PACK = LOWBIT ? Stage<W_BIT>::PACK : 1;
  constexpr int GSZ = LOWBIT ? GS : KS;
  constexpr int NGS = GSZ < KS ? KS / GSZ : 1;  // groups touched per stage
  constexpr float CB = OpBias<W_BIT, XDT>::value;
  constexpr uint32_t ZSYM = W_BIT == 4 ? 0x88888888u : 0xAAAAAAAAu;

  const int lane = threadIdx.x & 63;
  // wave index in an SGPR: the per-wave K range and the stage loop are then
  // scalar (threadIdx.x >> 6 alone is taken as divergent, and the loop would
  // run under an exec mask with its ring registers reused as temporaries)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int S = SPLIT ? splits_of(tile_opts) : 1;
  const int w0 = xcd_remap(blockIdx.x, gridDim.x);
  const int split = SPLIT ? w0 % S : 0;
  const int w = SPLIT ? w0 / S : w0;  // tile
  const int nt = w % n_tiles, mt_idx = w / n_tiles;
  const int m0 = mt_idx * 16 * MT;
  const int strips = N / 16;
  const int s0 = nt * NT;
  const int nblk = K / KB;
  const int nst = (nblk + BLK - 1) / BLK;  // stages along K
  // this workgroup's split of the stages, then this wave's share of it
  const int sper = (nst + S - 1) / S;
  const int sp0 = min(nst, split * sper), sp1 = min(nst, sp0 + sper);
  const int per = (sp1 - sp0 + WAVES - 1) / WAVES;
  const int st0 = min(sp1, sp0 + wave * per);
  const int st1 = min(sp1, st0 + per);

  // x of a stage arrives as whole rows (CH 16-byte chunks of a row per
  // stage, 64 / CH rows per load: a fragment-order load would touch 16 rows
  // x 64 bytes, which the memory pipeline serves at well under half the
  // rate) and is turned into A-operand fragments through a per-wave LDS
  // tile of 16 rows x CH chunks; chunk c of row r sits at slot CH r + (c ^ r),
  // so both the row-wise writes and the fragment reads (16 rows, one chunk
  // each) hit 16 distinct bank groups.  A wave's LDS operations run in
  // order, so the tile needs no barrier between stages.  The reduction of
  // the waves' partial tiles reuses the same LDS after the K loop.
  constexpr int CH = KS / 8, RPL = 64 / CH;
  constexpr int ROWS = 16 * MT, COLS = 16 * NT;
  constexpr size_t XT_BYTES = (size_t)WAVES * MT * 16 * CH * 16;
  constexpr size_t RED_BYTES = (size_t)WAVES * ROWS * (COLS + 1) * 4;
  static_assert(XT_BYTES <= 160 * 1024 && RED_BYTES <= 96 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) unsigned char smem[XT_BYTES > RED_BYTES ? XT_BYTES : RED_BYTES];
  u32x4_t* const xt = reinterpret_cast<u32x4_t*>(smem);
  auto xswz = [](int r, int c) { return CH * r + (c ^ r); };

  // One stage in registers: weight slots, x rows, and the
  // scales / zero words of the groups the stage touches.
  struct StageRegs {
    u32x4_t w[NT][BLK];
    u32x4_t a[MT][STEPS];
    uint32_t sc[NT][NGS];
    uint32_t zw[NT];
  };
  // Stage loads are buffer loads through descriptors based at this
  // workgroup's strips, rows and columns: offsets stay within 32 bits (the
  // host refuses K >= 2^24 and scale tables of 2^30 entries or more), and a
  // strip or row past the edge reads zeros (the hardware range check)
  // instead of needing a clamped index.  They are
  // intrinsic calls, so the compiler keeps each one where it is written: a
  // plain load that is only used after the loop's back edge gets moved down
  // to its use, which empties the ring.  Raw values go into the ring; every
  // conversion happens where the value is used.
  const int strips_here = min(NT, strips - s0);
  const int rows_here = min(16 * MT, M - m0);
  const buf_t qbuf = make_buf(Qt + (size_t)s0 * nblk * 64, (uint32_t)strips_here * nblk * 1024u);
  const buf_t xbuf = make_buf(x + (size_t)m0 * K, (uint32_t)rows_here * K * 2u);
  const uint16_t* s16 = reinterpret_cast<const uint16_t*>(scales);
  const int G = LOWBIT && gmask != 0 ? K / GS : 1;  // scale rows (per-column: one)
  const buf_t sbuf = make_buf(s16 + 16 * s0, LOWBIT ? (uint32_t)((size_t)G * N - 16 * s0) * 2u : 0u);
  const bool zp = qz != nullptr;
  const int zrows = (G + PACK - 1) / PACK;
  const buf_t zbuf = make_buf(zp ? qz + 16 * s0 : reinterpret_cast<const uint32_t*>(Qt),
                              zp ? (uint32_t)((size_t)zrows * N - 16 * s0) * 4u : 0u);
  auto load_stage = [&](int st, StageRegs& R) {
#pragma unroll
    for (int s = 0; s < NT; ++s)
#pragma unroll
      for (int b = 0; b < BLK; ++b) {
        const int kb = min(st * BLK + b, nblk - 1);
        R.w[s][b] = buf_load128(qbuf, ((s * nblk + kb) * 64 + lane) * 16);
      }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int k = 0; k < STEPS; ++k) {
        // contiguous rows: load k of row tile i is rows RPL k .. RPL k +
        // RPL - 1, 16-byte chunk lane % CH of each row's stage.  (int8: a
        // stage past the last 64-deep block reads the next row or zeros into
        // its upper chunks, which only the skipped k steps would use.)
        const int row = 16 * i + RPL * k + lane / CH;
        R.a[i][k] = buf_load128(xbuf, (row * K + st * KS + 8 * (lane % CH)) * 2);
      }
    if constexpr (LOWBIT) {
      const int g0 = (st * KS) / GS;
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        const int nl = 16 * s + l16;  // column within the workgroup's strips
#pragma unroll
        for (int q = 0; q < NGS; ++q)
          R.sc[s][q] = buf_load16(sbuf, (((g0 + q) & gmask) * N + nl) * 2);
        R.zw[s] = buf_load32(zbuf, (((g0 & gmask) / PACK) * N + nl) * 4);
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

  auto compute_stage = [&](int st, const StageRegs& R, bool last) {
    // x through the wave's LDS tile: rows in, A-operand fragments out
    u32x4_t af[MT][STEPS];
    u32x4_t* xw = xt + (size_t)wave * MT * 16 * CH;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int k = 0; k < STEPS; ++k)
        xw[i * 16 * CH + xswz(RPL * k + lane / CH, lane % CH)] = R.a[i][k];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int k = 0; k < STEPS; ++k) af[i][k] = xw[i * 16 * CH + xswz(l16, 4 * k + quad)];
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      if (!LOWBIT && st * KS + 32 * k >= K) break;  // int8: half stage past K
#pragma unroll
      for (int i = 0; i < MT; ++i) xs[i] = mfma16<XDT>(af[i][k], ones, xs[i]);
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        const u32x4_t b = bfrag<W_BIT, XDT>(R.w[s], k);
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i][s] = mfma16<XDT>(af[i][k], b, acc[i][s]);
      }
      if constexpr (LOWBIT) {
        const int kend = st * KS + 32 * (k + 1);  // one past this step
        if (kend % GS == 0 || (k == STEPS - 1 && last)) {
          const int q = GS < KS ? (32 * k) / GS : 0;
          const int g = ((st * KS) / GS + q) & gmask;
          float sc[NT], bz[NT];
#pragma unroll
          for (int s = 0; s < NT; ++s) {
            sc[s] = f16_bits_to_f32((uint16_t)R.sc[s][q]);
            const uint32_t zw = zp ? R.zw[s] : ZSYM;
            bz[s] = CB + (float)((zw >> ((g % PACK) * W_BIT)) & ((1u << W_BIT) - 1u));
          }
          flush(sc, bz);
        }
      }
    }
  };

  // DEPTH-deep ring of stages in registers: stage st + DEPTH is requested
  // while stage st computes (loads past the range re-read its last stage)
  if (st0 < st1) {
    StageRegs ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load_stage(min(st0 + d, st1 - 1), ring[d]);
      // issue order = ring order, as in the loop: the wait at the loop head
      // then only needs this slot's loads, not the later slots'
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int st = st0; st < st1; st += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (st + d < st1) compute_stage(st + d, ring[d], st + d == st1 - 1);
        load_stage(min(st + d + DEPTH, st1 - 1), ring[d]);  // on every path
      }
    }
  }
  if constexpr (!LOWBIT) {
    float sc[NT], bz[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      sc[s] = reinterpret_cast<const float*>(scales)[16 * min(s0 + s, strips - 1) + l16];
      bz[s] = CB;
    }
    flush(sc, bz);
  }

  // ---- the waves' K ranges meet in LDS (over the x tiles: wait for all) ---
  __syncthreads();
  float (*red)[ROWS][COLS + 1] = reinterpret_cast<float (*)[ROWS][COLS + 1]>(smem);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][16 * i + 4 * quad + r][16 * s + l16] = yacc[i][s][r];
  __syncthreads();
  if constexpr (!SPLIT) {
    with_y(y, ydt, [&](auto* yt) {
      using T = typename std::remove_pointer<decltype(yt)>::type;
      for (int o = threadIdx.x; o < ROWS * COLS; o += 64 * WAVES) {
        const int rr = o / COLS, cc = o % COLS;
        const int m = m0 + rr, n = 16 * s0 + cc;
        if (m < M && n < N) {
          float sum = 0.f;
#pragma unroll
          for (int v = 0; v < WAVES; ++v) sum += red[v][rr][cc];
          yt[(size_t)m * N + n] = (T)sum;
        }
      }
    });
  } else {
    // Workspace: one ticket per tile (zero between calls), padded to 256
    // bytes, then S partial tiles of ROWS x COLS fp32 per tile.  The partial
    // goes out with coherent stores; once they have completed (vmcnt 0 in
    // every wave, then the barrier) one lane takes the tile's ticket.  The
    // ticket is an agent-scope atomic, so whichever workgroup draws S - 1 is
    // the last, and every other partial of its tile is already past the L2s;
    // it re-arms the ticket and reads the S partials back with coherent
    // loads.  Nobody waits on anybody: the workgroups that are not last end.
    const int tiles = gridDim.x / S;
    uint32_t* tickets = ws;
    float* parts = reinterpret_cast<float*>(ws + ((tiles + 63) & ~63));
    constexpr int PART = ROWS * COLS;  // floats per partial
    const buf_t pbuf = make_buf(parts + (size_t)w * S * PART, (uint32_t)S * PART * 4u);
    for (int o = 4 * threadIdx.x; o < PART; o += 4 * 64 * WAVES) {
      const int rr = o / COLS, cc = o % COLS;  // 4 columns of one row (COLS % 16 == 0)
      u32x4_t v;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) sum += red[q][rr][cc + c];
        v[c] = __builtin_bit_cast(uint32_t, sum);
      }
      buf_store128_coherent(v, pbuf, (split * PART + o) * 4);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t ticket =
          __hip_atomic_fetch_add(tickets + w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = ticket == (uint32_t)(S - 1);
      if (last) __hip_atomic_store(tickets + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    with_y(y, ydt, [&](auto* yt) {
      using T = typename std::remove_pointer<decltype(yt)>::type;
      for (int o = 4 * threadIdx.x; o < PART; o += 4 * 64 * WAVES) {
        f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < S; ++q)
          sum += __builtin_bit_cast(f32x4_t, buf_load128_coherent(pbuf, (q * PART + o) * 4));
        const int rr = o / COLS, cc = o % COLS;
        const int m = m0 + rr, n = 16 * s0 + cc;
        if (m < M && n < N) {
#pragma unroll
          for (int c = 0; c < 4; ++c) yt[(size_t)m * N + n + c] = (T)sum[c];
        }
      }
    });
  }
}

template <int W_BIT, int XDT, int GS, int MT, int NT, int DEPTH, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const void* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int M, int N, int K, int tile_opts) {
  skinny_body<W_BIT, XDT, GS, MT, NT, DEPTH, WAVES, false>(x, Qt, scales, qz, y, nullptr, M, N,
                                                           K, tile_opts);
}

template <int W_BIT, int XDT, int GS, int MT, int NT, int DEPTH, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_split_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const void* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    uint32_t* __restrict__ ws, int M, int N, int K, int tile_opts) {
  skinny_body<W_BIT, XDT, GS, MT, NT, DEPTH, WAVES, true>(x, Qt, scales, qz, y, ws, M, N, K,
                                                          tile_opts);
}

// ---------------------------------------------------------------------------
// Large-M kernel (prefill), matrix-core bound.
//  * workgroup tile 256 x 256, 4 waves side by side along N: a wave owns all
//    256 rows x 4 strips (64 columns) = 16 x 4 MFMA tiles, 256 fp32
//    accumulators per lane (the matrix-core register file);
//  * weights: each wave streams its own 4 strips straight from the tile
//    layout into B operands (no LDS, no duplication across waves) and
//    dequantizes them to the MFMA's 16-bit type: w = (q - z) * s is formed
//    exactly in fp32 (a 4-bit by 11-bit product) and rounded once to
//    fp16 / bf16 (round to nearest even);
//  * x: the 256 x 128 tile of a stage is shared by the 4 waves through
//    double-buffered LDS, stored fragment-major (16 rows x 32 k = one 1 KiB
//    block in MFMA A-operand lane order), so every operand read is one
//    conflict-free ds_read_b128;
//  * stage s + 1's x tile and weight slots are loaded while stage s runs.
template <int XDT> struct WType;
template <> struct WType<XF16> {
  // (a, b) fp32 -> packed fp16 pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
};
template <> struct WType<XBF16> {
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    bf16x2_t h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
};

// B operand (8 dequantized weights of one column) for k step `st` of a
// 128-deep stage: int4 word st of the slot; int2 word st / 2, k half st % 2.
// sc = scale, zs = z * scale of the step's group: w = q * s - z * s, exact.
template <int W_BIT, int XDT>
__device__ __forceinline__ u32x4_t bfrag_scaled(const u32x4_t& slot, int st, float sc, float zs) {
  float f[8];
  if constexpr (W_BIT == 4) {
    const uint32_t w = slot[st];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int field = (i & 1) ? 4 + (i >> 1) : (i >> 1);
      f[i] = (float)((w >> (4 * field)) & 0xFu);
    }
  } else {
    const uint32_t w = slot[st >> 1];
    const int h = st & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int field = (i & 1) ? 8 + 4 * h + (i >> 1) : 4 * h + (i >> 1);
      f[i] = (float)((w >> (2 * field)) & 0x3u);
    }
  }
  u32x4_t b;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    b[t] = WType<XDT>::pack(__builtin_fmaf(f[2 * t], sc, -zs), __builtin_fmaf(f[2 * t + 1], sc, -zs));
  return b;
}

// MFMA whose accumulator is pinned to the matrix-core (AGPR) registers: the
// large-M kernel keeps 256 accumulators per lane live across its K loop,
// and without the pin the register allocator shuttles them between register
// files every iteration.  Independent MFMAs sit between two uses of the same
// accumulator, so no extra wait states are needed inside the loop.
template <int XDT> __device__ __forceinline__ void mfma16_acc(f32x4_t& c, const u32x4_t& a,
                                                             const u32x4_t& b);
template <> __device__ __forceinline__ void mfma16_acc<XF16>(f32x4_t& c, const u32x4_t& a,
                                                            const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <> __device__ __forceinline__ void mfma16_acc<XBF16>(f32x4_t& c, const u32x4_t& a,
                                                             const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// 16-row tiles per workgroup in the large-M kernel (256 rows: one wave per
// SIMD, 256 fp32 accumulators per lane).
constexpr int kLargeMT = 16;
// eighths of a stage's row tiles over which its loads are issued
constexpr int kLoadSpan = 4;

// s_waitcnt with vmcnt = 0 and the other counters at their maximum.
static constexpr int kWaitVm0 = 0x0F70;

// Operand register t (k = 2t, 2t + 1 of one column) of a pre-scaled B
// fragment: W = (q - z) * s rounded once to the MFMA's 16-bit type.
// The two codes are masked into the mantissa of fp16 1024 (exact: 1024 + q),
// then
//   bf16: v_fma_mix_f32 forms (1024 + q) * s - (1024 + z) * s in fp32 --
//         both products fit 22 bits and their difference (q - z) * s is
//         representable, so the fused result is exact -- and
//         v_cvt_pk_bf16_f32 rounds the pair to nearest even;
//   fp16: v_pk_add_f16 gives q - z exactly, v_pk_mul_f16 rounds (q - z) * s
//         once to nearest even.
// int4: word bits (4t, 16 + 4t) hold fields (t, 4 + t); int2: word bits
// (2(4h + t), 16 + 2(4h + t)) hold fields (4h + t, 8 + 4h + t).
struct GroupConst {
  float s;          // scale
  float zb_s;       // (1024 + z) * s
  float s16;        // s / 16            (int4 bf16: odd fields, read as 1024 + 16 q)
  float zb16_s;     // (64 + z) * s
  uint32_t s_h2;    // scale as an fp16 pair
  uint32_t nzb_h2;  // -(1024 + z) as an fp16 pair
};

template <int W_BIT, int XDT>
__device__ __forceinline__ uint32_t bpair_scaled(uint32_t w, int h, int t, const GroupConst& g,
                                              uint32_t hi_bits) {
  if constexpr (W_BIT == 4 && XDT == XBF16) {
    // Fields t = 1, 3 are taken where they sit, at bits 4-7 of each half:
    // OR-ed under the fp16 1024 pattern they read 1024 + 16 q, and
    // (1024 + 16 q) * s / 16 - (64 + z) * s = (q - z) * s, still exact in
    // fp32 (11-bit by 11-bit products, power-of-two scaling).  One shift
    // by 8 serves fields 2 and 3, so a word costs one shift and four
    // mask-ors instead of three shifts.  Same bits out as the plain path.
    const uint32_t v = t >= 2 ? w >> 8 : w;
    const uint32_t m = (v & ((t & 1) ? 0x00F000F0u : 0x000F000Fu)) | hi_bits;
    const half2_t mh = __builtin_bit_cast(half2_t, m);
    const float sc = (t & 1) ? g.s16 : g.s;
    const float zb = (t & 1) ? g.zb16_s : g.zb_s;
    const float lo = __builtin_fmaf((float)mh[0], sc, -zb);
    const float hi = __builtin_fmaf((float)mh[1], sc, -zb);
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  constexpr uint32_t FIELD2 = W_BIT == 4 ? 0x000F000Fu : 0x00030003u;
  const int sh = W_BIT == 4 ? 4 * t : 2 * (4 * h + t);
  const uint32_t m = ((w >> sh) & FIELD2) | hi_bits;
  const half2_t mh = __builtin_bit_cast(half2_t, m);
  if constexpr (XDT == XBF16) {
    const float lo = __builtin_fmaf((float)mh[0], g.s, -g.zb_s);
    const float hi = __builtin_fmaf((float)mh[1], g.s, -g.zb_s);
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  } else {
    const half2_t d = mh + __builtin_bit_cast(half2_t, g.nzb_h2);
    return __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(half2_t, g.s_h2));
  }
}

// Inputs of one operand register (the bpair_scaled recipes).  bf16: the word
// shifted so that its two codes sit under `mask`, and the fp32 scale and
// bias product that turn the fp16 1024 + c (or 1024 + 16 c) into (c - z) * s.
//   fp16: the word shifted to its two codes, and the pairs -(1024 + z) and
//   s (v_pk_add_f16 then v_pk_mul_f16, the bpair_scaled fp16 recipe).
struct BSrc {
  uint32_t v, mask;
  uint32_t p, q;  // bf16: scale and bias product (fp32 bits); fp16: -(1024 + z) and s pairs
};
template <int W_BIT, int XDT>
__device__ __forceinline__ BSrc bsrc(uint32_t w, int h, int t, const GroupConst& g) {
  if constexpr (XDT == XBF16) {
    if constexpr (W_BIT == 4) {
      const float sc = (t & 1) ? g.s16 : g.s, zb = (t & 1) ? g.zb16_s : g.zb_s;
      return {t >= 2 ? w >> 8 : w, (t & 1) ? 0x00F000F0u : 0x000F000Fu,
              __builtin_bit_cast(uint32_t, sc), __builtin_bit_cast(uint32_t, zb)};
    } else {
      return {w >> (2 * (4 * h + t)), 0x00030003u, __builtin_bit_cast(uint32_t, g.s),
              __builtin_bit_cast(uint32_t, g.zb_s)};
    }
  } else {
    if constexpr (W_BIT == 4) return {w >> (4 * t), 0x000F000Fu, g.nzb_h2, g.s_h2};
    else return {w >> (2 * (4 * h + t)), 0x00030003u, g.nzb_h2, g.s_h2};
  }
}

// The NT MFMAs of one row tile (bf16) with one operand register of a later
// k step made between them: mask-or, the two mixed-precision FMAs, the
// rounding to a bf16 pair -- each issues while an MFMA runs instead of
// waiting behind the row tile's MFMAs.  One asm block, because the
// scheduler does not see the accumulator-pinned MFMAs as MFMAs.  No
// hazards inside: the conversion writes only its own (early-clobber)
// registers, none of which an MFMA here reads.
__device__ __forceinline__ uint32_t mfma_row_deq(f32x4_t (&c)[4], const u32x4_t& a,
                                                 const u32x4_t (&b)[4], const BSrc& src,
                                                 uint32_t hi_bits) {
  uint32_t out, m;
  float lo, up;
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_or_b32 %[m], %[v], %[mask], %[hi]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_fma_mix_f32 %[lo], %[m], %[sc], -%[zb] op_sel_hi:[1,0,0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c2], %[a], %[b2], %[c2]\n\t"
      "v_fma_mix_f32 %[up], %[m], %[sc], -%[zb] op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c3], %[a], %[b3], %[c3]\n\t"
      "v_cvt_pk_bf16_f32 %[out], %[lo], %[up]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [out] "=&v"(out),
        [m] "=&v"(m), [lo] "=&v"(lo), [up] "=&v"(up)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]),
        [v] "v"(src.v), [mask] "s"(src.mask), [hi] "v"(hi_bits), [sc] "v"(src.p),
        [zb] "v"(src.q));
  return out;
}
__device__ __forceinline__ uint32_t mfma_row_deq(f32x4_t (&c)[3], const u32x4_t& a,
                                                 const u32x4_t (&b)[3], const BSrc& src,
                                                 uint32_t hi_bits) {
  uint32_t out, m;
  float lo, up;
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_or_b32 %[m], %[v], %[mask], %[hi]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_fma_mix_f32 %[lo], %[m], %[sc], -%[zb] op_sel_hi:[1,0,0]\n\t"
      "v_mfma_f32_16x16x32_bf16 %[c2], %[a], %[b2], %[c2]\n\t"
      "v_fma_mix_f32 %[up], %[m], %[sc], -%[zb] op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_cvt_pk_bf16_f32 %[out], %[lo], %[up]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [out] "=&v"(out), [m] "=&v"(m),
        [lo] "=&v"(lo), [up] "=&v"(up)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [v] "v"(src.v),
        [mask] "s"(src.mask), [hi] "v"(hi_bits), [sc] "v"(src.p), [zb] "v"(src.q));
  return out;
}

// fp16: mask-or, (1024 + q) - (1024 + z) exact, times s rounded once.
__device__ __forceinline__ uint32_t mfma_row_deq_f16(f32x4_t (&c)[4], const u32x4_t& a,
                                                     const u32x4_t (&b)[4], const BSrc& src,
                                                     uint32_t hi_bits) {
  uint32_t out, m, d;
  asm volatile(
      "v_mfma_f32_16x16x32_f16 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_or_b32 %[m], %[v], %[mask], %[hi]\n\t"
      "v_mfma_f32_16x16x32_f16 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_pk_add_f16 %[d], %[m], %[nz]\n\t"
      "v_mfma_f32_16x16x32_f16 %[c2], %[a], %[b2], %[c2]\n\t"
      "v_pk_mul_f16 %[out], %[d], %[sh]\n\t"
      "v_mfma_f32_16x16x32_f16 %[c3], %[a], %[b3], %[c3]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [out] "=&v"(out),
        [m] "=&v"(m), [d] "=&v"(d)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]),
        [v] "v"(src.v), [mask] "s"(src.mask), [hi] "v"(hi_bits), [nz] "v"(src.p),
        [sh] "v"(src.q));
  return out;
}
__device__ __forceinline__ uint32_t mfma_row_deq_f16(f32x4_t (&c)[3], const u32x4_t& a,
                                                     const u32x4_t (&b)[3], const BSrc& src,
                                                     uint32_t hi_bits) {
  uint32_t out, m, d;
  asm volatile(
      "v_mfma_f32_16x16x32_f16 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_or_b32 %[m], %[v], %[mask], %[hi]\n\t"
      "v_mfma_f32_16x16x32_f16 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_pk_add_f16 %[d], %[m], %[nz]\n\t"
      "v_mfma_f32_16x16x32_f16 %[c2], %[a], %[b2], %[c2]\n\t"
      "v_pk_mul_f16 %[out], %[d], %[sh]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [out] "=&v"(out), [m] "=&v"(m),
        [d] "=&v"(d)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [v] "v"(src.v),
        [mask] "s"(src.mask), [hi] "v"(hi_bits), [nz] "v"(src.p), [sh] "v"(src.q));
  return out;
}

template <int W_BIT, int XDT, int GS, bool ZP, int NT>
__global__ __launch_bounds__(256, 1) void gemm_large_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int M, int N, int K, int tile_opts, int strip0) {
  const int n_tiles = tiles_of(tile_opts), ydt = ydt_of(tile_opts), gmask = gmask_of(tile_opts);
  constexpr int MT = kLargeMT;          // 16-row tiles per workgroup
  constexpr int BM = 16 * MT;           // rows per workgroup
  constexpr int KS = 128;               // k per stage
  constexpr int STEPS = KS / 32;        // MFMA k steps per stage
  constexpr int KB = W_BIT == 4 ? 128 : 256;  // layout block depth
  constexpr int FRAGS = MT * STEPS;     // 1 KiB A fragments per stage
  constexpr int PACK = 32 / W_BIT;
  constexpr int NGS = GS < KS ? KS / GS : 1;  // groups per stage
  // symmetric zero 2^(w_bit-1) in every field of a word
  constexpr uint32_t ZSYM = W_BIT == 4 ? 0x88888888u : 0xAAAAAAAAu;

  __shared__ u32x4_t xa[2][FRAGS * 64];

  // fp16 1024 in both halves, held in a register: mask-and-or of the codes
  // is then one v_and_or_b32 (an instruction takes one literal at most)
  uint32_t hi_bits;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(hi_bits));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = w % n_tiles, mt_idx = w / n_tiles;
  const int m0 = mt_idx * BM;
  const int strips = N / 16;
  const int s0 = strip0 + (nt * 4 + wave) * NT;  // this wave's first strip
  const int nblk = K / KB;
  const int nst = K / KS;

  // Every load goes through a buffer descriptor whose range ends where the
  // operand does: rows past M and strips past N read zeros (they only feed
  // outputs that are never stored), and each address is a per-lane offset
  // fixed for the whole K loop plus a wave-uniform offset for the stage.
  //   x: the workgroup's rows; weights: the wave's strips (1 KiB blocks,
  //   strip-major); scales / zero words: from the wave's first column on.
  const int sc0 = min(s0, strips);
  const int nvalid = min(NT, strips - sc0);
  const int G = gmask != 0 ? K / GS : 1;
  const buf_t xb = make_buf(x + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K * 2));
  const buf_t qb = make_buf(Qt + (size_t)sc0 * nblk * 64, (uint32_t)(nvalid * nblk * 1024));
  const buf_t sb = make_buf(scales + 16 * sc0, (uint32_t)(((size_t)G * N - 16 * sc0) * 2));
  const buf_t zb = make_buf(qz + 16 * sc0,
                            ZP ? (uint32_t)(((size_t)((G + PACK - 1) / PACK) * N - 16 * sc0) * 4)
                               : 0u);

  // The x tile of a stage is stored by row tile: 16 rows x 16 chunks of 16
  // bytes (the stage's 128 k of a row), chunk c of row r at slot 16 r +
  // (c ^ r).  Load unit f (1 KiB, row tile f / 4) fills slots 64 (f % 4) ..
  // + 63 of its tile: lane p's 16 bytes land at slot 64 (f % 4) + p, i.e.
  // row r = 4 (f % 4) + p / 16, position p % 16 -- so lane p fetches chunk
  // (p % 16) ^ r of that row, and one load reads 4 whole rows (256
  // contiguous bytes each; the fragment-order alternative, 16 rows x 64
  // bytes per load, is served at well under half the rate).  A fragment
  // (row l16, chunk 4 kk + quad) is then one conflict-free ds_read_b128.
  // Each wave moves FRAGS / 4 units straight from memory into LDS (buffer
  // loads to LDS: the destination is a wave-uniform LDS address, lane p
  // writing 16 bytes at + 16 p).
  static_assert(KS == 128 && STEPS == 4, "x tile layout: 16 chunks per row, 4 loads per row tile");
  static_assert(MT % 4 == 0, "a wave's load units cover whole row-tile quarters");
  int xo[4];  // lane byte offset for units with f % 4 = c
#pragma unroll
  for (int c = 0; c < 4; ++c) xo[c] = (quad * K + 8 * (l16 ^ (4 * c + quad))) * 2;
  auto x_unit = [&](int j, int sx, int buf) {
    const int f = wave * (FRAGS / 4) + j;
    const int row = 16 * (f / 4) + 4 * (j % 4);  // first of the unit's 4 rows
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xb, (__attribute__((address_space(3))) void*)(&xa[buf][f * 64]), 16, xo[j % 4],
        (row * K + sx * KS) * 2, 0, 0);
  };
  auto load_x = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < FRAGS / 4; ++j) x_unit(j, st, buf);
  };

  // a stage's words of a strip: int4 the lane's whole 16-byte slot of the
  // 128-deep block; int2 the half (8 bytes) of the 256-deep block's slot
  // that holds the stage's 128 k
  using Slot = typename std::conditional<W_BIT == 4, u32x4_t, u32x2_t>::type;
  struct WRegs {
    Slot slot[NT];
    uint32_t sc[NT][NGS];
    uint32_t zw[NT];
  };
  const int qv = lane * 16, sv = l16 * 2, zv = l16 * 4;
  auto load_slot = [&](int s, int st, WRegs& R) {
    const int kb = (st * KS) / KB;
    if constexpr (W_BIT == 4)
      R.slot[s] = __builtin_amdgcn_raw_buffer_load_b128(qb, qv, (s * nblk + kb) * 1024, 0);
    else
      R.slot[s] = __builtin_amdgcn_raw_buffer_load_b64(qb, qv, (s * nblk + kb) * 1024 + 8 * (st & 1), 0);
  };
  auto load_scale = [&](int s, int q, int st, WRegs& R) {
    const int g = ((st * KS) / GS + q) & gmask;
    R.sc[s][q] = __builtin_amdgcn_raw_buffer_load_b16(sb, sv + 32 * s, g * N * 2, 0);
  };
  auto load_zero = [&](int s, int st, WRegs& R) {
    if constexpr (ZP) {
      const int g = ((st * KS) / GS) & gmask;
      R.zw[s] = __builtin_amdgcn_raw_buffer_load_b32(zb, zv + 64 * s, (g / PACK) * N * 4, 0);
    } else {
      R.zw[s] = ZSYM;
    }
  };
  auto load_w = [&](int st, WRegs& R) {
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      load_slot(s, st, R);
#pragma unroll
      for (int q = 0; q < NGS; ++q) load_scale(s, q, st, R);
      load_zero(s, st, R);
    }
  };
  // Loads issued during a stage, one at a time: j < NWL are weight-side
  // (slots, then scales, then zero words) of stage sw, the rest this wave's
  // x fragments of stage sx.  The k loop issues them spread over its first
  // row tiles: a wave issues in order, so a burst of loads at the top of a
  // stage would hold its MFMAs back until the memory pipeline had taken
  // them all; what is issued late in the stage has little time left to land
  // before the stage's closing wait.
  constexpr int NWL = NT * (2 + NGS);
  constexpr int NLD = NWL + FRAGS / 4;
  auto load_part = [&](int j, int sw, int sx, int buf, WRegs& R) {
    if (j < NT) load_slot(j, sw, R);
    else if (j < NT + NT * NGS) load_scale((j - NT) / NGS, (j - NT) % NGS, sw, R);
    else if (j < NWL) load_zero(j - NT - NT * NGS, sw, R);
    else x_unit(j - NWL, sx, buf);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) acc[i][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // dequant constants of strip s for each group of the stage at K position
  // sa, from that stage's scale and zero words
  auto group_consts = [&](const WRegs& R, int sa, int s, GroupConst (&g)[NGS]) {
    const int g0 = (sa * KS) / GS;
#pragma unroll
    for (int q = 0; q < NGS; ++q) {
      const uint32_t sbits = R.sc[s][q] & 0xFFFFu;
      const float sc = f16_bits_to_f32((uint16_t)sbits);
      const uint32_t z = (R.zw[s] >> ((((g0 + q) & gmask) % PACK) * W_BIT)) & ((1u << W_BIT) - 1u);
      const float zbias = 1024.0f + (float)z;
      g[q].s = sc;
      g[q].zb_s = zbias * sc;
      g[q].s16 = sc * 0.0625f;
      g[q].zb16_s = (64.0f + (float)z) * sc;
      g[q].s_h2 = sbits | (sbits << 16);
      const uint32_t nzb = __builtin_bit_cast(uint16_t, (_Float16)(-zbias));
      g[q].nzb_h2 = nzb | (nzb << 16);
    }
  };
  // layout word of k step kk of a stage (int4: one word per step; int2: one
  // per two steps, the stage being half `sub` of a 256-deep block)
  auto word_of = [&](const WRegs& R, int s, int sub, int kk) {
    (void)sub;
    return W_BIT == 4 ? R.slot[s][kk] : R.slot[s][kk >> 1];
  };

  // Weight registers of three stages: the current one, the next (loaded
  // during the previous stage) and the one after (loading now).  The x
  // tile of the next stage goes straight to LDS, and while such a load is
  // in flight the compiler can only wait for every earlier load (vmcnt 0):
  // loading weights two stages ahead lets the last k step read the next
  // stage's weights, complete since the previous stage's closing wait.
  WRegs cur, nx1, nx2;
  load_x(0, 0);
  load_w(0, cur);
  load_w(min(1, nst - 1), nx1);
  // pin the loads above the wait (the compiler may otherwise sink them
  // into the loop preheader, where they would still be in flight)
  auto pin = [](const WRegs& R) {
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      asm volatile("" ::"v"(R.slot[s]), "v"(R.zw[s]));
#pragma unroll
      for (int q = 0; q < NGS; ++q) asm volatile("" ::"v"(R.sc[s][q]));
    }
  };
  pin(cur);
  pin(nx1);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  // The first stage's group constants and first B fragment are made here;
  // from then on each stage makes the next one's during its last k step,
  // so a stage opens straight into its MFMAs.
  GroupConst gc[NT][NGS];
  u32x4_t b[NT], bn[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    group_consts(cur, 0, s, gc[s]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      b[s][t] = bpair_scaled<W_BIT, XDT>(word_of(cur, s, 0, 0), 0, t, gc[s][0], hi_bits);
  }
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const int sub = W_BIT == 2 ? (st & 1) : 0;  // int2: which half of the 256-deep block
    // the next stage, loaded during this one (the last iteration re-reads
    // the final stage into the idle buffer, keeping the loop free of
    // branches)
    const int stn = min(st + 1, nst - 1);
    const int stw = min(st + 2, nst - 1);  // weights loaded now
    const int subn = W_BIT == 2 ? (stn & 1) : 0;
    const u32x4_t* xs_buf = &xa[buf][0];

    // Software pipeline inside the stage: while the NT MFMAs of row tile i of
    // k step k run, (1) the A fragment two tiles ahead is read from LDS,
    // (2) part of the next k step's B fragments is dequantized (the NT x 4
    // operand registers spread over the MT row tiles) -- in the last k step
    // those of the next stage, after its group constants -- and (3) part of
    // the next stage's loads is issued.  The scheduling barriers hold this
    // interleave; without them the compiler hoists every read and every
    // conversion (and spills).
    // fragment (row tile i, k step kk) = slot 256 i + 16 l16 + ((4 kk + quad) ^ l16)
    auto afrag = [&](int i, int kk) { return xs_buf[256 * i + 16 * l16 + ((4 * kk + quad) ^ l16)]; };
    u32x4_t a0 = afrag(0, 0);
    u32x4_t a1 = afrag(1, 0);
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      const int kn = k + 1;
      const int qn = GS < KS ? (32 * kn) / GS : 0;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int t2 = k * MT + i + 2;  // fragment two ahead, in (k, i) order
        u32x4_t an = a1;
        if (t2 < STEPS * MT) an = afrag(t2 % MT, t2 / MT);
        // this row tile's operand register of the next k step (of the next
        // stage in the last k step), made between its MFMAs
        const int r0 = i * NT * 4 / MT, r1 = (i + 1) * NT * 4 / MT;
        static_assert(NT * 4 <= MT, "one operand register per row tile at most");
        // (the last k step makes the next stage's group constants in place:
        // this stage's are no longer read by then)
        if (kn == STEPS && i < NT) group_consts(nx1, stn, i, gc[i]);
        if (r0 < r1) {
          const int r = r0;
          const BSrc src =
              kn < STEPS ? bsrc<W_BIT, XDT>(word_of(cur, r / 4, sub, kn), (STEPS * sub + kn) & 1,
                                            r % 4, gc[r / 4][qn])
                         : bsrc<W_BIT, XDT>(word_of(nx1, r / 4, subn, 0), (STEPS * subn) & 1,
                                            r % 4, gc[r / 4][0]);
          if constexpr (XDT == XBF16) bn[r / 4][r % 4] = mfma_row_deq(acc[i], a0, b, src, hi_bits);
          else bn[r / 4][r % 4] = mfma_row_deq_f16(acc[i], a0, b, src, hi_bits);
        } else {
#pragma unroll
          for (int s = 0; s < NT; ++s) mfma16_acc<XDT>(acc[i][s], a0, b[s]);
        }
        // this row tile's share of the loads, spread over the first
        // kLoadSpan eighths of the row tiles
        {
          constexpr int SPAN = kLoadSpan * STEPS * MT / 8;
          static_assert(NLD <= 2 * SPAN, "two loads per row tile at most");
          const int p = k * MT + i;
          const int j0 = (p * NLD + SPAN - 1) / SPAN;
          const int j1 = min(NLD, ((p + 1) * NLD + SPAN - 1) / SPAN);
          if (j0 < j1) load_part(j0, stw, stn, buf ^ 1, nx2);
          if (j0 + 1 < j1) load_part(j0 + 1, stw, stn, buf ^ 1, nx2);
        }
        a0 = a1;
        a1 = an;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) b[s] = bn[s];
    }
    cur = nx1;
    nx1 = nx2;
    // the next stage's x tile was written to LDS by the memory pipeline:
    // wait for this wave's loads, then for every wave's
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
  // the accumulators were last written by MFMAs the compiler does not see
  // as such: give them their result latency before they are read.  Each
  // accumulator then passes through an empty asm ordered after the wait, so
  // no read of it can be moved above the wait (they are register reads,
  // which the wait's memory clobber alone does not hold back).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) asm volatile("" : "+a"(acc[i][s]));
  __builtin_amdgcn_sched_barrier(0);

  // y goes out through LDS, one 16-row tile at a time: the wave's 16 x 16 NT
  // block is written row-major into its own LDS region (row stride 68
  // floats: both the column-wise writes and the row-wise reads hit 64
  // distinct banks), then read back so that each store instruction covers
  // 4 whole rows of the block (16 lanes x 4 columns per row) with 16-byte
  // (fp32) or 8-byte (16-bit) stores: every row segment leaves as whole
  // 128-byte lines (direct stores from
  // the accumulator layout write 64-byte halves, measured 1.27x the
  // output's bytes in HBM writes).  The x buffers are free: the K loop
  // ended with a barrier.  A wave's LDS operations run in order, so the
  // region needs no barrier between tiles.
  float* const yl = reinterpret_cast<float*>(&xa[0][0]) + wave * (16 * 68);
  const int prow = lane >> 4, pcol = 4 * (lane & 15);  // row within 4, first column
  const bool pcol_ok = (lane & 15) < 4 * NT && s0 + ((lane & 15) >> 2) < strips;
  with_y(y, ydt, [&](auto* yt) {
    using T = typename std::remove_pointer<decltype(yt)>::type;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int s = 0; s < NT; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) yl[(4 * quad + r) * 68 + 16 * s + l16] = acc[i][s][r];
      f32x4_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = *reinterpret_cast<const f32x4_t*>(yl + (4 * j + prow) * 68 + pcol);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + 16 * i + 4 * j + prow;
        if (m < M && pcol_ok) {
          T* dst = yt + (size_t)m * N + 16 * s0 + pcol;
          if constexpr (std::is_same<T, float>::value) {
            *reinterpret_cast<f32x4_t*>(dst) = v[j];
          } else {
            T t[4] = {(T)v[j][0], (T)v[j][1], (T)v[j][2], (T)v[j][3]};
            *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, t);
          }
        }
      }
    }
  });
}

// ---------------------------------------------------------------- host side
static void skinny_shape(int M, int N, int* mt, int* nt) {
  *mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  // widest strip count (more x reuse per wave) that still leaves about as
  // many workgroups as CUs (measured: 4 strips at N = 14336, 2 at N = 8192)
  const int strips = N / 16;
  *nt = strips / 4 >= 192 ? 4 : (strips / 2 >= 192 ? 2 : 1);
  static const int want = env_int("QMM_SKINNY_NT");
  if (want == 1 || want == 2 || want == 4) *nt = want;
}

// Compute units of the current device (256 on MI355X), read once per device.
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// Large-M column split.  A workgroup (one per CU) takes full tiles of 16
// strips (4 waves x 4) or narrow tiles of 12 strips (4 waves x 3), each over
// all K; the workgroups of one launch run in rounds of `cus`.  Full tiles
// cover the first n_full column tiles, narrow ones the rest, launched after
// them: of the splits, the one with the least estimated time -- rounds of
// full tiles plus rounds of narrow ones, a narrow round costing kNarrowCost
// of a full one (3 of 4 strips' MFMAs; the x tile is loaded whole either
// way).  At M = 4096, N = 11008 (16 x 43 full tiles, 2.69 rounds on 256
// CUs) this gives 2 rounds of full tiles and 1 of narrow ones.
constexpr double kNarrowCost = 0.8;
static void large_split(int m_tiles, int strips, int* n_full, int* n_tail) {
  const long cus = device_cus();
  const int max_full = (strips + 15) / 16;
  auto rounds = [&](long wgs) { return (wgs + cus - 1) / cus; };
  auto tail_of = [&](int f) { return (std::max(0, strips - 16 * f) + 11) / 12; };
  int best = max_full;
  double best_cost = (double)rounds((long)m_tiles * max_full);
  for (int f = max_full - 1; f >= 0; --f) {
    const double c = rounds((long)m_tiles * f) + kNarrowCost * rounds((long)m_tiles * tail_of(f));
    if (c < best_cost - 1e-9) {
      best_cost = c;
      best = f;
    }
  }
  static const int want = env_int("QMM_LARGE_FULL_TILES");
  if (want >= 0) best = std::min(want, max_full);
  *n_full = best;
  *n_tail = tail_of(best);
}

GemmPlan plan_gemm(int M, int N, int K, int w_bit, int group_size, bool with_workspace) {
  GemmPlan p{};
  (void)group_size;
  static const int big = env_int("QMM_GEMM_LARGE_MIN_M");
  if (w_bit != 8 && M > (big > 0 ? big : 64) && K % 128 == 0) {
    p.kind = 1;
    p.mtile = 16 * kLargeMT;
    p.m_tiles = (M + p.mtile - 1) / p.mtile;
    large_split(p.m_tiles, N / 16, &p.n_tiles, &p.tail_tiles);
    p.nt = 16;
    p.waves = 4;
    p.splits = 1;
    p.workspace_bytes = 0;
    return p;
  }
  // Low-bit decode: the VALU GEMV on the tile layout, one strip per
  // workgroup, every wave load 1 KiB of consecutive bytes.  Measured at
  // K=N=4096 (us; this GEMV / the skinny MFMA kernel below): int4 g128 M=1
  // 4.81 / 6.23, M=2 5.38 / 6.25, M=4 6.50 / 6.30; int2 g64 M=1 5.29 / 7.55,
  // M=4 7.08 / 7.57; int4 g32 M=4 8.65 / 7.93.  So M <= 2, and int2 to M=4.
  static const int want_tile = env_int("QMM_GEMV_TILE");
  const bool tile = M <= 2 || (w_bit == 2 && M <= kGemvTileMaxM);
  if (w_bit != 8 && (want_tile > 0 ? M <= kGemvTileMaxM : tile) && want_tile != 0) {
    p.kind = 2;
    p.mtile = M;
    p.n_tiles = N / 16;
    p.m_tiles = 1;
    p.nt = 1;
    p.waves = 4;
    p.splits = 1;
    p.workspace_bytes = 0;
    return p;
  }
  int mt, nt;
  skinny_shape(M, N, &mt, &nt);
  p.kind = 0;
  p.mtile = 16 * mt;
  p.n_tiles = (N / 16 + nt - 1) / nt;
  p.m_tiles = (M + p.mtile - 1) / p.mtile;
  p.nt = nt;
  const long tiles = (long)p.n_tiles * p.m_tiles;
  const int kb = w_bit == 8 ? 128 : mfma_kblock(w_bit);
  const int nst = (K + kb - 1) / kb;
  // Few tiles (small N, long K) leave most CUs idle.  With a workspace, K is
  // split over S workgroups per tile (the last to arrive adds the partials),
  // as many as one round of workgroups holds (tiles * S <= 256), each wave
  // keeping >= 2 stages, and at most 4: every split adds a serial chain to
  // the tile's end (its partial written through to memory, the ticket, the
  // partials read back).  Measured at M=16, K=14336, N=1024 (64 tiles): S = 1
  // 13.4 us, 2 10.4, 3 9.3, 4 9.1, 6 10.6, 8 11.5; at 224 tiles (int8,
  // N=14336) S = 2 is 1.3x slower than none.  Without a workspace, 8 waves
  // per workgroup put twice as much of K in flight and their partial sums
  // still meet in LDS.
  p.splits = 1;
  static const int want_s = env_int("QMM_SKINNY_SPLITS");
  if (with_workspace && tiles <= 128) {
    int s = (int)(256 / tiles);
    if (s > 4) s = 4;
    while (s > 1 && nst / s < 8) --s;  // 4 waves x 2 stages
    p.splits = s;
  }
  if (with_workspace && want_s >= 1 && want_s <= 16) p.splits = want_s;
  const bool w8 = nt == 1 && (mt == 1 || (mt == 2 && w_bit != 2));
  p.waves = (p.splits == 1 && tiles < 128 && w8 && nst >= 16) ? 8 : 4;
  static const int want = env_int("QMM_SKINNY_WAVES");
  if (p.splits == 1 && (want == 4 || (want == 8 && w8))) p.waves = want;
  p.workspace_bytes = 0;
  if (p.splits > 1) {
    const size_t tickets = (size_t)((tiles + 63) & ~63L) * 4;
    p.workspace_bytes = tickets + (size_t)tiles * p.splits * p.mtile * 16 * nt * 4;
  }
  return p;
}

template <int W_BIT, int XDT, int GS, int MT, int NT, int WAVES>
static hipError_t launch_skinny_w(const MatmulArgs& a, const GemmPlan& p) {
  // register budget: 4 waves per SIMD at 16 waves leave 128 registers a lane
  constexpr int DEPTH = MT >= 4 ? 2 : 3;
  const long blocks = (long)p.n_tiles * p.m_tiles;
  if constexpr (WAVES == 4) {
    if (p.splits > 1)
      return launch_kernel(gemm_skinny_split_kernel<W_BIT, XDT, GS, MT, NT, DEPTH, WAVES>,
                           dim3((unsigned)(blocks * p.splits)), dim3(64 * WAVES), a.stream, a.x,
                           a.Q, a.scales, a.zeros, a.y, a.workspace, a.M, a.N, a.K,
                           pack_tiles(p.n_tiles, a.y_dtype, a.group_mask == 0, p.splits));
  }
  return launch_kernel(gemm_skinny_kernel<W_BIT, XDT, GS, MT, NT, DEPTH, WAVES>,
                       dim3((unsigned)blocks), dim3(64 * WAVES), a.stream, a.x, a.Q, a.scales,
                       a.zeros, a.y, a.M, a.N, a.K,
                       pack_tiles(p.n_tiles, a.y_dtype, a.group_mask == 0));
}

template <int W_BIT, int XDT, int GS, int MT, int NT>
static hipError_t launch_skinny(const MatmulArgs& a, const GemmPlan& p) {
  // 8 waves only where the register ring still fits without spilling
  if constexpr (NT == 1 && (MT == 1 || (MT == 2 && W_BIT != 2))) {
    if (p.waves == 8) return launch_skinny_w<W_BIT, XDT, GS, MT, NT, 8>(a, p);
  }
  return launch_skinny_w<W_BIT, XDT, GS, MT, NT, 4>(a, p);
}

template <int W_BIT, int XDT, int GS, int MT>
static hipError_t launch_nt(const MatmulArgs& a, const GemmPlan& p) {
  switch (p.nt) {
    case 1: return launch_skinny<W_BIT, XDT, GS, MT, 1>(a, p);
    case 2: return launch_skinny<W_BIT, XDT, GS, MT, 2>(a, p);
    case 4: return launch_skinny<W_BIT, XDT, GS, MT, 4>(a, p);
  }
  return hipErrorInvalidValue;
}

template <int W_BIT, int XDT, int GS>
static hipError_t launch_mt(const MatmulArgs& a, const GemmPlan& p) {
  switch (p.mtile) {
    case 16: return launch_nt<W_BIT, XDT, GS, 1>(a, p);
    case 32: return launch_nt<W_BIT, XDT, GS, 2>(a, p);
    case 64: return launch_nt<W_BIT, XDT, GS, 4>(a, p);
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

template <int W_BIT, int XDT, int GS, bool ZP>
static hipError_t launch_large_k(const MatmulArgs& a, const GemmPlan& p) {
  const bool per_column = a.group_mask == 0;
  hipError_t e = hipSuccess;
  if (p.n_tiles > 0)
    e = launch_kernel(gemm_large_kernel<W_BIT, XDT, GS, ZP, 4>,
                      dim3((unsigned)(p.n_tiles * p.m_tiles)), dim3(256), a.stream, a.x, a.Q,
                      a.scales, a.zeros, a.y, a.M, a.N, a.K,
                      pack_tiles(p.n_tiles, a.y_dtype, per_column), 0);
  if (e == hipSuccess && p.tail_tiles > 0)
    e = launch_kernel(gemm_large_kernel<W_BIT, XDT, GS, ZP, 3>,
                      dim3((unsigned)(p.tail_tiles * p.m_tiles)), dim3(256), a.stream, a.x, a.Q,
                      a.scales, a.zeros, a.y, a.M, a.N, a.K,
                      pack_tiles(p.tail_tiles, a.y_dtype, per_column), 16 * p.n_tiles);
  return e;
}

template <int W_BIT, int XDT, int GS>
static hipError_t launch_large_z(const MatmulArgs& a, const GemmPlan& p) {
  return a.zeros != nullptr ? launch_large_k<W_BIT, XDT, GS, true>(a, p)
                            : launch_large_k<W_BIT, XDT, GS, false>(a, p);
}

template <int W_BIT, int XDT>
static hipError_t launch_large(const MatmulArgs& a, const GemmPlan& p) {
  switch (a.group_size) {
    case 32: return launch_large_z<W_BIT, XDT, 32>(a, p);
    case 64: return launch_large_z<W_BIT, XDT, 64>(a, p);
    case 128: return launch_large_z<W_BIT, XDT, 128>(a, p);
    case 256: return launch_large_z<W_BIT, XDT, 256>(a, p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const MatmulArgs& a, const GemmPlan& p) {
  const bool f16 = a.x_dtype == XF16;
  if (p.kind == 2) return launch_gemv_tile(a);
  if (p.kind == 1) {
    if (a.w_bit == 4) return f16 ? launch_large<4, XF16>(a, p) : launch_large<4, XBF16>(a, p);
    return f16 ? launch_large<2, XF16>(a, p) : launch_large<2, XBF16>(a, p);
  }
  switch (a.w_bit) {
    case 4: return f16 ? launch_gs<4, XF16>(a, p) : launch_gs<4, XBF16>(a, p);
    case 2: return f16 ? launch_gs<2, XF16>(a, p) : launch_gs<2, XBF16>(a, p);
    case 8: return f16 ? launch_gs<8, XF16>(a, p) : launch_gs<8, XBF16>(a, p);
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
