// gemm_mfma.hip -- qmm_gemm's planner and its skinny matrix-core kernel:
// y = x * dequant(Q) with Q in the tile layout written by qmm_pack
// (repack.hip), on v_mfma_f32_16x16x32_{f16,bf16} (large M: gemm_large.hip;
// M <= 2: the tile GEMV, gemv_tile.hip).
//
// Skinny kernel (decode batches, M up to a few 16-row tiles), HBM-bound:
//  * a workgroup = 4 waves on one M-tile (MT 16-row tiles) and NT 16-column
//    strips; the 4 waves split K into quarters, and their partial tiles meet
//    in LDS at the end.  When the tiles leave most CUs idle, K is also split
//    over up to 4 workgroups per tile (with a workspace): each writes its
//    partial tile through to memory, and the last to take the tile's ticket
//    adds them in a fixed order;
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
  // the grid (tiles x splits), from the arguments: no read of the dispatch's
  // grid size, which is a memory load at wave start
  const int m_tiles = (M + 16 * MT - 1) / (16 * MT);
  const int w0 = xcd_remap(blockIdx.x, n_tiles * m_tiles * S);
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
        R.w[s][b] = buf_load128_stream(qbuf, ((s * nblk + kb) * 64 + lane) * 16);
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

  // int8 column scales, requested before the weights so that their latency
  // overlaps the K loop's instead of following it
  float csc[LOWBIT ? 1 : NT];
  if constexpr (!LOWBIT) {
#pragma unroll
    for (int s = 0; s < NT; ++s)
      csc[s] = reinterpret_cast<const float*>(scales)[16 * min(s0 + s, strips - 1) + l16];
  }
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
    float bz[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) bz[s] = CB;
    flush(csc, bz);
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
    // Workspace: the first kTicketSlots words hold one ticket per tile (zero
    // between calls), then S partial tiles of ROWS x COLS fp32 per tile.  The partial
    // goes out with coherent stores; once they have completed (vmcnt 0 in
    // every wave, then the barrier) one lane takes the tile's ticket.  The
    // ticket is an agent-scope atomic, so whichever workgroup draws S - 1 is
    // the last, and every other partial of its tile is already written
    // through; it re-arms the ticket and reads the S partials back (from its
    // XCD's L2 when all splits ran there, else with coherent loads).  Nobody
    // waits on anybody: the workgroups that are not last end.
    uint32_t* tickets = ws;  // kTicketSlots of them, then the partial tiles
    float* parts = reinterpret_cast<float*>(ws + kTicketSlots);
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
    // The ticket counts arrivals per XCD (ticket_arrivals).  When every
    // split of the tile ran on this workgroup's XCD, their write-through
    // stores are in this XCD's L2 and the partials are read from it;
    // otherwise from past the L2s.
    const uint32_t xcc = xcc_id();
    __shared__ int last, local;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t ticket = __hip_atomic_fetch_add(tickets + w, 1u << (4 * xcc), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t n = ticket_arrivals(ticket);
      last = n == (uint32_t)(S - 1);
      local = ((ticket >> (4 * xcc)) & 15u) == n;
      if (last) __hip_atomic_store(tickets + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    const bool here = local != 0;
    with_y(y, ydt, [&](auto* yt) {
      using T = typename std::remove_pointer<decltype(yt)>::type;
      for (int o = 4 * threadIdx.x; o < PART; o += 4 * 64 * WAVES) {
        // all S loads in flight at once, then added in split order
        u32x4_t pv[kMaxSplits];
        if (here) {
#pragma unroll
          for (int q = 0; q < kMaxSplits; ++q)
            if (q < S) pv[q] = buf_load128_xcd(pbuf, (q * PART + o) * 4);
        } else {
#pragma unroll
          for (int q = 0; q < kMaxSplits; ++q)
            if (q < S) pv[q] = buf_load128_coherent(pbuf, (q * PART + o) * 4);
        }
        f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < kMaxSplits; ++q)
          if (q < S) sum += __builtin_bit_cast(f32x4_t, pv[q]);
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
    int M, int N, int K, int tile_opts, uint32_t* __restrict__ ws) {
  skinny_body<W_BIT, XDT, GS, MT, NT, DEPTH, WAVES, true>(x, Qt, scales, qz, y, ws, M, N, K,
                                                          tile_opts);
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

GemmPlan plan_gemm(int M, int N, int K, int w_bit, int group_size, bool with_workspace) {
  GemmPlan p{};
  (void)group_size;
  static const int big = env_int("QMM_GEMM_LARGE_MIN_M");
  if (w_bit != 8 && M > (big > 0 ? big : 64) && K % 128 == 0) {
    p.kind = 1;
    p.mtile = kLargeRows;
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
  // int8 at 16-64 rows: the medium kernel, whose workgroups cover 128
  // columns and share their x rows through LDS (the skinny kernel's 64-column
  // workgroups each re-read all of x), K split over workgroups so that about
  // one round of them covers the CUs.  It needs the split's workspace unless
  // the tiles alone fill the CUs.  At 16 rows (K = 4096, N = 14336) it
  // measured 16.3 us against the skinny kernel's 16.9 on the same box; below
  // 16 rows the skinny kernel stays.
  static const int want_med = env_int("QMM_MEDIUM");
  static const int want_med_nt = env_int("QMM_MEDIUM_NT");
  static const int want_med_s = env_int("QMM_MEDIUM_SPLITS");
  static const int med_min = env_int("QMM_MEDIUM_MIN_M");
  if (w_bit == 8 && M > (med_min >= 0 ? med_min : 15) && M <= 64 && K % 128 == 0 &&
      want_med != 0) {
    const int mmt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    // 64 rows: 8 waves of one strip (two per SIMD) measured 21.8-22.2 us
    // against 24.2 for 4 waves of two strips; 32 rows: 4 waves (17.9-18.2
    // against 18.0-18.3)
    static const int want_med_w = env_int("QMM_MEDIUM_WAVES");
    const int mw = mmt == 1 ? 4 : (want_med_w == 4 || want_med_w == 8) ? want_med_w : (mmt == 4 ? 8 : 4);
    const int mnt = mw == 8 ? 1 : ((want_med_nt == 2 || want_med_nt == 4) ? want_med_nt : 2);
    const int n_tiles = (N / 16 + mw * mnt - 1) / (mw * mnt);
    const long tiles = n_tiles;
    const int nst = K / 128;
    int s = 1;
    if (with_workspace)
      while (s < 8 && tiles * (s + 1) <= 248 && nst / (s + 1) >= 4) ++s;
    if (with_workspace && want_med_s >= 1 && want_med_s <= kMaxSplits) s = want_med_s;
    if (tiles > kTicketSlots) s = 1;
    if (s > 1 || tiles >= 192) {
      p.kind = 3;
      p.mtile = 16 * mmt;
      p.nt = mnt;
      p.n_tiles = n_tiles;
      p.m_tiles = 1;
      p.waves = mw;
      p.splits = s;
      p.workspace_bytes = medium_workspace_bytes((int)tiles, s, mmt, mw * mnt);
      return p;
    }
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
  if (with_workspace && want_s >= 1 && want_s <= kMaxSplits && tiles <= kTicketSlots)
    p.splits = want_s;
  const bool w8 = nt == 1 && (mt == 1 || (mt == 2 && w_bit != 2));
  p.waves = (p.splits == 1 && tiles < 128 && w8 && nst >= 16) ? 8 : 4;
  static const int want = env_int("QMM_SKINNY_WAVES");
  if (p.splits == 1 && (want == 4 || (want == 8 && w8))) p.waves = want;
  p.workspace_bytes = 0;
  if (p.splits > 1) {
    p.workspace_bytes = (size_t)kTicketSlots * 4 + (size_t)tiles * p.splits * p.mtile * 16 * nt * 4;
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
                           a.Q, a.scales, a.zeros, a.y, a.M, a.N, a.K,
                           pack_tiles(p.n_tiles, a.y_dtype, a.group_mask == 0, p.splits),
                           static_cast<uint32_t*>(a.workspace));
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

hipError_t launch_gemm(const MatmulArgs& a, const GemmPlan& p) {
  const bool f16 = a.x_dtype == XF16;
  if (p.kind == 2) return launch_gemv_tile(a);
  if (p.kind == 1) return launch_gemm_large(a, p);
  if (p.kind == 3) return launch_gemm_medium(a, p);
  switch (a.w_bit) {
    case 4: return f16 ? launch_gs<4, XF16>(a, p) : launch_gs<4, XBF16>(a, p);
    case 2: return f16 ? launch_gs<2, XF16>(a, p) : launch_gs<2, XBF16>(a, p);
    case 8: return f16 ? launch_gs<8, XF16>(a, p) : launch_gs<8, XBF16>(a, p);
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
