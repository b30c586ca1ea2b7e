// ternary_large.hip -- int8 x ternary product at large M (prefill) on
// v_mfma_i32_16x16x64_i8 (liger-kernel ops/experimental/mm_int8int2.py:
// int8 A times weights in {-1, 0, +1}, exact int32 sums), reading the tile
// layout written by qmm_t2_pack (ternary.hip).
//
//  * workgroup tile 256 rows x 16 NT columns, one workgroup per CU, 4 waves
//    side by side along N: a wave owns all 256 rows x NT strips = 16 x NT
//    MFMA tiles, 64 NT int32 accumulators per lane in the matrix-core
//    (AGPR) register file.  NT = 4 (full tiles) or 3
//    (narrow tiles ending N, so that the last round of workgroups is
//    shorter; the split is the low-bit prefill's, large_split);
//  * stages of 256 k: a wave's weights of a stage are one 16-byte slot per
//    strip (the 1 KiB block of that strip and stage), loaded two stages
//    ahead into registers; each of its 4 words gives the 16 codes of one
//    64-deep k step, turned into the int8 B operand by a mask and one
//    v_perm_b32 table lookup per 4 codes ({-1, 0, +1, +2} for codes 0..3).
//    One operand register is made per row tile, between that tile's MFMAs;
//  * x: the 256 x 256-byte tile of a stage is shared by the 4 waves through
//    double-buffered LDS, loaded by buffer loads straight to LDS in the
//    swizzled row layout of the other x tiles (whole 256-byte rows per
//    load, conflict-free ds_read_b128 fragments);
//  * every load is a buffer load whose descriptor ends at its operand's
//    edge (rows past M and strips past N read zeros and feed only outputs
//    that are never stored), addressed by a per-lane offset fixed for the
//    K loop plus a wave-uniform stage offset; the loads of a stage are
//    spread over its first row tiles.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kT2MT = kLargeRows / 16;  // 16-row tiles per workgroup
constexpr int kT2Frags = kT2MT * 4;     // 1 KiB x units per 256-deep stage
constexpr int kT2LoadSpan = 4;          // eighths of a stage's row tiles carrying its loads
// A fragments read from LDS ahead of the MFMAs that use them (3 and 4
// measured no faster than 2)
constexpr int kT2FragAhead = 2;
static constexpr int kT2WaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters at maximum

__device__ __forceinline__ void mfma_i8(i32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// The MFMAs of one row tile (accumulators pinned to the matrix-core
// registers) with one B operand register of a later k step made between
// them: `v` holds the codes in bits 0-1 of each byte once masked, and the
// byte table maps code c to the int8 c - 1.  One asm block, because the
// scheduler does not see the pinned MFMAs as MFMAs; the conversion writes
// only its own (early-clobber) registers, none of which an MFMA here reads.
__device__ __forceinline__ uint32_t mfma_row_t2(i32x4_t (&c)[4], const u32x4_t& a,
                                                const u32x4_t (&b)[4], uint32_t v, uint32_t mask,
                                                uint32_t table) {
  uint32_t out, m;
  asm volatile(
      "v_mfma_i32_16x16x64_i8 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_b32 %[m], %[mask], %[v]\n\t"
      "v_mfma_i32_16x16x64_i8 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_perm_b32 %[out], 0, %[tab], %[m]\n\t"
      "v_mfma_i32_16x16x64_i8 %[c2], %[a], %[b2], %[c2]\n\t"
      "v_mfma_i32_16x16x64_i8 %[c3], %[a], %[b3], %[c3]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [out] "=&v"(out),
        [m] "=&v"(m)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [v] "v"(v),
        [mask] "s"(mask), [tab] "s"(table));
  return out;
}
__device__ __forceinline__ uint32_t mfma_row_t2(i32x4_t (&c)[3], const u32x4_t& a,
                                                const u32x4_t (&b)[3], uint32_t v, uint32_t mask,
                                                uint32_t table) {
  uint32_t out, m;
  asm volatile(
      "v_mfma_i32_16x16x64_i8 %[c0], %[a], %[b0], %[c0]\n\t"
      "v_and_b32 %[m], %[mask], %[v]\n\t"
      "v_mfma_i32_16x16x64_i8 %[c1], %[a], %[b1], %[c1]\n\t"
      "v_perm_b32 %[out], 0, %[tab], %[m]\n\t"
      "v_mfma_i32_16x16x64_i8 %[c2], %[a], %[b2], %[c2]"
      : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [out] "=&v"(out), [m] "=&v"(m)
      : [a] "v"(a), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [v] "v"(v),
        [mask] "s"(mask), [tab] "s"(table));
  return out;
}

// One workgroup's tile: work item `bid` of `nblocks` over n_tiles column
// tiles of 16 NT columns starting at strip strip0, and every M tile.
template <int NT>
__device__ __forceinline__ void i8t2_large_body(const int8_t* __restrict__ x,
                                                const u32x4_t* __restrict__ Wt,
                                                int32_t* __restrict__ y, int M, int N, int K,
                                                int n_tiles, int strip0, int bid, int nblocks,
                                                u32x4_t (*xa)[kT2Frags * 64]) {
  constexpr int MT = kT2MT;
  constexpr int BM = 16 * MT;
  constexpr int KS = 256;                // k per stage = one layout block
  constexpr int STEPS = KS / 64;         // MFMA k steps per stage
  constexpr int FRAGS = kT2Frags;
  static_assert(STEPS == 4 && MT % 4 == 0, "x tile: 16 chunks per row, 4 loads per row tile");

  const uint32_t kMask = 0x03030303u, kTable = 0x020100FFu;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int w = xcd_remap(bid, nblocks);
  const int nt = w % n_tiles, m0 = (w / n_tiles) * BM;
  const int strips = N / 16, nst = K / KS;
  const int s0 = strip0 + (nt * 4 + wave) * NT;  // this wave's first strip
  const int sc0 = min(s0, strips);
  const int nvalid = min(NT, strips - sc0);
  // x: the workgroup's rows; weights: the wave's strips (strip-major blocks)
  const buf_t xb = make_buf(x + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
  const buf_t wb = make_buf(Wt + (size_t)sc0 * nst * 64, (uint32_t)(nvalid * nst * 1024));

  // x tile of a stage by row tile: 16 rows x 16 chunks of 16 bytes, chunk c
  // of row r at slot 16 r + (c ^ r).  Load unit f (1 KiB, row tile f / 4)
  // fills slots 64 (f % 4) .. + 63 of its tile: lane p's 16 bytes land at
  // slot 64 (f % 4) + p, row r = 4 (f % 4) + p / 16, so lane p fetches chunk
  // (p % 16) ^ r of that row and a load reads 4 whole rows.  Fragment (row
  // tile i, k step kk) is row l16, chunk 4 kk + quad.
  int xo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) xo[c] = quad * K + 16 * (l16 ^ (4 * c + quad));
  auto x_unit = [&](int j, int sx, int buf) {
    const int f = wave * (FRAGS / 4) + j;
    const int row = 16 * (f / 4) + 4 * (j % 4);  // first of the unit's 4 rows
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xb, (__attribute__((address_space(3))) void*)(&xa[buf][f * 64]), 16, xo[j % 4],
        row * K + sx * KS, 0, 0);
  };
  auto load_slot = [&](int s, int st, u32x4_t (&R)[NT]) {
    R[s] = __builtin_amdgcn_raw_buffer_load_b128(wb, lane * 16, (s * nst + st) * 1024, 0);
  };
  auto load_x = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < FRAGS / 4; ++j) x_unit(j, st, buf);
  };
  auto load_w = [&](int st, u32x4_t (&R)[NT]) {
#pragma unroll
    for (int s = 0; s < NT; ++s) load_slot(s, st, R);
  };
  // loads issued during a stage, one at a time: j < NXL this wave's x units
  // of stage sx, the rest the weight slots of stage sw.  A stage ends
  // waiting for its x tile only (vmcnt(NT)): the weight slots issued after
  // it, two stages ahead, may stay in flight.
  constexpr int NXL = FRAGS / 4;
  constexpr int NLD = NT + NXL;
  auto load_part = [&](int j, int sw, int sx, int buf, u32x4_t (&R)[NT]) {
    if (j < NXL) x_unit(j, sx, buf);
    else load_slot(j - NXL, sw, R);
  };
  constexpr int kWaitXTile = (NT & 15) | 0x0F70;

  i32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) acc[i][s] = i32x4_t{0, 0, 0, 0};

  // Weight registers of three stages: the current one, the next (loaded
  // during the previous stage) and the one after (loading now); the last
  // k step reads the next stage's words, where the compiler waits for
  // exactly them.  The three sets take turns over an unrolled loop: moving
  // registers from one set to another would make the compiler wait for
  // their loads at the move.
  u32x4_t ra[NT], rb[NT], rc[NT];
  load_x(0, 0);
  load_w(0, ra);
  load_w(min(1, nst - 1), rb);
#pragma unroll
  for (int s = 0; s < NT; ++s) asm volatile("" ::"v"(ra[s]), "v"(rb[s]));
  __builtin_amdgcn_s_waitcnt(kT2WaitVm0);
  __syncthreads();

  // operand register r (strip r / 4, dword r % 4) of a k step from its word
  auto operand = [&](uint32_t word, int t) {
    return __builtin_amdgcn_perm(0u, kTable, (word >> (2 * t)) & kMask);
  };
  u32x4_t b[NT], bn[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) b[s][t] = operand(ra[s][0], t);

  auto stage = [&](int st, const u32x4_t (&cur)[NT], const u32x4_t (&nx1)[NT],
                   u32x4_t (&nx2)[NT]) {
    const int buf = st & 1;
    // the last iterations re-read the final stage into the idle registers
    // and buffer, keeping the loop free of branches
    const int stn = min(st + 1, nst - 1);
    const int stw = min(st + 2, nst - 1);
    const u32x4_t* xs_buf = &xa[buf][0];
    auto afrag = [&](int i, int kk) {
      return xs_buf[256 * i + 16 * l16 + ((4 * kk + quad) ^ l16)];
    };
    // While the NT MFMAs of row tile i of k step k run: the A fragment two
    // tiles ahead is read from LDS, one operand register of the next k step
    // (of the next stage in the last k step) is made, and part of the next
    // stages' loads is issued.  The scheduling barriers hold this order.
    constexpr int P = kT2FragAhead;
    static_assert(P >= 1 && P <= STEPS * MT, "prefetch distance");
    u32x4_t ar[P];
#pragma unroll
    for (int q = 0; q < P; ++q) ar[q] = afrag(q % MT, q / MT);
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      const int kn = k + 1;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int t2 = k * MT + i + P;  // fragment P ahead, in (k, i) order
        const u32x4_t a0 = ar[0];
        u32x4_t an = ar[P - 1];
        if (t2 < STEPS * MT) an = afrag(t2 % MT, t2 / MT);
        const int r0 = i * NT * 4 / MT, r1 = (i + 1) * NT * 4 / MT;
        static_assert(NT * 4 <= MT, "one operand register per row tile at most");
        if (r0 < r1) {
          const int r = r0, t = r % 4;
          const uint32_t word = kn < STEPS ? cur[r / 4][kn] : nx1[r / 4][0];
          bn[r / 4][t] = mfma_row_t2(acc[i], a0, b, word >> (2 * t), kMask, kTable);
        } else {
#pragma unroll
          for (int s = 0; s < NT; ++s) mfma_i8(acc[i][s], a0, b[s]);
        }
        {
          constexpr int SPAN = kT2LoadSpan * STEPS * MT / 8;
          static_assert(NLD <= 2 * SPAN, "two loads per row tile at most");
          const int p = k * MT + i;
          const int j0 = (p * NLD + SPAN - 1) / SPAN;
          const int j1 = min(NLD, ((p + 1) * NLD + SPAN - 1) / SPAN);
          if (j0 < j1) load_part(j0, stw, stn, buf ^ 1, nx2);
          if (j0 + 1 < j1) load_part(j0 + 1, stw, stn, buf ^ 1, nx2);
        }
#pragma unroll
        for (int q = 0; q + 1 < P; ++q) ar[q] = ar[q + 1];
        ar[P - 1] = an;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) b[s] = bn[s];
    }
    // the next stage's x tile was written to LDS by the memory pipeline:
    // wait for this wave's part of it, then for every wave's
    __builtin_amdgcn_s_waitcnt(kWaitXTile);
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 3) {
    stage(st, ra, rb, rc);
    if (st + 1 < nst) stage(st + 1, rb, rc, ra);
    if (st + 2 < nst) stage(st + 2, rc, ra, rb);
  }
  __builtin_amdgcn_s_waitcnt(kT2WaitVm0);  // the last re-reads of the final stage
  // the accumulators were last written by MFMAs the compiler does not see
  // as such: give them their result latency, then pass each through an
  // empty asm ordered after that, so no read of one moves above it
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) asm volatile("" : "+a"(acc[i][s]));
  __builtin_amdgcn_sched_barrier(0);

  // y through LDS per 16-row tile: the wave's 16 x 16 NT block goes in
  // row-major (row stride 68 words, no bank conflicts either way) and
  // leaves as 4 whole rows per store instruction (16 lanes x 16 bytes per
  // row): whole 128-byte lines.  The x buffers are free (the K loop ended
  // with a barrier); a wave's LDS operations run in order.
  int32_t* const yl = reinterpret_cast<int32_t*>(&xa[0][0]) + wave * (16 * 68);
  const int prow = lane >> 4, pcol = 4 * (lane & 15);
  const bool pcol_ok = (lane & 15) < 4 * NT && s0 + ((lane & 15) >> 2) < strips;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int s = 0; s < NT; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) yl[(4 * quad + r) * 68 + 16 * s + l16] = acc[i][s][r];
    i32x4_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *reinterpret_cast<const i32x4_t*>(yl + (4 * j + prow) * 68 + pcol);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 16 * i + 4 * j + prow;
      if (m < M && pcol_ok) *reinterpret_cast<i32x4_t*>(y + (size_t)m * N + 16 * s0 + pcol) = v[j];
    }
  }
}

// The whole plan in one launch: work items [0, full) take full tiles over
// the first n_full column tiles, the rest narrow tiles over the remaining
// columns (dispatched last, so they start on whichever CUs free up first).
__global__ __launch_bounds__(256, 1) void i8t2_large_kernel(const int8_t* __restrict__ x,
                                                            const u32x4_t* __restrict__ Wt,
                                                            int32_t* __restrict__ y, int M, int N,
                                                            int K, int n_full, int tail_tiles) {
  __shared__ u32x4_t xa[2][kT2Frags * 64];
  const int m_tiles = (M + kLargeRows - 1) / kLargeRows;
  const int full = n_full * m_tiles;
  const int b = (int)blockIdx.x;
  if (b < full)
    i8t2_large_body<4>(x, Wt, y, M, N, K, n_full, 0, b, full, xa);
  else
    i8t2_large_body<3>(x, Wt, y, M, N, K, tail_tiles, 16 * n_full, b - full,
                       tail_tiles * m_tiles, xa);
}

// ---------------------------------------------------------------- host side
hipError_t launch_i8t2_large(const void* x, const void* Wt, int32_t* y, int M, int N, int K,
                             hipStream_t st) {
  const int m_tiles = (M + kLargeRows - 1) / kLargeRows;
  int n_full = 0, n_tail = 0;
  large_split(m_tiles, N / 16, &n_full, &n_tail);
  return launch_kernel(i8t2_large_kernel, dim3((unsigned)((n_full + n_tail) * m_tiles)),
                       dim3(256), st, static_cast<const int8_t*>(x),
                       static_cast<const u32x4_t*>(Wt), y, M, N, K, n_full, n_tail);
}

}  // namespace qmm
