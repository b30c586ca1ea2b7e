// ternary.hip -- int8 activations x ternary weights on the int8 matrix cores
// (liger-kernel ops/experimental/mm_int8int2.py: matmul of int8 A by weights
// in {-1, 0, +1} stored as 2-bit codes value + 1, int32 accumulation).
//
// Page layout of the weight (pack_weights): (K/4, N) uint8, K split into four
// consecutive quarters of R = K/4 rows, quarter i in bits 2i..2i+1, so
// element k of column n is code (Wp[k mod R][n] >> 2 (k div R)) & 3.  A lane
// of an MFMA needs 16 consecutive k of one column, which that layout spreads
// over 16 rows N bytes apart; qmm_t2_pack therefore rewrites it once into the
// tile layout below, and the GEMM streams that:
//  * 1 KiB blocks, one per (16-column strip, 256-deep K block), strip-major;
//    bytes [16 L, 16 L + 16) are lane L: column 16 s + L % 16, lane group
//    g = L / 16; dword j holds the 16 codes of k = 256 kb + 64 j + 16 g + e,
//    code e at bit 2 (4 (e % 4) + e / 4), so (w >> 2t) & 0x03030303 is codes
//    4t .. 4t + 3 in byte order;
//  * one v_perm_b32 per 4 codes maps code c to the int8 c - 1 through the
//    table {-1, 0, +1, +2} -- the page's "mask, shift, subtract 1" -- giving
//    the B operand of v_mfma_i32_16x16x64_i8 directly (the x operand uses the
//    same k order per lane group, so products pair up whatever order the
//    instruction sums in);
//  * x reaches the A operands through LDS tiles in a swizzled row layout
//    (whole rows per load, conflict-free ds_read_b128 fragments); the sums
//    are exact int32.
// This file holds the repack, the decode kernel (M <= 16) and the 16-row
// tile kernel (17-64 rows); ternary_large.hip the 256-row one.
#include <hip/hip_runtime.h>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// bit position of code e (0..15) inside a dword of the tile layout
__host__ __device__ constexpr int t2_pos(int e) { return 2 * (4 * (e % 4) + e / 4); }

// code of element (k, n) in the page layout
__device__ __forceinline__ uint32_t t2_code(const uint8_t* Wp, int N, int R, int k, int n) {
  return (Wp[(size_t)(k % R) * N + n] >> (2 * (k / R))) & 3u;
}

// One thread per output dword of the tile layout (dword t = block * 256 +
// lane * 4 + j).
__global__ void t2_pack_kernel(const uint8_t* __restrict__ Wp, uint32_t* __restrict__ Wt, int N,
                               int K) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int nkb = K / 256;
  const size_t total = (size_t)N * K / 16;
  if (t >= total) return;
  const int j = (int)(t % 4), lane = (int)((t / 4) % 64);
  const size_t blk = t / 256;
  const int s = (int)(blk / nkb), kb = (int)(blk % nkb);
  const int n = 16 * s + lane % 16, g = lane / 16;
  const int R = K / 4;
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) w |= t2_code(Wp, N, R, 256 * kb + 64 * j + 16 * g + e, n) << t2_pos(e);
  Wt[t] = w;
}

// Inverse: one thread per page byte (row r, column n), four quarters.
__global__ void t2_unpack_kernel(const uint32_t* __restrict__ Wt, uint8_t* __restrict__ Wp, int N,
                                 int K) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int R = K / 4;
  if (t >= (size_t)R * N) return;
  const int r = (int)(t / N), n = (int)(t % N);
  const int nkb = K / 256, s = n / 16;
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = i * R + r;
    const int kb = k / 256, rr = k % 256, j = rr / 64, g = (rr % 64) / 16, e = rr % 16;
    const uint32_t w = Wt[((size_t)s * nkb + kb) * 256 + (16 * g + n % 16) * 4 + j];
    b |= ((w >> t2_pos(e)) & 3u) << (2 * i);
  }
  Wp[t] = (uint8_t)b;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// the 16 int8 weights of one k step (dword w of a lane's slot)
__device__ __forceinline__ u32x4_t t2_operand(uint32_t w) {
  u32x4_t b;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    b[t] = __builtin_amdgcn_perm(0u, 0x020100FFu, (w >> (2 * t)) & 0x03030303u);
  return b;
}

// int8 MFMA whose accumulator is pinned to the matrix-core (AGPR) registers:
// with the builtin, the allocator splits the GEMM's MT x NT4 accumulators
// between the two register files and moves them back and forth every stage.
// Every accumulator is used once per MT x NT4 MFMAs, far beyond the result
// latency, so the loop needs no extra wait states.
__device__ __forceinline__ void mfma_i8_acc(i32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Workgroup tile 16 MT rows x 64 NT4 columns: 4 waves side by side along N,
// each NT4 strips of 16 columns, MT 16-row tiles; 256-deep stages.  Used at
// 17-64 rows (MT = NT4 = 1); larger M goes to the 256-row kernel of
// ternary_large.hip.
template <int MT, int NT4>
__global__ __launch_bounds__(256) void i8t2_gemm_kernel(const int8_t* __restrict__ x,
                                                        const u32x4_t* __restrict__ Wt,
                                                        int32_t* __restrict__ y, int M, int N,
                                                        int K, int n_tiles) {
  constexpr int STEPS = 4;              // 64-deep MFMA steps per stage
  constexpr int FRAGS = MT * STEPS;     // 1 KiB x fragments per stage
  constexpr int XPW = FRAGS / 4;        // fragments each wave loads
  static_assert(FRAGS % 4 == 0, "the 4 waves share the x fragments evenly");
  __shared__ u32x4_t xa[2][FRAGS * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int l16 = lane & 15, quad = lane >> 4;
  const int w = xcd_remap(blockIdx.x, n_tiles * ((M + 16 * MT - 1) / (16 * MT)));  // the grid
  const int nt = w % n_tiles, m0 = (w / n_tiles) * 16 * MT;
  const int strips = N / 16, nkb = K / 256;
  const int s0 = (nt * 4 + wave) * NT4;
  int sidx[NT4];
#pragma unroll
  for (int s = 0; s < NT4; ++s) sidx[s] = min(s0 + s, strips - 1);  // loads stay in bounds
  const int rows_left = M - 1 - m0;

  // The x tile of a stage is stored by row tile: 16 rows x 16 chunks of 16
  // bytes (the stage's 256 k of a row), chunk c of row r at slot 16 r +
  // (c ^ r).  Load unit f (1 KiB, row tile f / 4) fills slots 64 (f % 4) ..
  // + 63 of its tile, lane p's bytes landing at slot 64 (f % 4) + p: row
  // r = 4 (f % 4) + p / 16, position p % 16, so lane p fetches chunk
  // (p % 16) ^ r and one load reads 4 whole 256-byte rows (fragment order,
  // 16 rows x 64 bytes per load, is served at well under half the rate).
  // Fragment (row tile i, k step j) = row l16, chunk 4 j + quad: one
  // conflict-free ds_read_b128.  Rows past M read row M - 1 (never stored).
  static_assert(STEPS == 4, "16 chunks per row, 4 loads per row tile");
  auto load_x = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
      const int f = wave * XPW + j;
      const int r = 4 * (f % 4) + quad;
      const int rr = min(16 * (f / 4) + r, rows_left);
      const int k = st * 256 + 16 * (l16 ^ r);
      __builtin_amdgcn_global_load_lds((const void*)(x + (size_t)(m0 + rr) * K + k),
                                       (__attribute__((address_space(3))) void*)(&xa[buf][f * 64]),
                                       16, 0, 0);
    }
  };
  auto load_w = [&](int st, u32x4_t (&R)[NT4]) {
#pragma unroll
    for (int s = 0; s < NT4; ++s) R[s] = Wt[((size_t)sidx[s] * nkb + st) * 64 + lane];
  };

  i32x4_t acc[MT][NT4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT4; ++s) acc[i][s] = i32x4_t{0, 0, 0, 0};

  // One stage: MFMAs on the x tile in xa[st & 1] and the weights in `use`,
  // while the next stage's weights go to `fill` and its x tile to the other
  // buffer (the last stage re-reads itself, keeping the body branch-free).
  // Two register sets take turns (no loop-carried copy: a copy would be
  // scheduled right behind the loads and stall the stage on them).
  auto stage = [&](int st, const u32x4_t (&use)[NT4], u32x4_t (&fill)[NT4]) {
    const int buf = st & 1;
    const int stn = min(st + 1, nkb - 1);
    u32x4_t b[NT4];
#pragma unroll
    for (int s = 0; s < NT4; ++s) b[s] = t2_operand(use[s][0]);
    __builtin_amdgcn_sched_barrier(0);
    load_w(stn, fill);
    load_x(stn, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    // A fragments are read from LDS two row tiles ahead of their MFMAs, in
    // consumption order (k step major, row tile minor), so the LDS latency
    // overlaps the MFMAs of the tiles in between
    const u32x4_t* xs = &xa[buf][0];
    constexpr int NF = MT * STEPS;
    auto frag = [&](int c) {
      return xs[256 * (c % MT) + 16 * l16 + ((4 * (c / MT) + quad) ^ l16)];
    };
    u32x4_t ar[3];
    ar[0] = frag(0);
    if (NF > 1) ar[1] = frag(1);
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      u32x4_t bn[NT4];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int c = j * MT + i;
        if (c + 2 < NF) ar[(c + 2) % 3] = frag(c + 2);
        const u32x4_t a = ar[c % 3];
#pragma unroll
        for (int s = 0; s < NT4; ++s)
          mfma_i8_acc(acc[i][s], a, b[s]);
        // next k step's operands, spread over the row tiles
        if (j + 1 < STEPS) {
#pragma unroll
          for (int s = 0; s < NT4; ++s)
            if (i == s % MT) bn[s] = t2_operand(use[s][j + 1]);
        }
      }
      if (j + 1 < STEPS) {
#pragma unroll
        for (int s = 0; s < NT4; ++s) b[s] = bn[s];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the next stage's loads, this wave's
    __syncthreads();                      // ... and every wave's x tile
  };

  u32x4_t wa[NT4], wb[NT4];
  load_x(0, 0);
  load_w(0, wa);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int st = 0; st < nkb; st += 2) {
    stage(st, wa, wb);
    if (st + 1 < nkb) stage(st + 1, wb, wa);
  }
  // the accumulators were last written by MFMAs the compiler does not see as
  // such: give them their result latency, then pass each through an empty asm
  // ordered after that, so no read of one moves above it
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT4; ++s) asm volatile("" : "+a"(acc[i][s]));
  __builtin_amdgcn_sched_barrier(0);

  // each lane stores its accumulator elements (4 rows of one column)
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    if (s0 + s >= strips) continue;
    const int n = 16 * (s0 + s) + l16;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * quad + r;
        if (m < M) y[(size_t)m * N + n] = acc[i][s][r];
      }
  }
}

// Decode-sized M (one 16-row tile): a workgroup owns NT strips, and its 4
// waves split K into quarters (as the skinny low-bit GEMM does), each with
// up to 4 stages of weight slots and x rows in flight straight to
// registers (x then passes through a per-wave LDS tile into operand
// order); the 4 partial tiles meet in LDS.
template <int NT>
__global__ __launch_bounds__(256) void i8t2_skinny_kernel(const int8_t* __restrict__ x,
                                                          const u32x4_t* __restrict__ Wt,
                                                          int32_t* __restrict__ y, int M, int N,
                                                          int K, int n_tiles) {
  constexpr int DEPTH = 4;  // stages in flight per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int w = xcd_remap(blockIdx.x, n_tiles);  // the grid: one workgroup per strip
  const int nt = w % n_tiles, m0 = (w / n_tiles) * 16;
  const int strips = N / 16, nkb = K / 256;
  const int s0 = nt * NT;
  int sidx[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) sidx[s] = min(s0 + s, strips - 1);
  const int per = (nkb + 3) / 4;
  const int kb0 = min(nkb, wave * per), kb1 = min(nkb, kb0 + per);
  // x arrives as whole rows (load j: rows 4j .. 4j + 3, 16-byte chunk l16 of
  // each row's 256-byte block) and becomes A fragments through a per-wave
  // LDS tile, chunk c of row r at slot 16 r + (c ^ r) (conflict-free both
  // ways; a wave's LDS operations run in order, so no barrier): an
  // operand-order load would touch 16 rows x 64 bytes, a slow pattern.
  __shared__ u32x4_t xt[4][256];
  u32x4_t* const xw = xt[wave];
  const int8_t* xrows[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xrows[j] = x + (size_t)min(m0 + 4 * j + quad, M - 1) * K + 16 * l16;

  i32x4_t acc[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) acc[s] = i32x4_t{0, 0, 0, 0};
  for (int kb = kb0; kb < kb1; kb += DEPTH) {
    u32x4_t wr[DEPTH][NT], xr[DEPTH][4];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int k = min(kb + d, kb1 - 1);  // past the range: re-read, not used
#pragma unroll
      for (int s = 0; s < NT; ++s)
        wr[d][s] = __builtin_nontemporal_load(&Wt[((size_t)sidx[s] * nkb + k) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xr[d][j] = *reinterpret_cast<const u32x4_t*>(xrows[j] + (size_t)k * 256);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (kb + d < kb1) {
        u32x4_t af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xw[16 * (4 * j + quad) + (l16 ^ (4 * j + quad))] = xr[d][j];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = xw[16 * l16 + ((4 * j + quad) ^ l16)];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int s = 0; s < NT; ++s)
            acc[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                __builtin_bit_cast(i32x4_t, af[j]),
                __builtin_bit_cast(i32x4_t, t2_operand(wr[d][s][j])), acc[s], 0, 0, 0);
      }
    }
  }

  __shared__ int32_t red[4][16][16 * NT + 1];
#pragma unroll
  for (int s = 0; s < NT; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * quad + r][16 * s + l16] = acc[s][r];
  __syncthreads();
  for (int o = threadIdx.x; o < 16 * 16 * NT; o += 256) {
    const int rr = o / (16 * NT), cc = o % (16 * NT);
    const int m = m0 + rr, n = 16 * s0 + cc;
    if (m < M && n < N) y[(size_t)m * N + n] = red[0][rr][cc] + red[1][rr][cc] + red[2][rr][cc] +
                                               red[3][rr][cc];
  }
}

// ---------------------------------------------------------------- host side
hipError_t launch_t2_pack(const void* Wp, void* Wt, int N, int K, hipStream_t st) {
  const size_t total = (size_t)N * K / 16;
  return launch_kernel(t2_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), st, Wp, Wt,
                       N, K);
}

hipError_t launch_t2_unpack(const void* Wt, void* Wp, int N, int K, hipStream_t st) {
  const size_t total = (size_t)N * K / 4;
  return launch_kernel(t2_unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), st, Wt,
                       Wp, N, K);
}

template <int MT, int NT4>
static hipError_t launch_i8t2(const void* x, const void* Wt, int32_t* y, int M, int N, int K,
                              hipStream_t st) {
  const int strips = N / 16;
  const int n_tiles = (strips + 4 * NT4 - 1) / (4 * NT4);
  const int m_tiles = (M + 16 * MT - 1) / (16 * MT);
  return launch_kernel(i8t2_gemm_kernel<MT, NT4>, dim3((unsigned)(n_tiles * m_tiles)), dim3(256),
                       st, x, Wt, y, M, N, K, n_tiles);
}

hipError_t launch_i8t2_gemm(const void* x, const void* Wt, int32_t* y, int M, int N, int K,
                            hipStream_t st) {
  if (M <= 16) {
    // one strip per workgroup; K split over its 4 waves
    const int n_tiles = N / 16;
    return launch_kernel(i8t2_skinny_kernel<1>, dim3((unsigned)n_tiles), dim3(256), st, x, Wt, y,
                         M, N, K, n_tiles);
  }
  if (M <= 64) return launch_i8t2<1, 1>(x, Wt, y, M, N, K, st);  // 16-row tiles
  return launch_i8t2_large(x, Wt, y, M, N, K, st);
}

}  // namespace qmm
