// gemm_medium.hip -- int8 weights at medium batch sizes (17 to 64 rows) on
// the matrix cores: y = scale * (x . q) with the fp32 column scale after the
// sum (tiny-llm's int8 matmul), q in the tile layout written by qmm_pack.
//
// The skinny kernel (gemm_mfma.hip) gives each workgroup 64 columns, so at
// 64 rows every workgroup reads all of x (64 x K) for 64 columns of
// weights: at N = 14336 the 224 workgroups fetch x 224 times, twice the
// weights' bytes.  Here a workgroup covers 128 columns (WV waves side by
// side along N, NT strips each: 4 x 2 at 32 rows, 8 x 1 at 64) and shares
// one copy of its x rows through LDS, as the large-M kernel does; to keep
// every CU busy, K is split over S workgroups per tile, each writing its
// partial tile to the workspace, and the last of a tile's S workgroups to
// arrive adds them in split order.
//  * x: 16 MT rows x 128 k per stage, buffer loads into the stage's ring
//    registers, written at the top of the stage to a double-buffered LDS
//    tile in the swizzled row layout (chunk c of row r at slot 16 r +
//    (c ^ r)); every A operand is one conflict-free ds_read_b128;
//  * weights: each wave streams its strips' 1 KiB blocks from the tile
//    layout straight into B operands, a 4-deep ring of stages; the int8 codes
//    become exact 16-bit floats (fp16: the code's byte under the 1024
//    exponent, minus 1152; bf16: a signed byte convert) and the matrix
//    cores form x . q exactly per product, summed in fp32;
//  * partial tiles go out with coherent (L2-bypassing) stores in the
//    accumulator layout, whole 1 KiB runs per wave instruction; one agent-scope
//    ticket per tile elects the last workgroup, which re-arms it.
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

template <int XDT> __device__ __forceinline__ f32x4_t mfma_m(const u32x4_t& a, const u32x4_t& b,
                                                             const f32x4_t& c);
template <> __device__ __forceinline__ f32x4_t mfma_m<XF16>(const u32x4_t& a, const u32x4_t& b,
                                                            const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma_m<XBF16>(const u32x4_t& a, const u32x4_t& b,
                                                             const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// B operand of one 32-deep k step: the step's 8 code bytes of the lane's
// column (words lo, hi of its 16-byte slot) as exact 16-bit floats, pairs
// (k = 2t, 2t + 1) in register t.
template <int XDT> __device__ __forceinline__ u32x4_t i8_operand(uint32_t lo, uint32_t hi);
template <> __device__ __forceinline__ u32x4_t i8_operand<XF16>(uint32_t lo, uint32_t hi) {
  // u = q + 128 (flip the sign bit) under the fp16 exponent of 1024 gives
  // 1024 + u exactly; subtracting 1152 leaves q, exactly
  const half2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint32_t ul = lo ^ 0x80808080u, uh = hi ^ 0x80808080u;
  u32x4_t b;
  b[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, ul, 0x04010400u)) + off);
  b[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, ul, 0x04030402u)) + off);
  b[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, uh, 0x04010400u)) + off);
  b[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, uh, 0x04030402u)) + off);
  return b;
}
template <> __device__ __forceinline__ u32x4_t i8_operand<XBF16>(uint32_t lo, uint32_t hi) {
  // every int8 value is exact in bf16 (8 significant bits)
  auto pair = [](uint32_t w, int sh) {
    bf16x2_t p = {(__bf16)(float)(int8_t)(w >> sh), (__bf16)(float)(int8_t)(w >> (sh + 8))};
    return __builtin_bit_cast(uint32_t, p);
  };
  u32x4_t b;
  b[0] = pair(lo, 0);
  b[1] = pair(lo, 16);
  b[2] = pair(hi, 0);
  b[3] = pair(hi, 16);
  return b;
}

}  // namespace

template <int XDT, int MT, int NT, int WV, int D, bool SPLIT>
__global__ __launch_bounds__(64 * WV, 1) void gemm_int8_medium_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const float* __restrict__ scales, void* __restrict__ y, uint32_t* __restrict__ ws, int M,
    int N, int K, int tile_opts) {
  const int n_tiles = tiles_of(tile_opts), ydt = ydt_of(tile_opts);
  constexpr int KB = 64;                // int8 layout block depth
  constexpr int KS = 128;               // k per stage: two blocks
  constexpr int STEPS = KS / 32;        // MFMA k steps per stage
  constexpr int FRAGS = MT * STEPS;     // 1 KiB x units per stage
  constexpr int BM = 16 * MT;
  static_assert(FRAGS % WV == 0, "whole load units per wave");

  __shared__ u32x4_t xa[2][FRAGS * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int S = SPLIT ? splits_of(tile_opts) : 1;
  const int m_tiles = (M + BM - 1) / BM;
  const int w0 = xcd_remap(blockIdx.x, n_tiles * m_tiles * S);  // the grid, from the arguments
  const int split = SPLIT ? w0 % S : 0;
  const int w = SPLIT ? w0 / S : w0;  // tile
  const int nt = w % n_tiles, mt_idx = w / n_tiles;
  const int m0 = mt_idx * BM;
  const int strips = N / 16;
  const int s0 = (nt * WV + wave) * NT;  // this wave's first strip
  const int nblk = K / KB;
  // this workgroup's stages of K
  const int nst_all = K / KS;
  const int per = (nst_all + S - 1) / S;
  const int sa = min(nst_all, split * per);
  const int nst = min(nst_all, sa + per) - sa;

  // buffer descriptors ending at the operands' edges: rows past M and
  // strips past N read zeros
  const buf_t xb = make_buf(x + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K * 2));
  const int sc0 = min(s0, strips);
  const int nvalid = min(NT, strips - sc0);
  const buf_t qb = make_buf(Qt + (size_t)sc0 * nblk * 64, (uint32_t)(nvalid * nblk * 1024));

  // x unit f (row tile f / 4, rows 4 (f % 4) .. + 3, 256 contiguous bytes
  // each): lane p's 16 bytes belong at slot 64 (f % 4) + p of the row tile
  // (chunk (p % 16) ^ r of row r = 4 (f % 4) + p / 16).  Units travel in the
  // stage's registers and are written to LDS at the top of their stage: the
  // loads then are all of one kind, so the compiler's waits for each ring
  // slot count only the later slots' loads (a load straight to LDS in
  // flight makes it wait for every load).
  auto x_unit = [&](int j, int st) {
    const int f = wave * (FRAGS / WV) + j;
    const int c = f % 4;
    const int r = 4 * c + quad;
    return __builtin_amdgcn_raw_buffer_load_b128(
        xb, (quad * K + 8 * (l16 ^ r)) * 2, ((16 * (f / 4) + 4 * c) * K + (sa + st) * KS) * 2, 0);
  };
  struct WRegs {
    u32x4_t slot[NT][2];
    u32x4_t xr[FRAGS / WV];
  };
  auto load_slot = [&](int s, int b, int st, WRegs& R) {
    R.slot[s][b] = __builtin_amdgcn_raw_buffer_load_b128(
        qb, lane * 16, (s * nblk + 2 * (sa + st) + b) * 1024, kStream);
  };
  constexpr int NWL = 2 * NT;  // weight slot loads per stage
  auto load_w = [&](int st, WRegs& R) {
#pragma unroll
    for (int j = 0; j < NWL; ++j) load_slot(j / 2, j % 2, st, R);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NT; ++s) acc[i][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // D-deep ring of stages in registers (x units and weight slots of stage t
  // in set t % D, issued in ring order); the x tile of stage t goes to LDS
  // buffer t % 2 at the top of the stage, then one barrier: every wave has
  // written its units of stage t and finished reading stage t - 1, whose
  // buffer stage t + 1 reuses.
  // column scales of the wave's strips (past N: zeros, never stored),
  // requested before the weights so that their latency overlaps the K
  // loop's instead of following it
  const buf_t sb = make_buf(scales + 16 * sc0, (uint32_t)(nvalid * 16 * 4));
  float sc[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s)
    sc[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sb, (16 * s + l16) * 4, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  WRegs ring[D];
  auto issue = [&](int t, int d) {
#pragma unroll
    for (int j = 0; j < FRAGS / WV; ++j) ring[d].xr[j] = x_unit(j, t);
    load_w(t, ring[d]);
  };
  if (nst > 0) {
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
      issue(min(d, nst - 1), d);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int t0 = 0; t0 < nst; t0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int t = t0 + d;
        if (t >= nst) break;
        issue(min(t + D - 1, nst - 1), (d + D - 1) % D);
        __builtin_amdgcn_sched_barrier(0);
        u32x4_t* xs_buf = &xa[t & 1][0];
#pragma unroll
        for (int j = 0; j < FRAGS / WV; ++j)
          xs_buf[(wave * (FRAGS / WV) + j) * 64 + lane] = ring[d].xr[j];
        __syncthreads();
        const WRegs& cur = ring[d];
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
          u32x4_t b[NT];
#pragma unroll
          for (int s = 0; s < NT; ++s) {
            const u32x4_t& sl = cur.slot[s][k / 2];
            b[s] = i8_operand<XDT>(sl[2 * (k % 2)], sl[2 * (k % 2) + 1]);
          }
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const u32x4_t a = xs_buf[256 * i + 16 * l16 + ((4 * k + quad) ^ l16)];
#pragma unroll
            for (int s = 0; s < NT; ++s) acc[i][s] = mfma_m<XDT>(a, b[s], acc[i][s]);
          }
        }
      }
    }
  }


  auto store_y = [&](const f32x4_t (&v)[MT][NT]) {
    with_y(y, ydt, [&](auto* yt) {
      using T = typename std::remove_pointer<decltype(yt)>::type;
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if (s0 + s >= strips) continue;
        const int n = 16 * (s0 + s) + l16;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + 16 * i + 4 * quad + r;
            if (m < M) yt[(size_t)m * N + n] = (T)(v[i][s][r] * sc[s]);
          }
      }
    });
  };
  if constexpr (!SPLIT) {
    store_y(acc);
  } else {
    // Workspace: the first kTicketSlots words hold one ticket per tile (zero
    // between calls), then S partial tiles per tile, each 256 lanes x MT NT x 16
    // bytes in the accumulator layout.  The partial goes out with coherent
    // stores; once they have completed (vmcnt 0 in every wave, then the
    // barrier) one lane takes the tile's ticket; the workgroup that draws
    // S - 1 is the last, re-arms the ticket and reads the S partials back
    // with coherent loads, in split order.  Nobody waits on anybody.
    uint32_t* tickets = ws;  // kTicketSlots of them, then the partial tiles
    constexpr int NTH = 64 * WV;
    constexpr int PART = MT * NT * NTH;  // 16-byte units per partial
    const buf_t pbuf = make_buf(ws + kTicketSlots + (size_t)w * S * PART * 4,
                                (uint32_t)(S * PART * 16));
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < NT; ++s)
        buf_store128_coherent(__builtin_bit_cast(u32x4_t, acc[i][s]), pbuf,
                              ((split * MT * NT + i * NT + s) * NTH + (int)threadIdx.x) * 16);
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
    f32x4_t sum[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < NT; ++s) sum[i][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int s = 0; s < NT; ++s)
          sum[i][s] += __builtin_bit_cast(
              f32x4_t, buf_load128_coherent(pbuf, ((q * MT * NT + i * NT + s) * NTH + (int)threadIdx.x) * 16));
    store_y(sum);
  }
}

// ---------------------------------------------------------------- host side
// stages in flight per workgroup
constexpr int kMediumDepth = 4;

size_t medium_workspace_bytes(int tiles, int splits, int mt, int strips_per_wg) {
  if (splits <= 1) return 0;
  return (size_t)kTicketSlots * 4 + (size_t)tiles * splits * mt * strips_per_wg * 64 * 16;
}

template <int XDT, int MT, int NT, int WV>
static hipError_t launch_medium_nt(const MatmulArgs& a, const GemmPlan& p) {
  const unsigned tiles = (unsigned)(p.n_tiles * p.m_tiles);
  if (p.splits > 1)
    return launch_kernel(gemm_int8_medium_kernel<XDT, MT, NT, WV, kMediumDepth, true>,
                         dim3(tiles * p.splits), dim3(64 * WV), a.stream, a.x, a.Q, a.scales, a.y,
                         a.workspace, a.M, a.N, a.K, pack_tiles(p.n_tiles, a.y_dtype, false, p.splits));
  return launch_kernel(gemm_int8_medium_kernel<XDT, MT, NT, WV, kMediumDepth, false>, dim3(tiles),
                       dim3(64 * WV), a.stream, a.x, a.Q, a.scales, a.y, nullptr, a.M, a.N, a.K,
                       pack_tiles(p.n_tiles, a.y_dtype, false));
}

template <int XDT>
static hipError_t launch_medium_x(const MatmulArgs& a, const GemmPlan& p) {
  const int mt = p.mtile / 16;
  if (p.waves == 8 && p.nt == 1) {
    if (mt == 1) return hipErrorInvalidValue;  // 4 x units per stage: not 8 waves
    return mt == 2 ? launch_medium_nt<XDT, 2, 1, 8>(a, p) : launch_medium_nt<XDT, 4, 1, 8>(a, p);
  }
  if (p.waves == 4 && p.nt == 2)
    return mt == 1   ? launch_medium_nt<XDT, 1, 2, 4>(a, p)
           : mt == 2 ? launch_medium_nt<XDT, 2, 2, 4>(a, p)
                     : launch_medium_nt<XDT, 4, 2, 4>(a, p);
  if (p.waves == 4 && p.nt == 4)
    return mt == 1   ? launch_medium_nt<XDT, 1, 4, 4>(a, p)
           : mt == 2 ? launch_medium_nt<XDT, 2, 4, 4>(a, p)
                     : launch_medium_nt<XDT, 4, 4, 4>(a, p);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_medium(const MatmulArgs& a, const GemmPlan& p) {
  return a.x_dtype == XF16 ? launch_medium_x<XF16>(a, p) : launch_medium_x<XBF16>(a, p);
}

}  // namespace qmm
