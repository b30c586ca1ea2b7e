// gemv_tile.hip -- decode GEMV (M <= 4) for int4 / int2 weights in the tile
// layout written by qmm_pack (repack.hip), on the vector ALUs.
//
// Why a second GEMV: in the canonical layout (BitDistiller's qw (K/pack, N))
// a workgroup that owns 16 columns over all of K reads 64 bytes of every
// 16 KiB row, half a 128-byte line per row; reading 8.4 MB that way takes
// 3.8 us per launch on MI355X against 3.0-3.25 us for 128-byte or longer
// runs (graph-replayed read-only kernels, one launch per call).  In the tile
// layout one 16-column strip is a single contiguous run (K/KB blocks of
// 1 KiB), so every wave load is 1 KiB of consecutive bytes.
//
// Shape of the work:
//  * a workgroup owns one strip (16 columns) over all of K: no partial sum
//    leaves it.  Its 4 waves take the strip's blocks in passes of 4 * NBW
//    consecutive blocks, wave w blocks [base + w NBW, base + (w + 1) NBW);
//  * lane L serves column 16 s + L % 16 and k-octet c = L / 16 of each block
//    (the layout's lane map): int4 word j holds codes of k = 128 kb + 32 j +
//    8 c + i, nibble t (t < 4) code 2t and nibble 4 + t code 2t + 1, so
//    (w >> 4t) & 0x000F000F is the code pair (2t, 2t + 1); int2 the same in
//    2-bit fields, two 32-k halves per word;
//  * per pass the loads go out in the order x slice, 3/8 of the weights,
//    scales and zero words, the other weights; only the x slice gates the dot
//    products (it is shared by every workgroup and comes from cache), each
//    block then waits for its own weights (and the loads issued before
//    them: loads complete in order), and the scales are needed only by the
//    closing group epilogue;
//  * the x slice goes to LDS unchanged (pairs of consecutive k are already
//    the dot2 operand pairs), with its per-octet sums;
//  * codes become (B + q_a, B + q_b) 16-bit pairs (B = 1024 fp16, 128 bf16)
//    by one v_and_or_b32 each and meet x in v_dot2c_f32 (fp32 accumulation);
//    bias and zero leave per group through
//        sum x (q - z) = sum x (B + q) - (B + z) sum x,
//    where the column-wide term (B + z) sum x comes from a per-pass table of
//    group sums of x and is taken by one of the column's four k-octet lanes;
//    the group scale multiplies once;
//  * the 4 lanes of a column meet through two lane swaps, the 4 waves
//    through LDS.
// Measured (graph-replayed over > 512 MB of weight copies, 50 calls per
// replay; M=1 K=N=4096 int4 g128 fp16): a kernel of the same grid that only
// loads the weights 3.1 us, this one 3.9 us (3.7 in 2000-call replays),
// against 4.5 for the canonical-layout GEMV on the same box.
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int W_BIT> struct TileK;
template <> struct TileK<4> { static constexpr int KB = 128, PACK = 8; };
template <> struct TileK<2> { static constexpr int KB = 256, PACK = 16; };

// Operand pairs of one code word, and how they are summed.  fp16: fields
// (t, 4 + t) for t = 0, 2 are masked where they sit -- (B + q_a, B + q_b) --
// and fields for t = 1, 3 in place too, four bits up, reading B + 16 q: one
// shift per word serves t = 2, 3.  The "unit" and "x16" pairs go to separate
// sums (acc[0], acc[1]) and the x16 sum is divided by 16 in the group
// epilogue, exactly (every code product is exact in fp32).  bf16 (7-bit
// significand) keeps one shift per pair, all pairs unit.
template <int W_BIT, int XDT> struct Pairs {
  static constexpr bool SPLIT = W_BIT == 4 && XDT == XF16;
};

// Phase stamps (QMM_PHASE_STAMPS builds only, never the product library):
// lane 0 of every wave records the 100 MHz real-time counter at fixed
// points of the kernel into a device array the host reads back.  Stamp
// slots per wave: 0 entry, 1 x slice and its sums in LDS, 2 group-sum table
// ready, 3 every weight block's dot products done (its loads returned),
// 4 scales and zero words ready (in LDS, where they go through it),
// 5 output stored, 6 the first block's dot products done, 7 the first half
// of the blocks' done.
#ifdef QMM_PHASE_STAMPS
constexpr int kStampSlots = 8;
constexpr int kStampWaves = 4 * 8192;  // up to 8192 workgroups of 4 waves
__device__ uint64_t phase_stamps[kStampWaves * kStampSlots];
#define QMM_STAMP(slot)                                                              \
  do {                                                                               \
    const uint64_t t_ = __builtin_amdgcn_s_memrealtime();                            \
    const int w_ = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));       \
    if ((threadIdx.x & 63) == 0 && w_ < kStampWaves) phase_stamps[w_ * kStampSlots + (slot)] = t_; \
  } while (0)
#else
#define QMM_STAMP(slot) \
  do {                  \
  } while (0)
#endif

// m_ydt: M in bits 0-7, output type in bits 8-9; gs_opt: log2 of the group
// size, or -1 for per-column scales (one group spanning K).  SPB: groups per
// block, max(1, KB / group size) (1 for per-column scales).
template <int W_BIT, int XDT, int MB, int NBW, int SPB, bool Y32, int WV>
__global__ __launch_bounds__(64 * WV) void gemv_tile_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const uint16_t* __restrict__ sc, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int m_ydt, int N, int K, int gs_opt) {
  constexpr int KB = TileK<W_BIT>::KB, PACK = TileK<W_BIT>::PACK;
  constexpr int NTH = 64 * WV;                   // threads per workgroup
  constexpr int PASS_K = WV * NBW * KB;          // k per pass
  constexpr int PO = PASS_K / 8;                 // 8-k octets per pass
  constexpr int OPB = KB / 8;                    // octets per block
  constexpr int UPB = KB / 32;                   // 32-k units per block (per lane: one octet each)
  constexpr uint32_t FIELD2 = W_BIT == 4 ? 0x000F000Fu : 0x00030003u;
  constexpr uint32_t ZMASK = (1u << W_BIT) - 1u;
  constexpr bool SPLIT = Pairs<W_BIT, XDT>::SPLIT;
  constexpr int NS = SPLIT ? 2 : 1;              // sums per octet / accumulators per group
  constexpr int GPP = WV * NBW * SPB;            // groups per pass at most
  constexpr int TE = MB * WV * NBW * SPB;        // group-sum entries per pass
  constexpr int ZR = GPP / PACK + 2;             // zero rows per pass at most
  constexpr float B = Bias<XDT>::value;
  const int M = m_ydt & 0xFF;
  const int ydt = Y32 ? (int)YF32 : (m_ydt >> 8) & 3;
  // group of k: (k >> gsh) & gmask -- group sizes are powers of two, and
  // per-column scales mask every index to 0 (no division, no branch)
  const int gsh = gs_opt < 0 ? 0 : gs_opt;
  const int gmask = gs_opt < 0 ? 0 : -1;
  const int G = gs_opt < 0 ? 1 : K >> gsh;

  QMM_STAMP(0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, oct = lane >> 4;
  const int s = xcd_remap(blockIdx.x, N >> 4);  // the grid: one workgroup per strip
  const int nblk = K / KB;

  // one pass in LDS: the x slice (row m at m * PASS_K, as stored), its octet
  // sums, per (row, block, group of the block) the pair (P, X) -- X = sum of
  // x over the group, P = B X (fp16 split: B X_unit + B/16 X_x16) -- in copy
  // 0 of gtab, zeros in copy 1, and the pass's scales [group][column] and
  // zero words [row][column]
  __shared__ __attribute__((aligned(16))) uint16_t xl[MB * PASS_K];
  __shared__ __attribute__((aligned(16))) float xsum[MB * PO * NS];
  __shared__ __attribute__((aligned(16))) float2 gtab[2][TE];
  // DIRECT: each lane loads the scales and zero words of its own blocks'
  // groups straight into registers (at most 8 of each), so the epilogue
  // needs neither an LDS exchange nor a barrier for them; otherwise they go
  // through LDS cooperatively
  constexpr bool DIRECT = NBW * SPB <= 8;
  __shared__ uint16_t sl[DIRECT ? 1 : GPP * 16];
  __shared__ uint32_t zl[DIRECT ? 1 : ZR * 16];
  __shared__ float red[WV][MB][16];  // per wave: its columns' sums

  // descriptors: a block past the strip, a row past M, a group past G read 0
  const buf_t qbuf = make_buf(Qt + (size_t)s * nblk * 64, (uint32_t)nblk * 1024u);
  const buf_t xbuf = make_buf(x, (uint32_t)M * K * 2u);
  const buf_t sbuf = make_buf(sc + 16 * s, (uint32_t)((size_t)G * N - 16 * s) * 2u);
  const int zrows = (G + PACK - 1) / PACK;
  const bool zp = qz != nullptr;
  const buf_t zbuf = make_buf(zp ? qz + 16 * s : reinterpret_cast<const uint32_t*>(Qt),
                              zp ? (uint32_t)((size_t)zrows * N - 16 * s) * 4u : 0u);
  constexpr int OUT = 0x7FFFFFF0;  // an offset past every descriptor's range: reads 0

  float r[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) r[m] = 0.f;
  // The field masks live in vector registers (an opaque move), so that each
  // mask-and-bias is one v_and_or_b32: with both constants as literals the
  // compiler must split it into an AND and an OR (no two literals per
  // three-operand instruction), twice the instructions in the inner loop.
  uint32_t mlo, mhi;
  asm("v_mov_b32 %0, %1" : "=v"(mlo) : "i"(FIELD2));
  asm("v_mov_b32 %0, %1" : "=v"(mhi) : "i"(FIELD2 << 4));

  constexpr int XCH = MB * PO;                   // 16-byte x chunks (one octet each)
  constexpr int XPT = (XCH + NTH - 1) / NTH;
  constexpr int SU = (GPP * 8 + NTH - 1) / NTH;  // 4-byte scale units (2 columns) per thread
  constexpr int ZU = (ZR * 16 + NTH - 1) / NTH;  // zero words per thread
  for (int k0 = 0; k0 < K; k0 += PASS_K) {
    const int gp0 = (k0 >> gsh) & gmask;         // first group of the pass
    const int zr0 = gp0 / PACK;                  // first zero row of the pass
    // 1. small loads first: x slice, scales, zero words (cooperative)
    u32x4_t xr[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int q = threadIdx.x + NTH * j;
      const int m = q / PO, k = k0 + 8 * (q % PO);
      xr[j] = buf_load128(xbuf, (q < XCH && m < M && k < K) ? (m * K + k) * 2 : OUT);
    }
    // 2. weights: one 1 KiB block per load instruction, the first 3/8 of
    // them here; then the scales and zero words, then the rest of the
    // weights.  Loads complete in order: the scale and zero loads (which
    // only the pass's closing epilogue reads) return while the later blocks
    // still stream in, and their scalar offset arithmetic does not hold back
    // the first blocks.  Measured at M=1 K=N=4096 int4 g128 with the weights
    // streamed (us per call, 2000-call replays, same box): weights 3 / 8
    // before them 3.656-3.657, 2 / 8 3.675-3.681, 4 / 8 3.652-3.668, 5 / 8
    // 3.665-3.679, 6 / 8 3.687-3.713, 7 / 8 3.82, all 8 3.94.
    const int kb0 = k0 / KB + wave * NBW;        // this wave's first block
    constexpr int WEARLY = NBW * 3 / 8;
    u32x4_t wq[NBW];
#pragma unroll
    for (int i = 0; i < WEARLY; ++i) wq[i] = buf_load128_stream(qbuf, ((kb0 + i) * 64 + lane) * 16);
    __builtin_amdgcn_sched_barrier(0);

    uint32_t su[DIRECT ? 1 : SU], zu[DIRECT ? 1 : ZU];
    uint32_t sd[DIRECT ? NBW * SPB : 1], zd[DIRECT ? NBW * SPB : 1];
    if constexpr (DIRECT) {
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int e = 0; e < SPB; ++e) {
          const int g = ((((kb0 + i) * KB) >> gsh) & gmask) + e;
          sd[i * SPB + e] = buf_load16(sbuf, (g * N + col) * 2);
          zd[i * SPB + e] = buf_load32(zbuf, ((g / PACK) * N + col) * 4);
        }
    } else {
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int u = threadIdx.x + NTH * j;
        const int gl = u >> 3, cp = u & 7;
        su[j] = buf_load32(sbuf, u < GPP * 8 ? ((gp0 + gl) * N + 2 * cp) * 2 : OUT);
      }
#pragma unroll
      for (int j = 0; j < ZU; ++j) {
        const int u = threadIdx.x + NTH * j;
        zu[j] = buf_load32(zbuf, u < ZR * 16 ? ((zr0 + (u >> 4)) * N + (u & 15)) * 4 : OUT);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = WEARLY; i < NBW; ++i) wq[i] = buf_load128_stream(qbuf, ((kb0 + i) * 64 + lane) * 16);
    // 3. the pass to LDS
    if (k0 > 0) __syncthreads();  // the previous pass is done reading
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int q = threadIdx.x + NTH * j;
      if (XCH % NTH == 0 || q < XCH) {
        *reinterpret_cast<u32x4_t*>(xl + 8 * q) = xr[j];
        const int dst = q;  // (row, octet) in slice order
        if constexpr (SPLIT) {
          float a = dot2<XDT>(xr[j][0], Bias<XDT>::one_pair, 0.f);
          a = dot2<XDT>(xr[j][2], Bias<XDT>::one_pair, a);
          float b = dot2<XDT>(xr[j][1], Bias<XDT>::one_pair, 0.f);
          b = dot2<XDT>(xr[j][3], Bias<XDT>::one_pair, b);
          xsum[2 * dst] = a;
          xsum[2 * dst + 1] = b;
        } else {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) a = dot2<XDT>(xr[j][e], Bias<XDT>::one_pair, a);
          xsum[dst] = a;
        }
      }
    }
    __syncthreads();
    QMM_STAMP(1);
    // group sums of the pass: entry (m, block, e) adds the OPB / SPB octet
    // sums of group e of the block
#pragma unroll
    for (int j = 0; j < (TE + NTH - 1) / NTH; ++j) {
      const int u = threadIdx.x + NTH * j;
      if (TE % NTH == 0 || u < TE) {
        const int m = u / (WV * NBW * SPB), be = u % (WV * NBW * SPB);
        const float* o = xsum + NS * (m * PO + be * (OPB / SPB));
        float xu = 0.f, x16 = 0.f;
#pragma unroll
        for (int q = 0; q < OPB / SPB; ++q) {
          xu += o[NS * q];
          if constexpr (SPLIT) x16 += o[NS * q + 1];
        }
        gtab[0][u] = SPLIT ? float2{B * xu + (B / 16) * x16, xu + x16} : float2{B * xu, xu};
        gtab[1][u] = float2{0.f, 0.f};
      }
    }
    __syncthreads();
    QMM_STAMP(2);

    // 4. per block: dot products into per-block, per-group sums.  The x
    // operands of block i + 1 are read from LDS while block i is multiplied
    // (when they fit in 32 registers): read just before their use, the LDS
    // latency stood between every two words' dot products.
    float bacc[NBW][MB][SPB];
    constexpr bool XPF = MB * UPB * 4 <= 32;
    u32x4_t xc[XPF ? MB : 1][XPF ? UPB : 1], xn[XPF ? MB : 1][XPF ? UPB : 1];
    auto read_x = [&](int i, u32x4_t (&dst)[XPF ? MB : 1][XPF ? UPB : 1]) {
      const int kl = (kb0 + i) * KB - k0;
#pragma unroll
      for (int m = 0; m < (XPF ? MB : 1); ++m)
#pragma unroll
        for (int un = 0; un < (XPF ? UPB : 1); ++un)
          dst[m][un] = *reinterpret_cast<const u32x4_t*>(xl + m * PASS_K + kl + 32 * un + 8 * oct);
    };
    if constexpr (XPF) read_x(0, xc);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int kb = kb0 + i;
      const int kl = kb * KB - k0;               // block start within the pass
      if constexpr (XPF) {
        if (i + 1 < NBW) read_x(i + 1, xn);
      }
      float acc[MB][SPB][NS];
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int e = 0; e < SPB; ++e)
#pragma unroll
          for (int a = 0; a < NS; ++a) acc[m][e][a] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = wq[i][j];
        constexpr int HALVES = W_BIT == 4 ? 1 : 2;  // int2: two 32-k halves per word
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
          const int un = W_BIT == 4 ? j : 2 * j + h;  // 32-k unit of the block
          const int e = un * SPB / UPB;               // its group within the block
          uint32_t p[4];
          if constexpr (SPLIT) {
            const uint32_t w8 = w >> 8;
            p[0] = (w & mlo) | Bias<XDT>::pair;
            p[1] = (w & mhi) | Bias<XDT>::pair;
            p[2] = (w8 & mlo) | Bias<XDT>::pair;
            p[3] = (w8 & mhi) | Bias<XDT>::pair;
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              p[t] = ((w >> (W_BIT * (4 * h + t))) & mlo) | Bias<XDT>::pair;
          }
          // rows past M hold zeros in xl and add nothing
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            u32x4_t xv;
            if constexpr (XPF) xv = xc[m][un];
            else xv = *reinterpret_cast<const u32x4_t*>(xl + m * PASS_K + kl + 32 * un + 8 * oct);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[m][e][SPLIT ? (t & 1) : 0] =
                  dot2<XDT>(xv[t], p[t], acc[m][e][SPLIT ? (t & 1) : 0]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int e = 0; e < SPB; ++e) {
          bacc[i][m][e] = SPLIT ? acc[m][e][0] + 0.0625f * acc[m][e][1] : acc[m][e][0];
          // consumed here: the block's products stay ahead of the wait for
          // the scale loads (else they would be sunk to the epilogue)
          asm volatile("" : "+v"(bacc[i][m][e]));
        }
      if constexpr (XPF) {
        if (i + 1 < NBW) {
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int un = 0; un < UPB; ++un) xc[m][un] = xn[m][un];
        }
      }
      if (i == 0) QMM_STAMP(6);
      if (i == NBW / 2 - 1) QMM_STAMP(7);
    }
    QMM_STAMP(3);

    // 5. the pass's scales and zero words to LDS (the x slice and group table
    // are no longer written; every wave is past the table reads of step 3)
    // symmetric: every zero field holds 2^(w_bit-1) (the descriptor read 0)
    const uint32_t zfill = zp ? 0u : (W_BIT == 4 ? 0x88888888u : 0xAAAAAAAAu);
    if constexpr (!DIRECT) {
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int u = threadIdx.x + NTH * j;
        if (u < GPP * 8) reinterpret_cast<uint32_t*>(sl)[u] = su[j];
      }
#pragma unroll
      for (int j = 0; j < ZU; ++j) {
        const int u = threadIdx.x + NTH * j;
        if (u < ZR * 16) zl[u] = zu[j] | zfill;
      }
      __syncthreads();
    }
    QMM_STAMP(4);

    // 6. group epilogue: r += s (sum x (B + q) - B X - z X), where the
    // column-wide term (P + z X) is taken by the octet-0 lane alone (the
    // column's 4 octet lanes are added at the end); lanes of the other
    // octets read copy 1 of the table, all zeros
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int kb = kb0 + i;
      const int g0 = ((kb * KB) >> gsh) & gmask;
#pragma unroll
      for (int e = 0; e < SPB; ++e) {
        const int g = g0 + e;
        const float sv = f16_bits_to_f32(DIRECT ? (uint16_t)sd[i * SPB + e]
                                                : sl[(g - gp0) * 16 + col]);
        const uint32_t zw = DIRECT ? zd[i * SPB + e] | zfill : zl[(g / PACK - zr0) * 16 + col];
        const float zf = (float)((zw >> ((g % PACK) * W_BIT)) & ZMASK);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float2 pe = gtab[oct != 0][(m * WV * NBW + (kb - k0 / KB)) * SPB + e];
          r[m] += sv * (bacc[i][m][e] - (pe.x + zf * pe.y));
        }
      }
    }
  }

  // 7. the column's 4 k-octet lanes (the same lane of the wave's 4 rows of
  // 16) meet by two lane swaps (rows4_sum); then the waves meet in LDS, and
  // one thread per output adds them.
#pragma unroll
  for (int m = 0; m < MB; ++m) r[m] = rows4_sum(r[m]);
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < MB; ++m) red[wave][m][col] = r[m];
  }
  __syncthreads();
  auto store = [&](auto* yt) {
    using T = typename std::remove_pointer<decltype(yt)>::type;
    if (threadIdx.x < 16 * MB) {
      const int m = threadIdx.x >> 4, c = threadIdx.x & 15;
      if (m < M) {
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < WV; ++v) sum += red[v][m][c];
        yt[(size_t)m * N + 16 * s + c] = (T)sum;
      }
    }
  };
  if constexpr (Y32) store(reinterpret_cast<float*>(y));
  else with_y(y, ydt, store);
  QMM_STAMP(5);
}

// ---------------------------------------------------------------- host side
// Blocks per wave per pass (NBW): a pass is 4 * NBW blocks, and every wave
// should have blocks inside K -- int2 (256-deep blocks) takes 4, a pass of
// 4096 k; int4 takes 8 (4096 k) when K has at least 32 blocks, else 4.  The
// x slice of 4 rows is then at most 32 KiB of LDS.
template <int W_BIT, int XDT, int MB, int SPB, int NBW, int WV>
static hipError_t launch_tile_nbw(const MatmulArgs& a) {
  const int gs_opt = a.group_mask == 0 ? -1 : __builtin_ctz((unsigned)a.group_size);
  const int m_ydt = a.M | ((a.y_dtype == YF32 ? 0 : a.y_dtype) << 8);
  const dim3 grid((unsigned)(a.N >> 4)), block(64 * WV);
  if (a.y_dtype == YF32)
    return launch_kernel(gemv_tile_kernel<W_BIT, XDT, MB, NBW, SPB, true, WV>, grid, block,
                         a.stream, a.x, a.Q, a.scales, a.zeros, a.y, m_ydt, a.N, a.K, gs_opt);
  return launch_kernel(gemv_tile_kernel<W_BIT, XDT, MB, NBW, SPB, false, WV>, grid, block,
                       a.stream, a.x, a.Q, a.scales, a.zeros, a.y, m_ydt, a.N, a.K, gs_opt);
}

template <int W_BIT, int XDT, int MB, int SPB>
static hipError_t launch_tile_spb(const MatmulArgs& a) {
  if constexpr (W_BIT == 4) {
    // 4 waves of 8 blocks per pass: measured at M=1 K=N=4096 int4 g128
    // against 2 waves of 16 blocks (5.63 us) and 8 waves of 4 (5.07 us):
    // 4.84 us on the same box
    if (a.K / TileK<4>::KB >= 32) return launch_tile_nbw<W_BIT, XDT, MB, SPB, 8, 4>(a);
  }
  return launch_tile_nbw<W_BIT, XDT, MB, SPB, 4, 4>(a);
}

template <int W_BIT, int XDT, int MB>
static hipError_t launch_tile_mb(const MatmulArgs& a) {
  constexpr int KB = TileK<W_BIT>::KB;
  const int spb = (a.group_mask == 0 || a.group_size >= KB) ? 1 : KB / a.group_size;
  switch (spb) {
    case 1: return launch_tile_spb<W_BIT, XDT, MB, 1>(a);
    case 2: return launch_tile_spb<W_BIT, XDT, MB, 2>(a);
    case 4: return launch_tile_spb<W_BIT, XDT, MB, 4>(a);
    case 8:
      if constexpr (W_BIT == 2) return launch_tile_spb<W_BIT, XDT, MB, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <int W_BIT, int XDT>
static hipError_t launch_tile_x(const MatmulArgs& a) {
  if (a.M <= 1) return launch_tile_mb<W_BIT, XDT, 1>(a);
  if (a.M <= 2) return launch_tile_mb<W_BIT, XDT, 2>(a);
  return launch_tile_mb<W_BIT, XDT, 4>(a);
}

hipError_t launch_gemv_tile(const MatmulArgs& a) {
  if (a.M > kGemvTileMaxM) return hipErrorInvalidValue;
  if (a.w_bit == 4)
    return a.x_dtype == XF16 ? launch_tile_x<4, XF16>(a) : launch_tile_x<4, XBF16>(a);
  return a.x_dtype == XF16 ? launch_tile_x<2, XF16>(a) : launch_tile_x<2, XBF16>(a);
}

#ifdef QMM_PHASE_STAMPS
// The reference the stamps are read against: the same grid (one 256-thread
// workgroup per 16-column strip), each workgroup reading its strip's
// nblk KiB in 1 KiB wave loads (with the GEMV's non-temporal hint), 8 per
// wave in flight, summing and storing one value per lane.  Slots: 0 entry,
// 3 last load returned, 5 stored.
__global__ __launch_bounds__(256) void phase_readonly_kernel(const u32x4_t* __restrict__ src,
                                                             uint32_t* __restrict__ dst,
                                                             int nblk) {
  QMM_STAMP(0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const buf_t b = make_buf(src + (size_t)blockIdx.x * nblk * 64, (uint32_t)nblk * 1024u);
  uint32_t acc = 0;
  for (int kb = wave * 8; kb < nblk; kb += 32) {
    u32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = buf_load128_stream(b, ((kb + i) * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  asm volatile("" ::"v"(acc));  // every load has returned
  QMM_STAMP(3);
  dst[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
  QMM_STAMP(5);
}
#endif

}  // namespace qmm

#ifdef QMM_PHASE_STAMPS
// Host side of the stamp build: read the stamps back, and launch the
// read-only reference on `strips` workgroups of nblk blocks each.
extern "C" __attribute__((visibility("default"))) int qmm_phase_stamps_read(uint64_t* dst,
                                                                            size_t count) {
  if (count > (size_t)qmm::kStampWaves * qmm::kStampSlots) return -1;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(qmm::phase_stamps), count * sizeof(uint64_t), 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" __attribute__((visibility("default"))) int qmm_phase_readonly(const void* src,
                                                                         void* dst, int strips,
                                                                         int nblk, void* stream) {
  if (strips <= 0 || strips > 8192 || nblk <= 0) return -1;
  return (int)qmm::launch_kernel(qmm::phase_readonly_kernel, dim3((unsigned)strips), dim3(256),
                                 reinterpret_cast<hipStream_t>(stream), src, dst, nblk);
}
#endif
