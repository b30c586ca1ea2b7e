// gemm_large.hip -- large-M (prefill) matrix-core GEMM on the tile layout
// written by qmm_pack: y = x * dequant(Q), v_mfma_f32_16x16x32_{f16,bf16}.
// Planned by plan_gemm (gemm_mfma.hip), which calls large_split below.
#include <algorithm>
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Large-M kernel (prefill), matrix-core bound.
//  * workgroup tile 256 rows x 16 NT columns, one workgroup per CU, 4 waves
//    side by side along N: a wave owns all 256 rows x NT strips = 16 x NT
//    MFMA tiles, 64 NT fp32 accumulators per lane in the matrix-core (AGPR)
//    register file.  NT = 4 (full tiles) or 3 (narrow tiles: the plan ends
//    N with them so that the last round of workgroups is shorter);
//  * weights: each wave streams its own strips straight from the tile
//    layout into B operands (no LDS, no duplication across waves) and
//    dequantizes them to the MFMA's 16-bit type: w = (q - z) * s is formed
//    exactly in fp32 (a 4-bit by 11-bit product) and rounded once to
//    fp16 / bf16 (round to nearest even).  One operand register is made per
//    row tile, its instructions placed between that tile's MFMAs;
//  * x: the 256 x 128 tile of a stage is shared by the 4 waves through
//    double-buffered LDS, filled by buffer loads straight to LDS in a
//    swizzled row layout so that every operand read is one conflict-free
//    ds_read_b128;
//  * every load is a buffer load whose descriptor ends at its operand's edge
//    (rows past M and strips past N read zeros), addressed by a per-lane
//    offset fixed for the whole K loop plus a wave-uniform stage offset;
//  * stage s + 1's x tile and stage s + 2's weight words are loaded while
//    stage s runs.
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
constexpr int kLargeMT = kLargeRows / 16;
// eighths of a stage's row tiles over which its loads are issued
constexpr int kLoadSpan = 4;
// A fragments read from LDS ahead of the MFMAs that use them (int4 g128
// M=4096 K=4096 N=11008: 3 measured 1% faster than 2, 4 no better than 3)
constexpr int kFragAhead = 3;

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

// x tile of a stage in LDS: MT row tiles x 4 k steps of 1 KiB fragments
constexpr int kLargeFrags = kLargeMT * 4;

// One workgroup's tile: work item `bid` of `nblocks` over n_tiles column
// tiles of 16 NT columns starting at strip strip0, and every M tile.
template <int W_BIT, int XDT, int GS, bool ZP, int NT>
__device__ __forceinline__ void large_body(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int M, int N, int K, int n_tiles, int ydt, int gmask, int strip0, int bid, int nblocks,
    u32x4_t (*xa)[kLargeFrags * 64]) {
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

  static_assert(FRAGS == kLargeFrags, "LDS tile");

  // fp16 1024 in both halves, held in a register: mask-and-or of the codes
  // is then one v_and_or_b32 (an instruction takes one literal at most)
  uint32_t hi_bits;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(hi_bits));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, quad = lane >> 4;
  const int w = xcd_remap(bid, nblocks);
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
  // Loads issued during a stage, one at a time: j < NXL are this wave's x
  // fragments of stage sx, the rest weight-side (slots, then scales, then
  // zero words) of stage sw.  The k loop issues them spread over its first
  // row tiles: a wave issues in order, so a burst of loads at the top of a
  // stage would hold its MFMAs back until the memory pipeline had taken
  // them all; what is issued late in the stage has little time left to land
  // before the stage's closing wait.
  constexpr int NWL = NT * (2 + NGS);
  constexpr int NXL = FRAGS / 4;
  constexpr int NLD = NWL + NXL;
  auto load_part = [&](int j, int sw, int sx, int buf, WRegs& R) {
    if (j < NXL) {
      x_unit(j, sx, buf);
    } else {
      const int jw = j - NXL;
      if (jw < NT) load_slot(jw, sw, R);
      else if (jw < NT + NT * NGS) load_scale((jw - NT) / NGS, (jw - NT) % NGS, sw, R);
      else load_zero(jw - NT - NT * NGS, sw, R);
    }
  };
  // A stage ends waiting for its x tile but not for the weight-side loads
  // it issued after it (they are two stages ahead): vmcnt(NWL).
  static_assert(NWL < 64, "vmcnt field");
  constexpr int kWaitXTile = (NWL & 15) | ((NWL >> 4) << 14) | 0x0F70;

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
  // during the previous stage) and the one after (loading now).  A stage
  // issues the next x tile's loads first and the weight side last, and
  // ends waiting for the x tile only, so the weights it loaded have until
  // the next stage's last k step (where the compiler waits for exactly
  // them) to land.  The three sets take turns over an unrolled loop:
  // moving registers from one set to another would make the compiler wait
  // for their loads at the move.
  WRegs ra, rb, rc;  // the three stages' roles rotate (no register copies)
  load_x(0, 0);
  load_w(0, ra);
  load_w(min(1, nst - 1), rb);
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
  pin(ra);
  pin(rb);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  // The first stage's group constants and first B fragment are made here;
  // from then on each stage makes the next one's during its last k step,
  // so a stage opens straight into its MFMAs.
  GroupConst gc[NT][NGS];
  u32x4_t b[NT], bn[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    group_consts(ra, 0, s, gc[s]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      b[s][t] = bpair_scaled<W_BIT, XDT>(word_of(ra, s, 0, 0), 0, t, gc[s][0], hi_bits);
  }
  // One stage: cur holds its weights, nx1 the next stage's (loaded during
  // the previous stage), nx2 receives the weights two stages ahead.
  auto stage = [&](int st, const WRegs& cur, const WRegs& nx1, WRegs& nx2) {
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
    // k step k run, (1) the A fragment kFragAhead tiles ahead is read from LDS,
    // (2) part of the next k step's B fragments is dequantized (the NT x 4
    // operand registers spread over the MT row tiles) -- in the last k step
    // those of the next stage, after its group constants -- and (3) part of
    // the next stage's loads is issued.  The scheduling barriers hold this
    // interleave; without them the compiler hoists every read and every
    // conversion (and spills).
    // fragment (row tile i, k step kk) = slot 256 i + 16 l16 + ((4 kk + quad) ^ l16)
    auto afrag = [&](int i, int kk) { return xs_buf[256 * i + 16 * l16 + ((4 * kk + quad) ^ l16)]; };
    constexpr int P = kFragAhead;
    static_assert(P >= 1 && P <= STEPS * MT, "prefetch distance");
    u32x4_t ar[P];
#pragma unroll
    for (int q = 0; q < P; ++q) ar[q] = afrag(q % MT, q / MT);
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      const int kn = k + 1;
      const int qn = GS < KS ? (32 * kn) / GS : 0;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int t2 = k * MT + i + P;  // fragment P ahead, in (k, i) order
        const u32x4_t a0 = ar[0];
        u32x4_t an = ar[P - 1];
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
#pragma unroll
        for (int q = 0; q + 1 < P; ++q) ar[q] = ar[q + 1];
        ar[P - 1] = an;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) b[s] = bn[s];
    }
    // the next stage's x tile was written to LDS by the memory pipeline:
    // wait for this wave's part of it (the weight-side loads issued after
    // it may stay in flight), then for every wave's
    __builtin_amdgcn_s_waitcnt(kWaitXTile);
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 3) {
    stage(st, ra, rb, rc);
    if (st + 1 < nst) stage(st + 1, rb, rc, ra);
    if (st + 2 < nst) stage(st + 2, rc, ra, rb);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the last re-reads of the final stage
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


// The whole plan in one launch: work items [0, full) take full tiles (4
// strips per wave) over the first n_full column tiles, the rest narrow tiles
// (3 strips per wave) over the remaining columns.  Workgroups are dispatched
// in order, so the narrow ones start on whichever CUs free up first.  The
// branch is uniform per workgroup; both bodies share the one LDS tile.
template <int W_BIT, int XDT, int GS, bool ZP>
__global__ __launch_bounds__(256, 1) void gemm_large_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ Qt,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz, void* __restrict__ y,
    int M, int N, int K, int tile_opts, int tail_tiles) {
  __shared__ u32x4_t xa[2][kLargeFrags * 64];
  const int n_full = tiles_of(tile_opts), ydt = ydt_of(tile_opts), gmask = gmask_of(tile_opts);
  const int m_tiles = (M + kLargeRows - 1) / kLargeRows;
  const int full = n_full * m_tiles;
  const int b = (int)blockIdx.x;
  if (b < full)
    large_body<W_BIT, XDT, GS, ZP, 4>(x, Qt, scales, qz, y, M, N, K, n_full, ydt, gmask, 0, b,
                                      full, xa);
  else
    large_body<W_BIT, XDT, GS, ZP, 3>(x, Qt, scales, qz, y, M, N, K, tail_tiles, ydt, gmask,
                                      16 * n_full, b - full, tail_tiles * m_tiles, xa);
}

// ---------------------------------------------------------------- host side
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
void large_split(int m_tiles, int strips, int* n_full, int* n_tail) {
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

template <int W_BIT, int XDT, int GS, bool ZP>
static hipError_t launch_large_k(const MatmulArgs& a, const GemmPlan& p) {
  return launch_kernel(gemm_large_kernel<W_BIT, XDT, GS, ZP>,
                       dim3((unsigned)((p.n_tiles + p.tail_tiles) * p.m_tiles)), dim3(256),
                       a.stream, a.x, a.Q, a.scales, a.zeros, a.y, a.M, a.N, a.K,
                       pack_tiles(p.n_tiles, a.y_dtype, a.group_mask == 0), p.tail_tiles);
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

hipError_t launch_gemm_large(const MatmulArgs& a, const GemmPlan& p) {
  const bool f16 = a.x_dtype == XF16;
  if (a.w_bit == 4) return f16 ? launch_large<4, XF16>(a, p) : launch_large<4, XBF16>(a, p);
  if (a.w_bit == 2) return f16 ? launch_large<2, XF16>(a, p) : launch_large<2, XBF16>(a, p);
  return hipErrorInvalidValue;
}

}  // namespace qmm
