// qmm_device.h -- device helpers shared by the qmm HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum { XF16 = 0, XBF16 = 1, YF32 = 2 };

// Runs f(yt) with y viewed as the caller's output type (float, _Float16 or
// __bf16); stores through it convert the fp32 result once, to nearest even.
// ydt is uniform across the launch, so the branch is taken once per call
// site and each store loop is compiled for one type.
template <class F>
__device__ __forceinline__ void with_y(void* y, int ydt, F&& f);

// Options carried in the top bits of a kernel's tile-count argument, so no
// kernel needs more than 56 bytes of explicit arguments (64 with a
// workspace, the workspace pointer last): 56 bytes are what the build
// preloads into SGPRs (14 user SGPRs beside the argument pointer), and one
// argument more (a 320-byte instead of a 312-byte argument segment, with the
// hidden arguments) had measured +0.3 us on every launch of a 6 us kernel
// before arguments were preloaded.
//   bits 0-23 tile count, bits 24-27 K splits - 1, bits 28-29 output type,
//   bit 30 per-column scales
constexpr int kTileBits = 24;
__host__ __device__ constexpr int pack_tiles(int tiles, int ydt, bool per_column, int splits = 1) {
  return tiles | ((splits - 1) << kTileBits) | (ydt << 28) | ((per_column ? 1 : 0) << 30);
}
__device__ __forceinline__ int tiles_of(int t) { return t & ((1 << kTileBits) - 1); }
__device__ __forceinline__ int splits_of(int t) { return ((t >> kTileBits) & 15) + 1; }
__device__ __forceinline__ int ydt_of(int t) { return (t >> 28) & 3; }
// group-index mask: 0 (every group is group 0) for per-column scales
__device__ __forceinline__ int gmask_of(int t) { return ((t >> 30) & 1) ? 0 : -1; }

template <class F>
__device__ __forceinline__ void with_y(void* y, int ydt, F&& f) {
  if (ydt == YF32) f(reinterpret_cast<float*>(y));
  else if (ydt == XF16) f(reinterpret_cast<_Float16*>(y));
  else f(reinterpret_cast<__bf16*>(y));
}

// "Magic" exponent bias: OR-ing a small unsigned integer c into the low
// mantissa bits of these 16-bit patterns gives the float B + c exactly
// (fp16: 0x6400 = 1024, unit step for c < 1024; bf16: 0x4300 = 128, unit
// step for c < 128).  The same exponent-bias idea appears in Marlin's int4
// dequant() for fp16.
template <int XDT> struct Bias;
template <> struct Bias<XF16> {
  static constexpr uint32_t pair = 0x64006400u;  // (1024, 1024)
  static constexpr float value = 1024.0f;
  static constexpr uint32_t one_pair = 0x3C003C00u;  // (1.0, 1.0)
};
template <> struct Bias<XBF16> {
  static constexpr uint32_t pair = 0x43004300u;  // (128, 128)
  static constexpr float value = 128.0f;
  static constexpr uint32_t one_pair = 0x3F803F80u;
};

// acc + a.lo * b.lo + a.hi * b.hi with fp32 accumulation (v_dot2c_f32_*).
template <int XDT> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot2<XF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                acc, false);
}
template <> __device__ __forceinline__ float dot2<XBF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two 16-bit lanes: low halves of (a, b) and high halves of (a, b).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// One DPP-moved copy of v added to v; CTRL / ROW_MASK are DPP controls.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the wave's 4 rows of 16 lanes at each lane position (lane l gets
// v(l % 16) + v(16 + l % 16) + v(32 + l % 16) + v(48 + l % 16)) by two lane
// swaps.  v_permlane16_swap exchanges the odd rows of its first operand with
// the even rows of its second: with both holding v, their sum is v(row 0) +
// v(row 1) in rows 0-1 and v(2) + v(3) in rows 2-3.  v_permlane32_swap
// exchanges the upper half of the first with the lower half of the second:
// the sum of both is then the 4 rows' total in every lane.  Written as asm:
// this compiler's builtins for the two swaps hand back the first register
// for both results.  The s_nop covers the hazard of a swap reading a
// register a VALU instruction has just written.
__device__ __forceinline__ float rows4_sum(float v) {
  float a0 = v, a1 = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a0), "+v"(a1));
  float c0 = a0 + a1, c1 = c0;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c0), "+v"(c1));
  return c0 + c1;
}

// Full-wave sum with DPP: butterfly inside each row of 16 lanes, then the
// row_bcast steps fold the four rows into lane 63, which is read back.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x124, 0xF>(v);  // row_ror:4
  v = dpp_add<0x128, 0xF>(v);  // row_ror:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Raw buffer loads (no format conversion) through a descriptor whose range
// is `bytes`: an offset at or past it reads zeros.  Word 3 is the raw-buffer
// configuration of the CDNA buffer descriptor (32-bit data format, no
// swizzle, no stride).
typedef __amdgpu_buffer_rsrc_t buf_t;
__device__ __forceinline__ buf_t make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load128(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, 0);
}
// Weights that a call reads exactly once go through the caches with the
// non-temporal hint (the `nt` cache-policy bit): their lines are not
// allocated for reuse, so the caches need not make room for them.  Measured
// on the headline GEMV (M=1 K=N=4096 int4 g128, weights rotated over > 512
// MB, replays after a cache-evicting pass): 4.72-4.75 -> 3.99-4.04 us per
// call in 50-call graph replays, unchanged in 2000-call ones; the int8
// medium GEMMs 4-10% and the int4 skinny ones 3% faster.  (A model whose
// weights would stay in the 256 MB Infinity Cache from one call to the next
// gives that reuse up; the prefill, which re-reads each weight tile once per
// row tile, keeps the default policy: with the hint it measured 3-8% slower.)
constexpr int kStream = 2;  // nt
__device__ __forceinline__ u32x4_t buf_load128_stream(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, kStream);
}
__device__ __forceinline__ uint32_t buf_load32(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(b, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load16(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b16(b, off, 0, 0);
}

// Accesses coherent across the XCDs' L2 caches without a fence: the sc1
// cache-policy bit (the one the compiler gives agent-scope atomic loads and
// stores on gfx950) makes a store write through this XCD's L2 and a load
// fetch past any copy an L2 may hold.  An agent-scope fence would instead
// write back and invalidate the whole L2 of the XCD.
constexpr int kCoherent = 16;  // sc1
__device__ __forceinline__ void buf_store128_coherent(u32x4_t v, buf_t b, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, b, off, 0, kCoherent);
}
__device__ __forceinline__ u32x4_t buf_load128_coherent(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, kCoherent);
}
// A load that misses this CU's L1 but may hit this XCD's L2 (the sc0 bit):
// coherent with stores that other CUs of the same XCD wrote through.
__device__ __forceinline__ u32x4_t buf_load128_xcd(buf_t b, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, 1);
}
// The XCD (accelerator complex die) this wave runs on, 0-7 (a hardware
// register read).
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 7u;
}
// Arrival ticket of a K-split tile: each workgroup adds one to the 4-bit
// count of its own XCD (bits 4x .. 4x + 3 for XCD x), so the value before
// an add tells both how many arrived (the sum of the counts) and whether
// they all ran on one XCD (one count holds it all).  At most 15 earlier
// arrivals.
__device__ __forceinline__ uint32_t ticket_arrivals(uint32_t t) {
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) n += (t >> (4 * i)) & 15u;
  return n;
}

// Work-item remap so that consecutive work ids land on one XCD: the
// dispatcher deals workgroups round-robin over the 8 XCDs, so block b runs
// on XCD b % 8.  Used only when the grid is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  if (total % 8 != 0) return b;
  return (b % 8) * (total / 8) + b / 8;
}

}  // namespace qmm
