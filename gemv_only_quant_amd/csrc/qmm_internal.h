// qmm_internal.h -- host-side launch plans and kernel launchers (not public).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace qmm {

// Launches kernel `k` on `s` and returns the status of this launch alone: an
// error that an earlier call left on the thread is neither reported nor
// cleared.  The arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> v(static_cast<P>(std::forward<A>(args))...);
  return std::apply(
      [&](auto&... e) {
        void* p[] = {static_cast<void*>(&e)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, p, 0, s);
      },
      v);
}

// Arguments shared by every matmul launcher, already validated.
struct MatmulArgs {
  const void* x;
  const void* Q;
  const void* scales;
  const void* zeros;
  void* y;
  int y_dtype;     // YF32, or XF16 / XBF16 (rounded once as stored)
  int M, N, K, w_bit;
  int group_size;  // the group size the kernel runs (K itself, or a built size, per column)
  int group_mask;  // -1, or 0 for per-column scales: every group index masked to 0
  int x_dtype;
  void* workspace;
  hipStream_t stream;
};

// ---- low-bit GEMV on the canonical layout -------------------------------
struct GemvLowbitPlan {
  int mb;        // M bucket (compiled row count >= M)
  int rl;        // packed rows per lane (divides group_size / pack)
  int n_tiles;   // 16-column workgroup tiles
  size_t workspace_bytes;  // always 0: a workgroup owns its columns over all of K
};
GemvLowbitPlan plan_gemv_lowbit(int M, int N, int K, int w_bit, int group_size);
hipError_t launch_gemv_lowbit(const MatmulArgs& a, const GemvLowbitPlan& p);

// ---- low-bit GEMV on the tile layout (qmm_gemm, small M) ----------------
constexpr int kGemvTileMaxM = 4;
hipError_t launch_gemv_tile(const MatmulArgs& a);

// ---- int8 GEMV on (N, K) int8 ------------------------------------------
struct GemvInt8Plan {
  int mb;        // M bucket
  int rn;        // output rows (n) per wave
  int blocks;
};
GemvInt8Plan plan_gemv_int8(int M, int N, int K);
hipError_t launch_gemv_int8(const MatmulArgs& a, const GemvInt8Plan& p);

// ---- repack / dequant ----------------------------------------------------
int mfma_kblock(int w_bit);  // K extent of one 1 KiB layout block
hipError_t launch_pack(const void* q_canon, void* q_mfma, int N, int K, int w_bit,
                       hipStream_t s);
hipError_t launch_unpack_layout(const void* q_mfma, void* q_canon, int N, int K, int w_bit,
                                hipStream_t s);
hipError_t launch_dequant(const void* Q, int layout, const void* scales, const void* zeros,
                          float* w, int N, int K, int w_bit, int group_size, hipStream_t s);

// ---- MFMA GEMM on the tile layout ---------------------------------------
struct GemmPlan {
  int kind;      // 0: skinny (registers-direct, K split over the waves), 1: large-M tiled,
                 // 2: VALU GEMV on the tile layout (small M, low-bit), 3: int8 medium M
                 // (x shared through LDS, K split over workgroups)
  int mtile;     // rows per M tile
  int nt;        // 16-column strips per workgroup (skinny)
  int waves;     // waves per workgroup, splitting K (skinny: 4 or 8)
  int splits;    // workgroups per tile splitting K (skinny; 1 = none)
  int n_tiles;   // column tiles (large-M: full 256-column tiles)
  int m_tiles;
  int tail_tiles;  // large-M: narrow 192-column tiles after the full ones (0: none)
  size_t workspace_bytes;  // tickets + partial tiles when splits > 1, else 0
};
// Workspace of a plan that splits K over workgroups: kTicketSlots 32-bit
// arrival tickets (one per tile, the rest unused), then the plan's partial
// tiles.  The ticket head has one fixed size for every plan, so the partial
// tiles of one shape never land on the tickets of another and a workspace
// serves calls of any shapes in sequence; plans split only when their tiles
// fit in it.
constexpr int kTicketSlots = 1024;
// Most workgroups a tile's K is split over (the ticket counts at most 15
// earlier arrivals per XCD; the last workgroup reads every partial at once).
constexpr int kMaxSplits = 16;
// with_workspace: whether the call has a workspace; without one the plan
// never splits K over workgroups.
GemmPlan plan_gemm(int M, int N, int K, int w_bit, int group_size, bool with_workspace = true);
hipError_t launch_gemm(const MatmulArgs& a, const GemmPlan& p);

// ---- large-M MFMA GEMM (gemm_large.hip) ----------------------------------
constexpr int kLargeRows = 256;  // rows per workgroup tile
// Column split of a large-M plan: n_full 256-column tiles, then n_tail
// 192-column ones, over `strips` 16-column strips and m_tiles row tiles.
void large_split(int m_tiles, int strips, int* n_full, int* n_tail);
hipError_t launch_gemm_large(const MatmulArgs& a, const GemmPlan& p);

// ---- int8 MFMA GEMM at medium M (gemm_medium.hip) --------------------------
// Workspace of a plan of `tiles` tiles split `splits` ways: the ticket head,
// then the partial tiles (mt 16-row tiles x strips_per_wg 16-column strips
// each).
size_t medium_workspace_bytes(int tiles, int splits, int mt, int strips_per_wg);
hipError_t launch_gemm_medium(const MatmulArgs& a, const GemmPlan& p);

// ---- int8 x ternary (ternary.hip) -----------------------------------------
hipError_t launch_t2_pack(const void* Wp, void* Wt, int N, int K, hipStream_t s);
hipError_t launch_t2_unpack(const void* Wt, void* Wp, int N, int K, hipStream_t s);
hipError_t launch_i8t2_gemm(const void* x, const void* Wt, int32_t* y, int M, int N, int K,
                            hipStream_t s);
// large M (ternary_large.hip): 256-row tiles, the column split of large_split
hipError_t launch_i8t2_large(const void* x, const void* Wt, int32_t* y, int M, int N, int K,
                             hipStream_t s);

// ---- round-to-nearest quantizer (quantize.hip) -----------------------------
hipError_t launch_quantize(const void* W, int w_dtype, void* qw, void* scales, void* qzeros,
                           int N, int K, int w_bit, int group_size, int symmetric, hipStream_t s);

// Optional integer override from the environment (tile sweeps); -1 if unset.
// Call sites keep the value in a function-local static, so each override is
// read once per process, at the first call that plans that kernel.
int env_int(const char* name);

}  // namespace qmm
