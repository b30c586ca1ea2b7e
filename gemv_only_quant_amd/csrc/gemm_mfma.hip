// gemm_mfma.hip -- MFMA path (placeholder until the matrix-core kernels land).
#include "qmm_internal.h"

namespace qmm {

GemmPlan plan_gemm(int M, int N, int K, int w_bit, int group_size) {
  (void)M; (void)N; (void)K; (void)w_bit; (void)group_size;
  GemmPlan p{};
  p.kind = -1;
  return p;
}

hipError_t launch_gemm(const MatmulArgs& a, const GemmPlan& p) {
  (void)a; (void)p;
  return hipErrorInvalidValue;
}

}  // namespace qmm
