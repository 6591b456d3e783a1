// Batched (matrix-core) products with bf16 weights.
#include "gemm_impl.h"

namespace e2b {
hipError_t launch_gemm_bf16(int tag, const Lin& W, int rows, const GemmA& A, const GemmPlan& plan,
                           const Epilogue& epi, int* nblk, hipStream_t st) {
  return launch_gemm_q<0>(tag, W, rows, A, plan, epi, nblk, st);
}
}  // namespace e2b
