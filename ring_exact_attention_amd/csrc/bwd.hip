// Backward kernels (placeholder until the MFMA backward lands).
#include "bwd_args.h"
#include "common.h"

namespace bwa {

bool bwd_supported(int dtype, int D) {
  (void)dtype;
  (void)D;
  return false;
}

size_t bwd_workspace_bytes(int64_t BH, int64_t SQ, int64_t SKV, int D, int n, int mode) {
  (void)BH; (void)SQ; (void)SKV; (void)D; (void)n; (void)mode;
  return 0;
}

hipError_t bwd_run(const BwdArgs& a, hipStream_t st) {
  (void)a;
  (void)st;
  return hipErrorNotSupported;
}

}  // namespace bwa
