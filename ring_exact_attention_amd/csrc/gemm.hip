// K/V recompute GEMM (placeholder until the MFMA GEMM lands).
#include "bwa.h"
#include "common.h"

namespace bwa {

hipError_t gemm_kv_launch(const void* y, const void* wk_t, const void* wv_t, int64_t B, int64_t S,
                          int64_t E, int64_t H, int64_t D, const bwa_tensor* k,
                          const bwa_tensor* v, hipStream_t st) {
  (void)y; (void)wk_t; (void)wv_t; (void)B; (void)S; (void)E; (void)H; (void)D; (void)k;
  (void)v; (void)st;
  return hipErrorNotSupported;
}

}  // namespace bwa
