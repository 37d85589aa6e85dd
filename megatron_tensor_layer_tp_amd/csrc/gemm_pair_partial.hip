// gemm_pair_partial.hip -- paired launches whose first product is a split-K
// weight gradient writing fp32 partials (a translation unit of its own so the
// pair kernels compile in parallel).  Dispatch in gemm_pair_impl.h.
#include "gemm_pair_impl.h"

hipError_t tp_launch_gemm_pair_tn_partial(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                                          const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st) {
  return first_tn<EPI_PARTIAL, true>(d1, v1, d2, v2, red, dry, st);
}
