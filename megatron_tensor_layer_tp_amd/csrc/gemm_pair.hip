// gemm_pair.hip -- launchers of paired bf16 products: two independent GEMMs of
// one pass (a weight gradient beside an activation gradient, or the QKV and
// output projections) in one launch, so that neither leaves CUs idle while the
// other drains.  Kernels in gemm_bf16_kernels.h, dispatch in gemm_pair_impl.h.
//
// Supported pairs (first = the long-K product, second = the short-K one), both
// with 256-row tiles and 16-byte-aligned operands:
//   first  TN store (bf16) or TN split-K partial (fp32; gemm_pair_partial.hip),
//          256, 192 or 128 columns
//   second NT store or NT activation backward (256, 192 or 128 columns), NT store
//          over K-segments or NT SwiGLU backward (256 or 128 columns);
//   first  NN store, second NN store (256 or 128 columns each).
#include "gemm_pair_impl.h"

namespace {

template <class C1>
hipError_t second_nn(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, bool dry, hipStream_t st) {
  if (v2.layout != GEMM_NN || v2.epi != EPI_STORE || v2.out_f32 || d2.kseg || v2.bm != 256)
    return hipErrorNotSupported;
  if (v2.bn == 256) return go<C1, CfgL<256, 256, GEMM_NN, EPI_STORE, false, false>>(d1, d2, dry, st);
  if (v2.bn == 128) return go<C1, CfgL<256, 128, GEMM_NN, EPI_STORE, false, false>>(d1, d2, dry, st);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t tp_launch_gemm_pair(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                               const GemmVariant &v2, bool dry, hipStream_t st) {
  if (!v1.vec || !v2.vec || d1.kseg || v1.bm != 256) return hipErrorNotSupported;
  if (v1.layout == GEMM_TN) {
    if (v1.epi == EPI_PARTIAL && v1.out_f32) return tp_launch_gemm_pair_tn_partial(d1, v1, d2, v2, dry, st);
    if (v1.epi == EPI_STORE && !v1.out_f32) return first_tn<EPI_STORE, false>(d1, v1, d2, v2, dry, st);
    return hipErrorNotSupported;
  }
  if (v1.layout == GEMM_NN && v1.epi == EPI_STORE && !v1.out_f32) {
    if (v1.bn == 256) return second_nn<CfgL<256, 256, GEMM_NN, EPI_STORE, false, false>>(d1, d2, v2, dry, st);
    if (v1.bn == 128) return second_nn<CfgL<256, 128, GEMM_NN, EPI_STORE, false, false>>(d1, d2, v2, dry, st);
  }
  return hipErrorNotSupported;
}
