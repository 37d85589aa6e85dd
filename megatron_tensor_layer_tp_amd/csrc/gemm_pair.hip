// gemm_pair.hip -- launchers of paired bf16 products: two independent GEMMs of
// one pass (a weight gradient beside an activation gradient, or the QKV and
// output projections) in one launch, so that neither leaves CUs idle while the
// other drains.  Kernels in gemm_bf16_kernels.h, dispatch in gemm_pair_impl.h.
//
// Supported pairs (first = the product with the longer tiles, second = the other), both
// with 16-byte-aligned operands and one residency: RES_TWO with 256-row tiles
// of 256 or 192 columns, RES_WAVES8 with 256x256 tiles, RES_SHARED (two
// workgroups per CU) with 128-row tiles of 192 or 128 columns:
//   first  TN store (bf16) or TN split-K partial (fp32; gemm_pair_partial.hip);
//   second NT store (also over K-segments), NT activation backward or NT SwiGLU
//          backward;
//   first  NN store, second NN store;
//   first  NT store or NT activation backward, second TN store (RES_WAVES8 and
//          RES_SHARED; gemm_pair_nt.hip).
#include "gemm_pair_impl.h"

namespace {

template <class C1, int RES>
hipError_t second_nn(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, const GemmDesc *red, bool dry,
                     hipStream_t st) {
  constexpr int BM = pair_bm(RES);
  if (v2.layout != GEMM_NN || v2.epi != EPI_STORE || v2.out_f32 || d2.kseg || v2.bm != BM || v2.res != RES)
    return hipErrorNotSupported;
  if (v2.bn == pair_wide(RES))
    return go<C1, CfgL<BM, pair_wide(RES), GEMM_NN, EPI_STORE, false, false>, RES>(d1, d2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (v2.bn == pair_narrow(RES))
      return go<C1, CfgL<BM, pair_narrow(RES), GEMM_NN, EPI_STORE, false, false>, RES>(d1, d2, red, dry, st);
  return hipErrorNotSupported;
}

template <int RES>
hipError_t first_nn(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2,
                    const GemmDesc *red, bool dry, hipStream_t st) {
  constexpr int BM = pair_bm(RES);
  if (v1.bm != BM) return hipErrorNotSupported;
  if (v1.bn == pair_wide(RES))
    return second_nn<CfgL<BM, pair_wide(RES), GEMM_NN, EPI_STORE, false, false>, RES>(d1, d2, v2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (v1.bn == pair_narrow(RES))
      return second_nn<CfgL<BM, pair_narrow(RES), GEMM_NN, EPI_STORE, false, false>, RES>(d1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t tp_launch_gemm_pair(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                               const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st) {
  if (!v1.vec || !v2.vec || d1.kseg || v1.res != v2.res) return hipErrorNotSupported;
  if (v1.layout == GEMM_TN) {
    if (v1.epi == EPI_PARTIAL && v1.out_f32) return tp_launch_gemm_pair_tn_partial(d1, v1, d2, v2, red, dry, st);
    if (v1.epi == EPI_STORE && !v1.out_f32) return first_tn<EPI_STORE, false>(d1, v1, d2, v2, red, dry, st);
    return hipErrorNotSupported;
  }
  if (v1.layout == GEMM_NT) return tp_launch_gemm_pair_nt_first(d1, v1, d2, v2, red, dry, st);
  if (v1.layout == GEMM_NN && v1.epi == EPI_STORE && !v1.out_f32) {
    if (v1.res == RES_TWO) return first_nn<RES_TWO>(d1, v1, d2, v2, red, dry, st);
    if (v1.res == RES_WAVES8) return first_nn<RES_WAVES8>(d1, v1, d2, v2, red, dry, st);
    if (v1.res == RES_SHARED) return first_nn<RES_SHARED>(d1, v1, d2, v2, red, dry, st);
  }
  return hipErrorNotSupported;
}
