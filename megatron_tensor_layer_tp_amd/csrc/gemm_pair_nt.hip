// gemm_pair_nt.hip -- paired launches whose first product is an activation
// gradient (NT: a plain store or the activation-backward epilogue) and whose
// second is a weight gradient (TN store).  This order serves shards with few
// tokens: the weight gradients' K is the token count, so their tiles are the
// short ones, and the long activation-gradient tiles are dispatched first with
// the weight-gradient tiles filling the CUs around them and after them.
// A translation unit of its own so the pair kernels compile in parallel;
// dispatch templates in gemm_pair_impl.h.
#include "gemm_pair_impl.h"

namespace {

template <class C1, int RES>
hipError_t second_tn(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, const GemmDesc *red, bool dry,
                     hipStream_t st) {
  constexpr int BM = pair_bm(RES);
  if (v2.layout != GEMM_TN || v2.epi != EPI_STORE || v2.out_f32 || d2.kseg || v2.bm != BM || v2.res != RES)
    return hipErrorNotSupported;
  if (v2.bn == pair_wide(RES))
    return go<C1, CfgL<BM, pair_wide(RES), GEMM_TN, EPI_STORE, false, false>, RES>(d1, d2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (v2.bn == pair_narrow(RES))
      return go<C1, CfgL<BM, pair_narrow(RES), GEMM_TN, EPI_STORE, false, false>, RES>(d1, d2, red, dry, st);
  return hipErrorNotSupported;
}

template <int EPI1, int RES>
hipError_t first_nt_res(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2,
                        const GemmDesc *red, bool dry, hipStream_t st) {
  constexpr int BM = pair_bm(RES);
  if (v1.bm != BM) return hipErrorNotSupported;
  if (v1.bn == pair_wide(RES))
    return second_tn<CfgL<BM, pair_wide(RES), GEMM_NT, EPI1, false, false>, RES>(d1, d2, v2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (v1.bn == pair_narrow(RES))
      return second_tn<CfgL<BM, pair_narrow(RES), GEMM_NT, EPI1, false, false>, RES>(d1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}

template <int EPI1>
hipError_t first_nt(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2,
                    const GemmDesc *red, bool dry, hipStream_t st) {
  if (v1.res == RES_WAVES8) return first_nt_res<EPI1, RES_WAVES8>(d1, v1, d2, v2, red, dry, st);
  if (v1.res == RES_SHARED) return first_nt_res<EPI1, RES_SHARED>(d1, v1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t tp_launch_gemm_pair_nt_first(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                                        const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st) {
  if (v1.layout != GEMM_NT || v1.out_f32 || d1.kseg) return hipErrorNotSupported;
  if (v1.epi == EPI_STORE) return first_nt<EPI_STORE>(d1, v1, d2, v2, red, dry, st);
  if (v1.epi == EPI_ACT_BWD) return first_nt<EPI_ACT_BWD>(d1, v1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}
