// gemm_pair.hip -- launchers of paired bf16 products: two independent GEMMs of
// one pass (a weight gradient beside an activation gradient, or the QKV and
// output projections) in one launch, so that neither leaves CUs idle while the
// other drains.  Kernels in gemm_bf16_kernels.h.
//
// Supported pairs (first = the long-K product, second = the short-K one), both
// with 256-row tiles of 256 or 128 columns and 16-byte-aligned operands:
//   first  TN store (bf16) or TN split-K partial (fp32)  second  NT store, NT
//          store over K-segments, NT activation backward, NT SwiGLU backward;
//   first  NN store                                      second  NN store.
#include "gemm_bf16_kernels.h"

namespace {

template <int BM, int BN, int LAYOUT, int EPI, bool OUT_F32, bool KSEG>
using CfgL = Cfg<BM, BN, LAYOUT != GEMM_TN, LAYOUT == GEMM_NT, EPI, OUT_F32, KSEG>;

template <class C1, class C2>
hipError_t go(const GemmDesc &d1, const GemmDesc &d2, bool dry, hipStream_t st) {
  if (dry) return hipSuccess;
  const int n1 = d1.tiles_m * d1.tiles_n * d1.splits;
  const int n2 = d2.tiles_m * d2.tiles_n * d2.splits;
  if (n1 + n2 == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dma_pair_kernel<C1, C2>), dim3(n1 + n2), dim3(NTHREADS), 0, st, d1, d2, n1, n2);
  return hipGetLastError();
}

template <int BM, int BN, int EPI, bool KSEG>
using NT2 = CfgL<BM, BN, GEMM_NT, EPI, false, KSEG>;

// first product fixed (C1): pick the second
template <class C1>
hipError_t second_nt(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, bool dry, hipStream_t st) {
  const bool w = v2.bn == 256;
  if (v2.layout != GEMM_NT || v2.bm != 256 || (v2.bn != 256 && v2.bn != 128) || v2.out_f32)
    return hipErrorNotSupported;
  switch (v2.epi) {
  case EPI_STORE:
    if (d2.kseg)
      return w ? go<C1, NT2<256, 256, EPI_STORE, true>>(d1, d2, dry, st)
               : go<C1, NT2<256, 128, EPI_STORE, true>>(d1, d2, dry, st);
    return w ? go<C1, NT2<256, 256, EPI_STORE, false>>(d1, d2, dry, st)
             : go<C1, NT2<256, 128, EPI_STORE, false>>(d1, d2, dry, st);
  case EPI_ACT_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    return w ? go<C1, NT2<256, 256, EPI_ACT_BWD, false>>(d1, d2, dry, st)
             : go<C1, NT2<256, 128, EPI_ACT_BWD, false>>(d1, d2, dry, st);
  case EPI_SWIGLU_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    return w ? go<C1, NT2<256, 256, EPI_SWIGLU_BWD, false>>(d1, d2, dry, st)
             : go<C1, NT2<256, 128, EPI_SWIGLU_BWD, false>>(d1, d2, dry, st);
  default: return hipErrorNotSupported;
  }
}

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
  if (!v1.vec || !v2.vec || d1.kseg || v1.bm != 256 || (v1.bn != 256 && v1.bn != 128))
    return hipErrorNotSupported;
  const bool w = v1.bn == 256;
  if (v1.layout == GEMM_TN) {
    if (v1.epi == EPI_PARTIAL && v1.out_f32)
      return w ? second_nt<CfgL<256, 256, GEMM_TN, EPI_PARTIAL, true, false>>(d1, d2, v2, dry, st)
               : second_nt<CfgL<256, 128, GEMM_TN, EPI_PARTIAL, true, false>>(d1, d2, v2, dry, st);
    if (v1.epi == EPI_STORE && !v1.out_f32)
      return w ? second_nt<CfgL<256, 256, GEMM_TN, EPI_STORE, false, false>>(d1, d2, v2, dry, st)
               : second_nt<CfgL<256, 128, GEMM_TN, EPI_STORE, false, false>>(d1, d2, v2, dry, st);
    return hipErrorNotSupported;
  }
  if (v1.layout == GEMM_NN && v1.epi == EPI_STORE && !v1.out_f32)
    return w ? second_nn<CfgL<256, 256, GEMM_NN, EPI_STORE, false, false>>(d1, d2, v2, dry, st)
             : second_nn<CfgL<256, 128, GEMM_NN, EPI_STORE, false, false>>(d1, d2, v2, dry, st);
  return hipErrorNotSupported;
}
