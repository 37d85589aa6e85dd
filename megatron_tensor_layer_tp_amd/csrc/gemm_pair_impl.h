// gemm_pair_impl.h -- dispatch templates of the paired bf16 launches (two
// independent GEMMs of one pass in one launch); shared by the translation units
// that instantiate them (gemm_pair.hip, gemm_pair_partial.hip).
#pragma once
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

template <int BN, int EPI, bool KSEG>
using NT2 = CfgL<256, BN, GEMM_NT, EPI, false, KSEG>;

// first product fixed (C1): pick the second, an NT product with 256-row tiles.
// Plain stores and the activation backward also take 192-column tiles.
template <class C1>
hipError_t second_nt(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, bool dry, hipStream_t st) {
  if (v2.layout != GEMM_NT || v2.bm != 256 || v2.out_f32) return hipErrorNotSupported;
  const int bn = v2.bn;
  switch (v2.epi) {
  case EPI_STORE:
    if (d2.kseg) {
      if (bn == 256) return go<C1, NT2<256, EPI_STORE, true>>(d1, d2, dry, st);
      if (bn == 128) return go<C1, NT2<128, EPI_STORE, true>>(d1, d2, dry, st);
      return hipErrorNotSupported;
    }
    if (bn == 256) return go<C1, NT2<256, EPI_STORE, false>>(d1, d2, dry, st);
    if (bn == 192) return go<C1, NT2<192, EPI_STORE, false>>(d1, d2, dry, st);
    if (bn == 128) return go<C1, NT2<128, EPI_STORE, false>>(d1, d2, dry, st);
    return hipErrorNotSupported;
  case EPI_ACT_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    if (bn == 256) return go<C1, NT2<256, EPI_ACT_BWD, false>>(d1, d2, dry, st);
    if (bn == 192) return go<C1, NT2<192, EPI_ACT_BWD, false>>(d1, d2, dry, st);
    if (bn == 128) return go<C1, NT2<128, EPI_ACT_BWD, false>>(d1, d2, dry, st);
    return hipErrorNotSupported;
  case EPI_SWIGLU_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    if (bn == 256) return go<C1, NT2<256, EPI_SWIGLU_BWD, false>>(d1, d2, dry, st);
    if (bn == 128) return go<C1, NT2<128, EPI_SWIGLU_BWD, false>>(d1, d2, dry, st);
    return hipErrorNotSupported;
  default: return hipErrorNotSupported;
  }
}

// a TN first product (weight gradient) with 256-row tiles of 256, 192 or 128 columns
template <int EPI1, bool F32>
hipError_t first_tn(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2, bool dry,
                    hipStream_t st) {
  if (v1.bn == 256) return second_nt<CfgL<256, 256, GEMM_TN, EPI1, F32, false>>(d1, d2, v2, dry, st);
  if (v1.bn == 192) return second_nt<CfgL<256, 192, GEMM_TN, EPI1, F32, false>>(d1, d2, v2, dry, st);
  if (v1.bn == 128) return second_nt<CfgL<256, 128, GEMM_TN, EPI1, F32, false>>(d1, d2, v2, dry, st);
  return hipErrorNotSupported;
}

}  // namespace
