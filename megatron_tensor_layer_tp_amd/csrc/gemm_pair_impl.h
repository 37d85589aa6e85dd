// gemm_pair_impl.h -- dispatch templates of the paired bf16 launches (two
// independent GEMMs of one pass in one launch); shared by the translation units
// that instantiate them (gemm_pair.hip, gemm_pair_partial.hip).
#pragma once
#include <algorithm>
#include <cstring>

#include "gemm_bf16_kernels.h"

namespace {

template <int BM, int BN, int LAYOUT, int EPI, bool OUT_F32, bool KSEG>
using CfgL = Cfg<BM, BN, LAYOUT != GEMM_TN, LAYOUT == GEMM_NT, EPI, OUT_F32, KSEG>;

// Launch the pair; `red` (may be null) is an earlier product's split-K
// reduction (bf16 output, 16-byte runs) run by extra workgroups at the end of
// the grid, about two runs of 8 columns per thread.
template <class C1, class C2, int RES>
hipError_t go(const GemmDesc &d1, const GemmDesc &d2, const GemmDesc *red, bool dry, hipStream_t st) {
  if (dry) return hipSuccess;
  const int n1 = d1.tiles_m * d1.tiles_n * d1.splits;
  const int n2 = d2.tiles_m * d2.tiles_n * d2.splits;
  GemmDesc d3;
  int n3 = 0;
  if (red != nullptr) {
    d3 = *red;
    const int64_t runs = (int64_t)d3.M * (d3.N / 8), per = 2 * 64 * res_waves(RES);
    n3 = (int)std::min<int64_t>((runs + per - 1) / per, 1024);
  } else {
    std::memset(&d3, 0, sizeof d3);
  }
  if (n1 + n2 + n3 == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dma_pair_kernel<C1, C2, RES>), dim3(n1 + n2 + n3), dim3(64 * res_waves(RES)), 0, st, d1,
                     d2, n1, n2, d3, n3);
  return hipGetLastError();
}

// Built pairs: RES_TWO with 256-row tiles of 256 or 192 columns, RES_WAVES8
// with 256x256 tiles, RES_SHARED with 128-row tiles of 192 or 128 columns, for
// both products.
constexpr int pair_bm(int res) { return res == RES_SHARED ? 128 : 256; }
constexpr int pair_wide(int res) { return res == RES_SHARED ? 192 : 256; }
constexpr int pair_narrow(int res) { return res == RES_SHARED ? 128 : res == RES_WAVES8 ? 256 : 192; }

template <int BN, int EPI, bool KSEG, int RES>
using NT2 = CfgL<pair_bm(RES), BN, GEMM_NT, EPI, false, KSEG>;

template <class C1, int RES, int EPI, bool KSEG>
hipError_t second_nt_bn(const GemmDesc &d1, const GemmDesc &d2, int bn, const GemmDesc *red, bool dry,
                        hipStream_t st) {
  if (bn == pair_wide(RES)) return go<C1, NT2<pair_wide(RES), EPI, KSEG, RES>, RES>(d1, d2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (bn == pair_narrow(RES)) return go<C1, NT2<pair_narrow(RES), EPI, KSEG, RES>, RES>(d1, d2, red, dry, st);
  return hipErrorNotSupported;
}

// first product fixed (C1): pick the second, an NT product with the same
// residency: a store (also over K-segments), activation backward or SwiGLU
// backward.
template <class C1, int RES>
hipError_t second_nt(const GemmDesc &d1, const GemmDesc &d2, const GemmVariant &v2, const GemmDesc *red, bool dry,
                     hipStream_t st) {
  if (v2.layout != GEMM_NT || v2.bm != pair_bm(RES) || v2.res != RES || v2.out_f32) return hipErrorNotSupported;
  switch (v2.epi) {
  case EPI_STORE:
    if (d2.kseg) return second_nt_bn<C1, RES, EPI_STORE, true>(d1, d2, v2.bn, red, dry, st);
    return second_nt_bn<C1, RES, EPI_STORE, false>(d1, d2, v2.bn, red, dry, st);
  case EPI_ACT_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    return second_nt_bn<C1, RES, EPI_ACT_BWD, false>(d1, d2, v2.bn, red, dry, st);
  case EPI_SWIGLU_BWD:
    if (d2.kseg) return hipErrorNotSupported;
    return second_nt_bn<C1, RES, EPI_SWIGLU_BWD, false>(d1, d2, v2.bn, red, dry, st);
  default: return hipErrorNotSupported;
  }
}

template <int EPI1, bool F32, int RES>
hipError_t first_tn_res(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2,
                        const GemmDesc *red, bool dry, hipStream_t st) {
  constexpr int BM = pair_bm(RES);
  if (v1.bm != BM) return hipErrorNotSupported;
  if (v1.bn == pair_wide(RES))
    return second_nt<CfgL<BM, pair_wide(RES), GEMM_TN, EPI1, F32, false>, RES>(d1, d2, v2, red, dry, st);
  if constexpr (pair_narrow(RES) != pair_wide(RES))
    if (v1.bn == pair_narrow(RES))
      return second_nt<CfgL<BM, pair_narrow(RES), GEMM_TN, EPI1, F32, false>, RES>(d1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}

// a TN first product (weight gradient)
template <int EPI1, bool F32>
hipError_t first_tn(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2, const GemmVariant &v2,
                    const GemmDesc *red, bool dry, hipStream_t st) {
  if (v1.res == RES_TWO) return first_tn_res<EPI1, F32, RES_TWO>(d1, v1, d2, v2, red, dry, st);
  if (v1.res == RES_WAVES8) return first_tn_res<EPI1, F32, RES_WAVES8>(d1, v1, d2, v2, red, dry, st);
  if (v1.res == RES_SHARED) return first_tn_res<EPI1, F32, RES_SHARED>(d1, v1, d2, v2, red, dry, st);
  return hipErrorNotSupported;
}

}  // namespace
