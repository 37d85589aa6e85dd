// gemm_bf16.hip -- launchers of single bf16 products (one GEMM per launch,
// optionally followed by the split-K reduction); kernels in gemm_bf16_kernels.h.
#include "gemm_bf16_kernels.h"

namespace {

template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool KSEG, int RES>
hipError_t launch_dma(const GemmDesc &d, hipStream_t st) {
  const int nblk = d.nblocks > 0 ? d.nblocks : d.tiles_m * d.tiles_n * d.splits;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, A_KC, B_KC, EPI, OUT_F32, KSEG, RES>), dim3(nblk),
                     dim3(64 * res_waves(RES)), 0, st, d);
  return hipGetLastError();
}

// The built (tile, residency) variants: 256x256 and 256x192 with two stages;
// 256x256 with 8 waves; 256x128, 128x256, 128x192 and
// 128x128 with three; 128x192 and 128x128 also two workgroups per CU.
// 192-column tiles not for the dual or CE epilogues.
template <bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool KSEG>
hipError_t launch_shape_k(const GemmDesc &d, int bm, int bn, int res, hipStream_t st, bool vec) {
  if (!vec) {  // element-wise loads (odd sizes / leading dimensions): 128x128 tiles only
    const int nblk = d.nblocks > 0 ? d.nblocks : d.tiles_m * d.tiles_n * d.splits;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, A_KC, B_KC, EPI, OUT_F32, false, KSEG>), dim3(nblk),
                       dim3(NTHREADS), 0, st, d);
    return hipGetLastError();
  }
  constexpr bool W192 = EPI != EPI_SWIGLU_FWD && EPI != EPI_CE_STATS;
  switch (res) {
  case RES_TWO:
    if (bm == 256 && bn == 256) return launch_dma<256, 256, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_TWO>(d, st);
    if constexpr (W192)
      if (bm == 256 && bn == 192) return launch_dma<256, 192, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_TWO>(d, st);
    break;
  case RES_WAVES8:
    if (bm == 256 && bn == 256) return launch_dma<256, 256, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_WAVES8>(d, st);
    break;
  case RES_THREE:
    if (bm == 256 && bn == 128) return launch_dma<256, 128, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_THREE>(d, st);
    if (bm == 128 && bn == 256) return launch_dma<128, 256, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_THREE>(d, st);
    if constexpr (W192)
      if (bm == 128 && bn == 192) return launch_dma<128, 192, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_THREE>(d, st);
    if (bm == 128 && bn == 128) return launch_dma<128, 128, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_THREE>(d, st);
    break;
  case RES_SHARED:
    if constexpr (W192)
      if (bm == 128 && bn == 192) return launch_dma<128, 192, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_SHARED>(d, st);
    if (bm == 128 && bn == 128) return launch_dma<128, 128, A_KC, B_KC, EPI, OUT_F32, KSEG, RES_SHARED>(d, st);
    break;
  default: break;
  }
  return hipErrorNotSupported;
}

template <bool A_KC, bool B_KC, int EPI, bool OUT_F32>
hipError_t launch_shape(const GemmDesc &d, int bm, int bn, int res, hipStream_t st, bool vec) {
  // K-segments are used only by the summed dX products (NT, plain store or split-K partial)
  if constexpr (A_KC && B_KC && (EPI == EPI_STORE || EPI == EPI_PARTIAL)) {
    if (d.kseg) return launch_shape_k<A_KC, B_KC, EPI, OUT_F32, true>(d, bm, bn, res, st, vec);
  }
  if (d.kseg) return hipErrorInvalidValue;
  return launch_shape_k<A_KC, B_KC, EPI, OUT_F32, false>(d, bm, bn, res, st, vec);
}

}  // namespace

// Launch one planned bf16 product.  `layout`: GEMM_NN (A k-contig, B n-contig),
// GEMM_NT (both k-contig), GEMM_TN (A m-contig, B n-contig).
hipError_t tp_launch_gemm_bf16(const GemmDesc &d, const GemmVariant &v, hipStream_t st) {
  const int layout = v.layout, epi = v.epi, bm = v.bm, bn = v.bn, res = v.res;
  const bool out_f32 = v.out_f32, vec = v.vec;
  hipError_t e = hipSuccess;
  switch (layout) {
  case GEMM_NN:
    switch (epi) {
    case EPI_STORE:
      e = out_f32 ? launch_shape<true, false, EPI_STORE, true>(d, bm, bn, res, st, vec)
                  : launch_shape<true, false, EPI_STORE, false>(d, bm, bn, res, st, vec);
      break;
    case EPI_ACT_FWD: e = launch_shape<true, false, EPI_ACT_FWD, false>(d, bm, bn, res, st, vec); break;
    case EPI_SWIGLU_FWD: e = launch_shape<true, false, EPI_SWIGLU_FWD, false>(d, bm, bn, res, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<true, false, EPI_PARTIAL, true>(d, bm, bn, res, st, vec); break;
    case EPI_CE_STATS: e = launch_shape<true, false, EPI_CE_STATS, true>(d, bm, bn, res, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  case GEMM_NT:
    switch (epi) {
    case EPI_STORE: e = launch_shape<true, true, EPI_STORE, false>(d, bm, bn, res, st, vec); break;
    case EPI_ACT_BWD: e = launch_shape<true, true, EPI_ACT_BWD, false>(d, bm, bn, res, st, vec); break;
    case EPI_SWIGLU_BWD: e = launch_shape<true, true, EPI_SWIGLU_BWD, false>(d, bm, bn, res, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<true, true, EPI_PARTIAL, true>(d, bm, bn, res, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  case GEMM_TN:
    switch (epi) {
    case EPI_STORE: e = launch_shape<false, false, EPI_STORE, false>(d, bm, bn, res, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<false, false, EPI_PARTIAL, true>(d, bm, bn, res, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  default: return hipErrorInvalidValue;
  }
  return e;
}

hipError_t tp_launch_splitk_reduce(const GemmDesc &d, bool out_f32, bool vec, hipStream_t st) {
  const int64_t total = (int64_t)d.M * (vec ? d.N / 8 : d.N);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 g((unsigned)blocks), b(256);
  if (out_f32 && vec) hipLaunchKernelGGL((splitk_reduce_kernel<true, true>), g, b, 0, st, d);
  else if (out_f32) hipLaunchKernelGGL((splitk_reduce_kernel<true, false>), g, b, 0, st, d);
  else if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<false, true>), g, b, 0, st, d);
  else hipLaunchKernelGGL((splitk_reduce_kernel<false, false>), g, b, 0, st, d);
  return hipGetLastError();
}
