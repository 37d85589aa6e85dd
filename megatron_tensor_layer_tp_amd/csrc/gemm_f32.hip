// gemm_f32.hip -- fp32 GEMM with the same descriptor and epilogues as the
// bf16 MFMA path.  It serves the fp32-storage variant of every call (the
// integer-valued configuration checks the shard algebra exactly: every
// intermediate is an integer below 2^24, so any summation order is exact).
// 64x64 tiles, 16-deep K slices through LDS, a 4x4 register block per thread;
// operands are read element by element, so any extents and layouts work.
#include "gemm_desc.h"
#include "launch.h"

namespace {

constexpr int T = TP_F32_TILE;  // 64
constexpr int KS = 16;

template <int EPI, bool DUAL>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmDesc d, int a_mc, int b_kc) {
  __shared__ float As[KS][T + 1];
  __shared__ float Bs[KS][T + 1];
  __shared__ float Bs2[DUAL ? KS : 1][T + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles = d.tiles_m * d.tiles_n;
  const int split = blockIdx.x / tiles;
  const int t = blockIdx.x - split * tiles;
  const int tm = t % d.tiles_m, tn = t / d.tiles_m;

  int sn = 0;
  if (!d.kseg)
    while (sn + 1 < d.nseg && tn >= d.seg_tile0[sn + 1]) ++sn;
  const int n0 = d.kseg ? tn * T : (tn - d.seg_tile0[sn]) * T;
  const int nlen = d.kseg ? d.N : d.seg_len[sn];
  const int m0 = tm * T;
  const int kt_total = d.kseg ? d.seg_tile0[d.nseg] : (d.K + T - 1) / T;
  const int kt_begin = split * d.kt_per_split;
  const int kt_end = min(kt_total, kt_begin + d.kt_per_split);

  float acc[4][4] = {}, acc2[4][4] = {};
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    int ks = 0;
    if (d.kseg)
      while (ks + 1 < d.nseg && kt >= d.seg_tile0[ks + 1]) ++ks;
    const int kbase = d.kseg ? (kt - d.seg_tile0[ks]) * T : kt * T;
    const int klen = d.kseg ? d.seg_len[ks] : d.K;
    const int ia = d.kseg ? ks : 0, ib = d.kseg ? ks : sn;
    const float *Ap = (const float *)d.A[ia];
    const float *Bp = (const float *)d.B[ib];
    const float *Bp2 = DUAL ? (const float *)d.B[1] : Bp;
    const int64_t lda = d.lda[ia], ldb = d.ldb[ib];
    for (int kq = 0; kq < T; kq += KS) {
      for (int q = tid; q < KS * T; q += 256) {
        const int r = q % T, kk = q / T;
        const int k = kbase + kq + kk;
        const int m = m0 + r, n = n0 + r;
        float a = 0.f, b = 0.f, b2 = 0.f;
        if (k < klen && m < d.M) a = a_mc ? Ap[(int64_t)k * lda + m] : Ap[(int64_t)m * lda + k];
        if (k < klen && n < nlen) {
          b = b_kc ? Bp[(int64_t)n * ldb + k] : Bp[(int64_t)k * ldb + n];
          if (DUAL) b2 = Bp2[(int64_t)k * ldb + n];
        }
        As[kk][r] = a;
        Bs[kk][r] = b;
        if (DUAL) Bs2[kk][r] = b2;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        float av[4], bv[4], bv2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = As[kk][ty + 16 * i];
          bv[i] = Bs[kk][tx + 16 * i];
          if (DUAL) bv2[i] = Bs2[kk][tx + 16 * i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            if (DUAL) acc2[i][j] = fmaf(av[i], bv2[j], acc2[i][j]);
          }
      }
      __syncthreads();
    }
  }

  const int sc = d.kseg ? 0 : sn;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * j;
      if (gm >= d.M || gn >= nlen) continue;
      const float x = acc[i][j];
      if constexpr (EPI == EPI_PARTIAL) {
        const int col = d.kseg ? gn : d.seg_col0[sn] + gn;
        d.ws[((int64_t)split * d.M + gm) * d.N + col] = x;
      } else if constexpr (EPI == EPI_STORE) {
        ((float *)d.C[sc])[(int64_t)gm * d.ldc[sc] + gn] = x;
      } else if constexpr (EPI == EPI_ACT_FWD) {
        if (d.ao0) ((float *)d.ao0)[(int64_t)gm * d.ldao + gn] = x;
        ((float *)d.C[0])[(int64_t)gm * d.ldc[0] + gn] = tp_act_fwd(d.act, x);
      } else if constexpr (EPI == EPI_ACT_BWD) {
        const float z = ((const float *)d.ai0)[(int64_t)gm * d.ldai + gn];
        ((float *)d.C[0])[(int64_t)gm * d.ldc[0] + gn] = x * tp_act_grad(d.act, z);
      } else if constexpr (EPI == EPI_SWIGLU_FWD) {
        const float u = acc2[i][j];
        ((float *)d.ao0)[(int64_t)gm * d.ldao + gn] = x;
        ((float *)d.ao1)[(int64_t)gm * d.ldao + gn] = u;
        ((float *)d.C[0])[(int64_t)gm * d.ldc[0] + gn] = x * tp_sigmoid(x) * u;
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const int64_t o = (int64_t)gm * d.ldai + gn;
        const float g = ((const float *)d.ai0)[o], u = ((const float *)d.ai1)[o];
        const float sg = tp_sigmoid(g);
        ((float *)d.C[0])[(int64_t)gm * d.ldc[0] + gn] = x * u * (sg * (1.f + g * (1.f - sg)));
        ((float *)d.ao0)[(int64_t)gm * d.ldao + gn] = x * g * sg;
      }
    }
}

template <int EPI, bool DUAL>
hipError_t go(const GemmDesc &d, int a_mc, int b_kc, hipStream_t st) {
  const int nblk = d.tiles_m * d.tiles_n * d.splits;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI, DUAL>), dim3(nblk), dim3(256), 0, st, d, a_mc, b_kc);
  return hipGetLastError();
}

}  // namespace

hipError_t tp_launch_gemm_f32(const GemmDesc &d, int layout, int epi, hipStream_t st) {
  const int a_mc = layout == GEMM_TN;
  const int b_kc = layout == GEMM_NT;
  switch (epi) {
  case EPI_STORE: return go<EPI_STORE, false>(d, a_mc, b_kc, st);
  case EPI_ACT_FWD: return go<EPI_ACT_FWD, false>(d, a_mc, b_kc, st);
  case EPI_ACT_BWD: return go<EPI_ACT_BWD, false>(d, a_mc, b_kc, st);
  case EPI_SWIGLU_FWD: return go<EPI_SWIGLU_FWD, true>(d, a_mc, b_kc, st);
  case EPI_SWIGLU_BWD: return go<EPI_SWIGLU_BWD, false>(d, a_mc, b_kc, st);
  case EPI_PARTIAL: return go<EPI_PARTIAL, false>(d, a_mc, b_kc, st);
  }
  return hipErrorInvalidValue;
}
