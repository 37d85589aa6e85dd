// launch.h -- internal launchers of libtpshard (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_desc.h"

enum GemmLayout : int {
  GEMM_NN = 0,  // A [M][K], B [K][N]
  GEMM_NT = 1,  // A [M][K], B [N][K]
  GEMM_TN = 2,  // A [K][M], B [K][N]
};

// bf16 MFMA tiles: bm in {128, 256}, bn in {128, 192, 256} (192 not for the
// dual or CE-statistics epilogues); vec = 16-byte loads are legal for
// every operand (aligned pointers, leading dimensions and extents multiple of 8).
hipError_t tp_launch_gemm_bf16(const GemmDesc &d, int layout, int epi, bool out_f32, int bm, int bn,
                               bool vec, hipStream_t st);
hipError_t tp_launch_splitk_reduce(const GemmDesc &d, bool out_f32, bool vec, hipStream_t st);

// Two independent bf16 products in one launch (the second must not be split).
// With dry = true nothing is launched: the return value only says whether the
// pair of variants is built (hipSuccess) or not (hipErrorNotSupported).
struct GemmVariant {
  int layout, epi;
  bool out_f32;
  int bm, bn;
  bool vec;
};
hipError_t tp_launch_gemm_pair(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                               const GemmVariant &v2, bool dry, hipStream_t st);
// the pairs whose first product is a TN split-K partial (called by tp_launch_gemm_pair)
hipError_t tp_launch_gemm_pair_tn_partial(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                                          const GemmVariant &v2, bool dry, hipStream_t st);

// fp32 storage and arithmetic (64x64 tiles, any layout, any extents).
constexpr int TP_F32_TILE = 64;
hipError_t tp_launch_gemm_f32(const GemmDesc &d, int layout, int epi, hipStream_t st);

hipError_t tp_launch_vocab_ce(int64_t s, int64_t Vs, int64_t start, const float *z, const int64_t *tgt,
                              float *m, float *se, float *tl, hipStream_t st);
hipError_t tp_launch_vocab_ce_bwd(bool bf16_out, int64_t s, int64_t Vs, int64_t start, const float *z,
                                  const int64_t *tgt, const float *M, const float *S, const float *g, void *out,
                                  hipStream_t st);
// merge the fused LM-head GEMM's per-part CE statistics ws [s][3][P] (parts of W columns)
hipError_t tp_launch_ce_merge(const float *ws, int P, int W, int64_t s, int64_t Vs, int64_t start,
                              const int64_t *tgt, float *m, float *se, float *tl, hipStream_t st);
hipError_t tp_launch_vocab_embed(int elem_bytes, int64_t n, int64_t Vs, int64_t h, int64_t start,
                                 const int64_t *ids, const void *table, void *out, hipStream_t st);

// causal attention core, head dim 128, bf16 Q [s][nq*128], K/V [s][nkv*128], O like Q, lse [nq][s]
hipError_t tp_launch_attn_fwd(int64_t s, int64_t nq, int64_t nkv, const void *Q, const void *K, const void *V,
                              void *O, float *lse, hipStream_t st);

// sequence-parallel region (residual + dropout + LayerNorm) on [n, h] bf16 rows
int tp_sp_ln_passes(int64_t h);        // register passes per row (h <= 8192: 1)
int tp_sp_ln_bwd_grid(int64_t n);      // row chunks of the backward = partial sums of dgamma/dbeta
hipError_t tp_launch_sp_ln_fwd(int64_t n, int64_t h, float keep, float eps, const void *y, const void *x,
                               const uint8_t *mask, const void *gamma, const void *beta, void *u, void *z,
                               float *mean, float *rstd, hipStream_t st);
hipError_t tp_launch_sp_ln_bwd(int64_t n, int64_t h, float keep, const void *dz, const void *dun, const void *u,
                               const float *mean, const float *rstd, const void *gamma, const uint8_t *mask,
                               void *dx, void *dy, void *dgamma, void *dbeta, float *part, hipStream_t st);
