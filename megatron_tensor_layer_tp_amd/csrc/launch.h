// launch.h -- internal launchers of libtpshard (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_desc.h"

enum GemmLayout : int {
  GEMM_NN = 0,  // A [M][K], B [K][N]
  GEMM_NT = 1,  // A [M][K], B [N][K]
  GEMM_TN = 2,  // A [K][M], B [K][N]
};

// Residency of a bf16 DMA kernel on a CU: how many LDS stages each workgroup
// keeps and how many workgroups share the CU.  Three stages give every tile
// DMA two K steps to land (two stages wait on it after one); two workgroups per
// CU run one's MFMAs under the other's load waits and epilogue.  Either needs
// the stages to fit the CU's 160 KB of LDS.
// RES_WAVES8 keeps one workgroup per CU but of 8 waves (two per SIMD, each a
// 128x64 sub-tile), so one wave's MFMAs cover the other's LDS reads and waits.
enum Residency : int {
  RES_TWO = 0,     // 2 stages, one 4-wave workgroup per CU
  RES_THREE = 1,   // 3 stages, one 4-wave workgroup per CU
  RES_SHARED = 2,  // 2 stages, two 4-wave workgroups per CU
  RES_WAVES8 = 3,  // 2 stages, one 8-wave workgroup per CU
};
constexpr int res_stages(int res) { return res == RES_THREE ? 3 : 2; }
constexpr int res_wgs(int res) { return res == RES_SHARED ? 2 : 1; }
constexpr int res_waves(int res) { return res == RES_WAVES8 ? 8 : 4; }
// columns of one wave's sub-tile (the waves form a 2 x waves/2 grid)
constexpr bool res_fits(int bm, int bn, int res) {
  return res_stages(res) * res_wgs(res) * 128 * (bm + bn) <= 160 * 1024;
}

// One launchable bf16 kernel variant.  Built tiles (bm x bn, residency):
// 256x256 and 256x192 with RES_TWO; 256x256 with RES_WAVES8; 256x128, 128x256, 128x192 and 128x128 with RES_THREE; 128x192 and
// 128x128 with RES_SHARED.  192 columns not for the dual or CE-statistics
// epilogues.  vec = 16-byte loads are legal for every operand
// (aligned pointers, leading dimensions and extents multiple of 8); without it
// a 128x128 element-wise kernel runs whatever the tile fields say.
struct GemmVariant {
  int layout, epi;
  bool out_f32;
  int bm, bn, res;
  bool vec;
};
hipError_t tp_launch_gemm_bf16(const GemmDesc &d, const GemmVariant &v, hipStream_t st);
hipError_t tp_launch_splitk_reduce(const GemmDesc &d, bool out_f32, bool vec, hipStream_t st);

// Two independent bf16 products in one launch (the second must not be split),
// both with the same residency (RES_TWO, RES_SHARED or RES_WAVES8).  `red`
// (may be null): the split-K reduction of an earlier launch's product (bf16
// output, 16-byte runs, partials not written by this launch), run by extra
// workgroups of this one.  With dry = true nothing is launched: the return
// value only says whether the pair of variants is built (hipSuccess) or not
// (hipErrorNotSupported).
hipError_t tp_launch_gemm_pair(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                               const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st);
// the pairs whose first product is a TN split-K partial (called by tp_launch_gemm_pair)
hipError_t tp_launch_gemm_pair_tn_partial(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                                          const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st);
// the pairs whose first product is an NT activation gradient and whose second is
// a TN weight gradient (called by tp_launch_gemm_pair)
hipError_t tp_launch_gemm_pair_nt_first(const GemmDesc &d1, const GemmVariant &v1, const GemmDesc &d2,
                                        const GemmVariant &v2, const GemmDesc *red, bool dry, hipStream_t st);

// fp32 storage and arithmetic (64x64 tiles, any layout, any extents).
constexpr int TP_F32_TILE = 64;
hipError_t tp_launch_gemm_f32(const GemmDesc &d, int layout, int epi, hipStream_t st);

hipError_t tp_launch_vocab_ce(int64_t s, int64_t Vs, int64_t start, const float *z, const int64_t *tgt,
                              float *m, float *se, float *tl, hipStream_t st);
hipError_t tp_launch_vocab_ce_bwd(bool bf16_out, int64_t s, int64_t Vs, int64_t start, const float *z,
                                  const int64_t *tgt, const float *M, const float *S, const float *g, void *out,
                                  hipStream_t st);
// merge the fused LM-head GEMM's per-tile-column CE statistics: ws = max [P][s], sum exp [P][s],
// target logit [s]
hipError_t tp_launch_ce_merge(const float *ws, int P, int64_t s, int64_t Vs, int64_t start, const int64_t *tgt,
                              float *m, float *se, float *tl, hipStream_t st);
hipError_t tp_launch_vocab_embed(int elem_bytes, int64_t n, int64_t Vs, int64_t h, int64_t start,
                                 const int64_t *ids, const void *table, void *out, hipStream_t st);

// causal attention core, head dim 128, bf16 Q [s][nq*128], K/V [s][nkv*128], O like Q, lse [nq][s]
hipError_t tp_launch_attn_fwd(int64_t s, int64_t nq, int64_t nkv, const void *Q, const void *K, const void *V,
                              void *O, float *lse, hipStream_t st);

// backward of the attention core: D = rowsum(dO * O) and dQ, then per-query-head
// partial dK / dV, then their fixed-order sum over each KV head's query heads
size_t tp_attn_bwd_ws_bytes(int64_t s, int64_t nq);
hipError_t tp_launch_attn_bwd(int64_t s, int64_t nq, int64_t nkv, const void *Q, const void *K, const void *V,
                              const void *O, const void *dO, const float *lse, void *dQ, void *dK, void *dV,
                              void *ws, hipStream_t st);

// sequence-parallel region (residual + dropout + LayerNorm) on [n, h] bf16 rows
int tp_sp_ln_passes(int64_t h);        // register passes per row (h <= 8192: 1)
int tp_sp_ln_bwd_grid(int64_t n, int64_t h);  // partial sums of dgamma/dbeta the backward writes
hipError_t tp_launch_sp_ln_fwd(int64_t n, int64_t h, float keep, float eps, const void *y, const void *x,
                               const uint8_t *mask, const void *gamma, const void *beta, void *u, void *z,
                               float *mean, float *rstd, hipStream_t st);
hipError_t tp_launch_sp_ln_bwd(int64_t n, int64_t h, float keep, const void *dz, const void *dun, const void *u,
                               const float *mean, const float *rstd, const void *gamma, const uint8_t *mask,
                               void *dx, void *dy, void *dgamma, void *dbeta, float *part, hipStream_t st);
