// gemm_desc.h -- problem descriptor shared by the host planner and the GEMM
// kernels of libtpshard, plus the element-wise epilogue math.
//
// Every matrix product of the shard is C[M,N] = sum_k A(m,k) B(k,n) with one
// of three operand layouts (row-major storage):
//   A "KC": A stored [M][K] (k contiguous)     -- X, dY, H, dZ, ...
//   A "MC": A stored [K][M] (m contiguous)     -- X^T, H^T, A^T, O^T (weight grads)
//   B "NC": B stored [K][N] (n contiguous)     -- the [in,out] weights in X.W
//   B "KC": B stored [N][K] (k contiguous)     -- W^T in dY.W^T
// Segments let one launch cover several products that share an operand:
//   N-segments (kseg = 0): one A, up to 3 (B, C) pairs side by side along N
//     (Q/K/V = X.[Wq|Wk|Wv], dW{q,k,v} = X^T.[dQ|dK|dV], dWg|dWu = X^T.[dG|dU]);
//   K-segments (kseg = 1): up to 3 (A, B) pairs summed into one C
//     (dX = dQ.Wq^T + dK.Wk^T + dV.Wv^T, dX = dG.Wg^T + dU.Wu^T).
// `dual` pairs two B matrices on the same columns (SwiGLU gate and up) so that
// one workgroup holds G and U for the same elements in its epilogue.
#pragma once
#include <stdint.h>

#define TP_MAX_SEG 3

enum EpiKind : int {
  EPI_STORE = 0,       // C = acc
  EPI_ACT_FWD = 1,     // C = act(acc); ao0 (may be null) = acc, the pre-activation
  EPI_ACT_BWD = 2,     // C = acc * act'(ai0)          (ai0 = Z, or H for the ReLU mask)
  EPI_SWIGLU_FWD = 3,  // dual: ao0 = g, ao1 = u, C = SiLU(g) * u
  EPI_SWIGLU_BWD = 4,  // C = acc * ai1 * SiLU'(ai0) (dG); ao0 = acc * SiLU(ai0) (dU)
  EPI_PARTIAL = 5,     // fp32 split-K partial into ws[split][M][N]
  EPI_CE_STATS = 6,    // logits stay on chip: per row and tile column (P = tiles_n parts),
                       // max into ws[P][M], sum exp(z - max) into ws[P + p][M], target logit ws[2P][M]
};

enum ActKind : int { ACT_RELU = 0, ACT_GELU = 1 };

struct GemmDesc {
  int32_t M, N, K;                 // N sums the N-segments, K sums the K-segments
  int32_t nseg;                    // 1..TP_MAX_SEG
  int32_t kseg;                    // 1: segments split K; 0: segments split N
  int32_t dual;                    // 1: B[0], B[1] share columns (N = their width)
  int32_t act;                     // ActKind for EPI_ACT_*
  int32_t seg_len[TP_MAX_SEG];     // extent of each segment along N or K
  int32_t seg_col0[TP_MAX_SEG];    // first global column (N-segments) of each segment
  int32_t seg_tile0[TP_MAX_SEG + 1];  // first N- or K-tile of each segment; [nseg] = total
  const void *A[TP_MAX_SEG];
  int64_t lda[TP_MAX_SEG];
  const void *B[TP_MAX_SEG];
  int64_t ldb[TP_MAX_SEG];
  void *C[TP_MAX_SEG];
  int64_t ldc[TP_MAX_SEG];
  const void *ai0, *ai1;           // epilogue inputs, indexed like C (one segment);
                                   // EPI_CE_STATS: ai0 = int64 target ids [M]
  int64_t ldai;
  void *ao0, *ao1;                 // epilogue extra outputs, indexed like C
  int64_t ldao;
  float *ws;                       // split-K partials [splits][M][N]
  int32_t splits;                  // >= 1
  int32_t kt_per_split;            // K-tiles handled by one split
  int32_t tiles_m, tiles_n;        // tile grid (tiles_n counts all N-segments)
  int32_t group_m;                 // tile-rows per L2 group
  int64_t vstart;                  // EPI_CE_STATS: global id of column 0
  int32_t stream_out;              // bf16 outputs stored non-temporally: bit 0 C, bit 1 ao0, bit 2 ao1
  int32_t nblocks;                 // > 0: launch only logical blocks [0, nblocks) (a prefix of the
                                   // tile order); 0: all tiles_m * tiles_n * splits
};

// ---------------------------------------------------------------------------
// element-wise math shared by the bf16 and fp32 kernels
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
#include <hip/hip_runtime.h>

// Element-wise activations, evaluated in fp32 with the hardware exp2 / rcp.
// erf comes from Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (Hastings): erf(x) = 1 - t (a1 + t (a2 + ... + t a5)) e^{-x^2},
// t = 1 / (1 + p |x|), |error| <= 1.5e-7 -- far below bf16's 2^-9 resolution.
// For GeLU the same e^{-z^2/2} serves Phi(z) = (1 + erf(z/sqrt 2)) / 2 and the
// normal density phi(z) = e^{-z^2/2} / sqrt(2 pi) of its derivative.
__device__ __forceinline__ float tp_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float tp_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Phi(z) given e = exp(-z*z/2)
__device__ __forceinline__ float tp_phi_cdf(float z, float e) {
  const float ax = fabsf(z) * 0.70710678118654752f;
  const float t = tp_rcp(fmaf(0.3275911f, ax, 1.f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  const float erf_ax = fmaf(-p * t, e, 1.f);
  return 0.5f + 0.5f * copysignf(erf_ax, z);
}
__device__ __forceinline__ float tp_gauss(float z) {  // exp(-z^2 / 2)
  return tp_exp2(-0.72134752044448170f * z * z);     // log2(e) / 2
}

__device__ __forceinline__ float tp_relu(float z) { return z > 0.f ? z : 0.f; }
__device__ __forceinline__ float tp_relu_grad(float z) { return z > 0.f ? 1.f : 0.f; }
__device__ __forceinline__ float tp_gelu(float z) {  // exact form z * Phi(z)
  return z * tp_phi_cdf(z, tp_gauss(z));
}
__device__ __forceinline__ float tp_gelu_grad(float z) {  // Phi(z) + z phi(z)
  const float e = tp_gauss(z);
  return fmaf(z * 0.39894228040143268f, e, tp_phi_cdf(z, e));
}
__device__ __forceinline__ float tp_act_fwd(int act, float z) {
  return act == ACT_RELU ? tp_relu(z) : tp_gelu(z);
}
__device__ __forceinline__ float tp_act_grad(int act, float z) {
  return act == ACT_RELU ? tp_relu_grad(z) : tp_gelu_grad(z);
}

__device__ __forceinline__ float tp_sigmoid(float z) {
  return tp_rcp(1.f + tp_exp2(-1.4426950408889634f * z));
}

// round-to-nearest-even fp32 -> bfloat16 bits
__device__ __forceinline__ uint16_t tp_f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float tp_bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
#endif
