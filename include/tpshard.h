/*
 * tpshard.h -- C ABI of libtpshard: one GPU's shard of a Megatron-style
 * tensor-parallel transformer layer, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow two public pages:
 *   [book]  "7.3 模型并行与张量并行：把一层切到多张卡上" (LLM internals book):
 *           §7.3.2 column and row splits with the two-card worked example,
 *           §7.3.3 the backward pass and the f / g operators,
 *           §7.3.4 attention by heads, SwiGLU, embedding and LM head by vocab;
 *   [lec16] CMU 11-868 lecture 16 notes, §5 "张量并行": §5.2 the MLP (column
 *           then row), §5.3 attention by heads, §5.5 vocab-parallel embedding
 *           and fused cross entropy.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are dense, row-major and contiguous.  Weights are stored
 *    [in, out] as the pages write them (Y = X.W), not [out, in].
 *  - Shard i of t holds columns [i*f/t, (i+1)*f/t) of a column-split weight and
 *    the same rows of the row-split weight that follows it ([book] §7.3.2: card
 *    0 holds the first columns of W1 and the first rows of W2).  The calls work
 *    on one shard; the caller passes that shard's slices and sizes.
 *  - Pointers X, W*, Z, ... are DEVICE pointers owned by the caller.  The
 *    library allocates no memory, frees nothing and keeps no state between
 *    calls (the one exception, the device array of tp_lm_head_ce_fwd_noalloc,
 *    is described there).  Every pointer must be 16-byte aligned (TP_EALIGN
 *    otherwise).
 *    Outputs are overwritten (never accumulated into) and must not alias any
 *    input or each other.  Inputs are never modified.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; results are valid once the caller synchronizes
 *    the stream.  Calls on different streams may run concurrently when their
 *    outputs and workspaces are distinct.  No call synchronizes, allocates or
 *    clears memory with hipMemsetAsync, so a sequence of calls can be captured
 *    into a HIP graph and replayed with the same pointers and sizes.
 *  - Every argument is checked before anything is enqueued: on an error no
 *    kernel runs, the call returns the status and tp_last_error() (per host
 *    thread) says which check failed.  A failed launch returns TP_EHIP.
 *    Faults inside a kernel surface at the caller's synchronization.
 *  - Sizes are int64_t.  Negative sizes are TP_ESHAPE.  A zero size is legal:
 *    outputs with no elements are not touched, and outputs of an empty
 *    contraction (zero inner size) are written as the activation of zero.
 *    Each size must be below 2^31.
 *  - dtype TP_DT_BF16: bfloat16 storage of every tensor (inputs, outputs,
 *    saved activations, gradients), fp32 accumulation, round-to-nearest-even
 *    on every store.  TP_DT_F32: fp32 storage and arithmetic throughout.
 *  - Thread safety: the library holds no shared mutable state except the
 *    per-thread last-error string and the per-device array of
 *    tp_lm_head_ce_fwd_noalloc.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 1

typedef enum {
    TP_OK = 0,
    TP_EINVAL = 1,        /* NULL pointer or bad enum value */
    TP_ESHAPE = 2,        /* negative size, size >= 2^31, or inconsistent sizes */
    TP_EDTYPE = 3,        /* dtype not valid for this call */
    TP_EALIGN = 4,        /* a pointer is not 16-byte aligned */
    TP_EWORKSPACE = 5,    /* workspace missing or smaller than the size query */
    TP_EHIP = 6,          /* the HIP runtime reported an error at launch */
    TP_EUNSUPPORTED = 7   /* valid request the library does not implement */
} tp_status;

typedef enum { TP_DT_F32 = 0, TP_DT_BF16 = 1 } tp_dtype;

/* Element-wise activation of the MLP shard.  GELU is the exact form
 * z * Phi(z) with Phi the standard normal CDF (the pages name GeLU without a
 * formula).  ReLU's derivative is taken as 0 at z = 0. */
typedef enum { TP_ACT_RELU = 0, TP_ACT_GELU = 1 } tp_act;

/* ------------------------------------------------------------------------ */
/* MLP shard: column-parallel GEMM + activation, row-parallel GEMM          */
/* ------------------------------------------------------------------------ */

/* Forward of the MLP shard ([lec16] §5.2; [book] §7.3.2):
 *     Z = X . W1(i)        X [s,h], W1(i) [h,ft]        -> Z [s,ft]
 *     H = act(Z)                                         -> H [s,ft]
 *     Y(i) = H . W2(i)     W2(i) [ft,h]                  -> Y [s,h]
 * Y(i) is this shard's partial sum: the g operator's all-reduce over the t
 * shards gives the layer output.  Z may be NULL when act is TP_ACT_RELU (the
 * backward then takes the mask from H > 0); it is required for GELU.
 * dt: TP_DT_F32 or TP_DT_BF16 for every tensor. */
int tp_mlp_fwd(int act, int dt, int64_t s, int64_t h, int64_t ft,
               const void *X, const void *W1, const void *W2,
               void *Z, void *H, void *Y, void *stream);

/* Bytes of device workspace tp_mlp_bwd needs for these sizes (0 on bad input). */
size_t tp_mlp_bwd_workspace(int dt, int64_t s, int64_t h, int64_t ft);

/* Backward of the MLP shard ([book] §7.3.3):
 *     dH = dY . W2(i)^T;  dZ = dH * act'(Z)   (ReLU: dZ = dH where Z > 0, else 0)
 *     dX(i) = dZ . W1(i)^T                     -> dX [s,h]: the partial sum the
 *                                                 f operator's all-reduce adds
 *     dW1(i) = X^T . dZ                        -> dW1 [h,ft]
 *     dW2(i) = H^T . dY                        -> dW2 [ft,h]
 * Z and H are the forward's outputs for the same X, W1 (Z may be NULL for
 * ReLU, then the mask is H > 0).  dY [s,h] is the full output gradient
 * (g's backward is the identity).  ws / ws_bytes: device workspace of at least
 * tp_mlp_bwd_workspace() bytes, 256-byte aligned (NULL when that is 0: the
 * planned launches split no product along K); its contents on entry do not
 * matter and are garbage on return. */
int tp_mlp_bwd(int act, int dt, int64_t s, int64_t h, int64_t ft,
               const void *X, const void *W1, const void *W2,
               const void *Z, const void *H, const void *dY,
               void *dX, void *dW1, void *dW2,
               void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* SwiGLU shard ([book] §7.3.4: gate and up split by columns, product on the */
/* shard, down split by rows).  Reading: A = SiLU(X.Wg) * (X.Wu), swish beta 1.*/
/* ------------------------------------------------------------------------ */

/* Forward:  G = X.Wg(i), U = X.Wu(i)  (Wg, Wu [h,ft])   -> G, U [s,ft]
 *           A = SiLU(G) * U                              -> A [s,ft]
 *           Y(i) = A . Wd(i)           (Wd [ft,h])       -> Y [s,h] partial sum
 * G, U and A are saved for the backward.  dt: TP_DT_BF16 or TP_DT_F32. */
int tp_swiglu_fwd(int dt, int64_t s, int64_t h, int64_t ft,
                  const void *X, const void *Wg, const void *Wu, const void *Wd,
                  void *G, void *U, void *A, void *Y, void *stream);

size_t tp_swiglu_bwd_workspace(int dt, int64_t s, int64_t h, int64_t ft);

/* Backward:  dA = dY . Wd^T;  dG = dA * U * SiLU'(G);  dU = dA * SiLU(G)
 *            dWd = A^T . dY                              -> [ft,h]
 *            dX(i) = dG . Wg^T + dU . Wu^T               -> [s,h] partial sum
 *            dWg = X^T . dG,  dWu = X^T . dU             -> [h,ft] each
 * G, U, A are the forward's outputs.  Workspace as for tp_mlp_bwd. */
int tp_swiglu_bwd(int dt, int64_t s, int64_t h, int64_t ft,
                  const void *X, const void *Wg, const void *Wu, const void *Wd,
                  const void *G, const void *U, const void *A, const void *dY,
                  void *dX, void *dWg, void *dWu, void *dWd,
                  void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Attention projections split by heads ([book] §7.3.4; [lec16] §5.3):       */
/* Q/K/V column-split (whole heads per shard), W_O row-split.  The attention  */
/* core between them is not part of these calls.                             */
/* ------------------------------------------------------------------------ */

/* Forward:  Q = X.Wq(i) [s,dq];  K = X.Wk(i) [s,dkv];  V = X.Wv(i) [s,dkv]
 *           Y(i) = O . Wo(i)      O [s,dq] (the core's output), Wo [dq,h]
 * Wq [h,dq], Wk and Wv [h,dkv].  Y is this shard's partial sum. */
int tp_attn_proj_fwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv,
                     const void *X, const void *Wq, const void *Wk, const void *Wv,
                     const void *O, const void *Wo,
                     void *Q, void *K, void *V, void *Y, void *stream);

size_t tp_attn_proj_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv);

/* Backward:  dX(i) = dQ.Wq^T + dK.Wk^T + dV.Wv^T   -> [s,h] partial sum (f's input)
 *            dWq = X^T.dQ, dWk = X^T.dK, dWv = X^T.dV
 *            dO = dY . Wo^T  [s,dq];  dWo = O^T . dY  [dq,h]
 * dQ, dK, dV are the gradients the attention core hands back; dY [s,h]. */
int tp_attn_proj_bwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv,
                     const void *X, const void *Wq, const void *Wk, const void *Wv,
                     const void *O, const void *Wo,
                     const void *dQ, const void *dK, const void *dV, const void *dY,
                     void *dX, void *dWq, void *dWk, void *dWv, void *dO, void *dWo,
                     void *ws, size_t ws_bytes, void *stream);

/* Attention core on the shard's heads ([book] §7.3.4: each card runs attention
 * on its own query heads -- 8 of Llama-3-70B's 64 at t = 8 -- which share its
 * key/value heads, 1 of 8; the outputs concatenate to [s, nq*d], the input of
 * the row-split W_O product).  Causal scaled dot-product attention:
 *     S = Q_j K_g^T / sqrt(d) over keys c <= r,  O_j[r] = softmax(S) V_g,
 *     lse[j][r] = ln sum_c exp(S[r][c]),
 * query head j reading KV head g = j / (nq / nkv).  Q [s][nq*d], K and V
 * [s][nkv*d], O [s][nq*d] (head j in columns [j*d, (j+1)*d)), lse [nq][s]
 * fp32.  dt must be TP_DT_BF16 and d = 128 (TP_EUNSUPPORTED otherwise); nq
 * must be a multiple of nkv (TP_ESHAPE).  Flash-style: the s x s scores are
 * never stored; P is rounded to bf16 before the product with V. */
int tp_attn_core_fwd(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d,
                     const void *Q, const void *K, const void *V, void *O, float *lse,
                     void *stream);

/* The two halves of tp_attn_proj_bwd as calls of their own, for a layer
 * backward that runs the attention core's backward between them (the core
 * needs dO, and produces the dQ, dK, dV the Q/K/V half consumes):
 *   tp_attn_out_bwd:  dO = dY . Wo^T [s,dq];  dWo = O^T . dY [dq,h]
 *   tp_attn_qkv_bwd:  dX(i) = dQ.Wq^T + dK.Wk^T + dV.Wv^T [s,h] (f's input);
 *                     dWq = X^T.dQ, dWk = X^T.dK, dWv = X^T.dV
 * Same results as the matching outputs of tp_attn_proj_bwd (same kernels and
 * plans).  ws: device scratch of the size query's bytes (0 possible: then ws
 * may be NULL), 256-byte aligned, contents garbage on return. */
size_t tp_attn_out_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq);
int tp_attn_out_bwd(int dt, int64_t s, int64_t h, int64_t dq, const void *O, const void *Wo, const void *dY,
                    void *dO, void *dWo, void *ws, size_t ws_bytes, void *stream);
size_t tp_attn_qkv_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv);
int tp_attn_qkv_bwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv,
                    const void *X, const void *Wq, const void *Wk, const void *Wv,
                    const void *dQ, const void *dK, const void *dV,
                    void *dX, void *dWq, void *dWk, void *dWv, void *ws, size_t ws_bytes, void *stream);

/* Backward of tp_attn_core_fwd (the same causal attention of the shard's nq
 * query heads on its nkv key/value heads).  With P the attention weights of
 * query head j (KV head g = j / (nq / nkv)), recomputed from Q, K and the
 * forward's lse instead of stored (the CS336 lecture-8 book, activation-memory
 * section: FlashAttention recomputes the s x s scores in the backward pass):
 *     dP = dO_j V_g^T,  D = rowsum(dO_j * O_j),  dS = P * (dP - D)
 *     dQ_j = dS K_g / sqrt(d)
 *     dK_g = sum over the query heads j of group g of dS^T Q_j / sqrt(d)
 *     dV_g = sum over the query heads j of group g of P^T dO_j
 * a shared KV head's gradient summed over its query heads in increasing head
 * order ([book] §7.3.4: a card's 8 query heads share its 1 KV head).
 * Q, O, dO, dQ [s][nq*d]; K, V, dK, dV [s][nkv*d]; lse [nq][s] fp32 from the
 * forward for the same Q, K, V; O the forward's output.  dt must be
 * TP_DT_BF16 and d = 128 (TP_EUNSUPPORTED otherwise); nq must be a positive
 * multiple of nkv, or both 0 (TP_ESHAPE).  P and dS are rounded to bf16
 * before the products that consume them; all sums are fp32 in a fixed order,
 * so results are identical run to run.  ws: device scratch of
 * tp_attn_core_bwd_workspace() bytes, 256-byte aligned, contents garbage on
 * return (per-query base-2 lse and D, and per-query-head fp32 partial dK and
 * dV: about 8 * nq * s * d bytes). */
size_t tp_attn_core_bwd_workspace(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d);
int tp_attn_core_bwd(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d,
                     const void *Q, const void *K, const void *V, const void *O, const void *dO,
                     const float *lse, void *dQ, void *dK, void *dV,
                     void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Sequence-parallel region ([book] §7.3.6)                                   */
/* ------------------------------------------------------------------------ */

/* Between a sublayer's reduce-scatter and the next sublayer's all-gather a
 * card holds only its n = s/t positions; LayerNorm and dropout act on each
 * position independently.  For every row r of the shard's [n, h] slice:
 *     u[r] = x[r] + y[r] * mask[r] / (1 - p)            (residual + dropout)
 *     z[r] = (u[r] - mean[r]) * rstd[r] * gamma + beta   (LayerNorm)
 * with mean[r] = mean_c u[r][c], rstd[r] = 1 / sqrt(mean_c (u - mean)^2 + eps).
 * y: the sublayer output after the reduce-scatter; x: the residual stream;
 * mask [n, h] uint8 (1 keep, 0 drop): the dropout draws, made by the caller
 * for drop probability p in [0, 1).  u, z [n, h] and gamma, beta [h] in bf16
 * (dt must be TP_DT_BF16); mean, rstd [n] fp32, kept for the backward.
 * h <= 16384 (TP_EUNSUPPORTED beyond). */
int tp_sp_ln_fwd(int dt, int64_t n, int64_t h, float p, float eps,
                 const void *y, const void *x, const uint8_t *mask,
                 const void *gamma, const void *beta,
                 void *u, void *z, float *mean, float *rstd, void *stream);

/* Backward: dz [n, h] is the gradient of z, dun [n, h] the gradient reaching u
 * along the residual stream from above.  With xh = (u - mean) * rstd and
 * g = dz * gamma:
 *     dx = dun + rstd * (g - mean_c g - xh * mean_c(g * xh))   (= du)
 *     dy = dx * mask / (1 - p)
 *     dgamma = sum_r dz * xh,  dbeta = sum_r dz    (this slice's share; the
 *     shards' shares are summed across cards)
 * ws: scratch of tp_sp_ln_bwd_workspace(dt, n, h) bytes, 256-byte aligned
 * (partial column sums of dgamma and dbeta, each over a fixed set of rows in
 * increasing order, reduced in a fixed order: rows h <= 8192 with h % 8 == 0
 * give min(n, 256) partials, others one per 16-row chunk). */
size_t tp_sp_ln_bwd_workspace(int dt, int64_t n, int64_t h);
int tp_sp_ln_bwd(int dt, int64_t n, int64_t h, float p,
                 const void *dz, const void *dun, const void *u,
                 const float *mean, const float *rstd, const void *gamma, const uint8_t *mask,
                 void *dx, void *dy, void *dgamma, void *dbeta,
                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Vocab-parallel output layer, cross entropy and embedding                   */
/* ([book] §7.3.4; [lec16] §5.5)                                              */
/* ------------------------------------------------------------------------ */

/* LM head split by vocab: logits(i) = Hf . Wlm(i), Hf [s,h], Wlm(i) [h,Vs],
 * logits [s,Vs] always fp32.  dt is the storage type of Hf and Wlm. */
int tp_lm_head_fwd(int dt, int64_t s, int64_t h, int64_t Vs,
                   const void *Hf, const void *Wlm, float *logits, void *stream);

/* The shard's cross-entropy statistics for every position r of its fp32
 * logit slice z [s,Vs], which covers global vocab ids [vocab_start,
 * vocab_start+Vs):
 *     lmax[r]    = max_j z[r,j]                       (-inf if Vs == 0)
 *     lsumexp[r] = sum_j exp(z[r,j] - lmax[r])        (0 if Vs == 0)
 *     tlogit[r]  = z[r, target[r]-vocab_start] if the target lies in the
 *                  shard, else 0.0
 * target [s] holds global int64 ids; any id outside the shard (negative or
 * beyond the vocabulary included) just gives tlogit = 0.  Combining the t
 * shards, M = max m_i, S = sum se_i exp(m_i - M), gives
 * loss = M + ln S - sum tlogit_i, three scalars per token exchanged instead of
 * the logits.  The sum of exponentials is taken against the shard's own max
 * (one pass); the combine rescales it.  vocab_start >= 0. */
int tp_vocab_ce(int64_t s, int64_t Vs, int64_t vocab_start,
                const float *logits, const int64_t *target,
                float *lmax, float *lsumexp, float *tlogit, void *stream);

/* Backward of the vocab-parallel cross entropy on the shard's logit slice
 * ([lec16] §5.5): with M[r], S[r] the combined maximum and sum of exponentials
 * over the whole vocabulary (M = max_i lmax_i, S = sum_i lsumexp_i
 * exp(lmax_i - M) over the shards) and dloss[r] the gradient arriving at
 * position r's loss (1/s for a mean),
 *     dlogits[r,j] = dloss[r] * (exp(z[r,j] - M[r]) / S[r] - [vocab_start + j == target[r]]),
 * softmax minus the one-hot target, restricted to the shard's columns.
 * logits [s,Vs] fp32; gmax, gsum, dloss [s] fp32 (gsum > 0, as any combine of
 * a non-empty vocabulary gives); dlogits [s,Vs] fp32 (dt = TP_DT_F32) or bf16
 * (dt = TP_DT_BF16).  A target outside the shard contributes no one-hot. */
int tp_vocab_ce_bwd(int dt, int64_t s, int64_t Vs, int64_t vocab_start,
                    const float *logits, const int64_t *target,
                    const float *gmax, const float *gsum, const float *dloss,
                    void *dlogits, void *stream);

/* LM head and cross-entropy statistics in one pass, the logits never written
 * ([lec16] §5.5: the fused vocab-parallel cross entropy keeps the [s, V/t]
 * logit slice on chip and hands on three scalars per position).  Same outputs
 * as tp_lm_head_fwd followed by tp_vocab_ce on its logits: lmax and tlogit
 * are the same fp32 values, lsumexp the same sum in another order (within
 * fp32 rounding).  Hf [s,h], Wlm [h,Vs], target [s] global ids; dt must be
 * TP_DT_BF16 (TP_EUNSUPPORTED otherwise).  ws: device scratch of at least
 * tp_lm_head_ce_workspace(dt, s, h, Vs) bytes, 256-byte aligned, overwritten
 * (per-position max and sum of exponentials of every column block of the
 * GEMM's tiling, plus the target logit: 4 * s * (2 * ceil(Vs / BN) + 1) bytes,
 * BN the tile width the call's plan takes, 128 or 256). */
size_t tp_lm_head_ce_workspace(int dt, int64_t s, int64_t h, int64_t Vs);
int tp_lm_head_ce_fwd(int dt, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start,
                      const void *Hf, const void *Wlm, const int64_t *target,
                      float *lmax, float *lsumexp, float *tlogit,
                      void *ws, size_t ws_bytes, void *stream);

/* The same as tp_lm_head_ce_fwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The per-part statistics go to a
 * scratch array the library holds on each GPU it runs on, of
 * tp_lm_head_ce_noalloc_max_bytes() = 32 MiB (with 256-wide tiles enough for
 * s * Vs up to about 1e9, e.g. s = 65536 positions of a 16032-wide shard):
 * larger requests return TP_EWORKSPACE before anything is enqueued.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The stream must belong to the current device.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (concurrent streams,
 * several host threads) race and must be serialised by the caller.  Nothing
 * in the scratch needs to start at zero: each call writes every slot it reads. */
size_t tp_lm_head_ce_noalloc_max_bytes(void);
int tp_lm_head_ce_fwd_noalloc(int dt, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start,
                              const void *Hf, const void *Wlm, const int64_t *target,
                              float *lmax, float *lsumexp, float *tlogit, void *stream);

/* Embedding rows of a vocab shard: out[r,:] = table[ids[r]-vocab_start, :]
 * when vocab_start <= ids[r] < vocab_start+Vs, else the zero vector (all bits
 * 0).  table [Vs,h], out [n,h]; dt is the element type (rows are copied bit
 * for bit).  Summing the t shards' outputs (the all-reduce) gives the full
 * lookup, since exactly one shard owns each valid id. */
int tp_vocab_embed(int dt, int64_t n, int64_t Vs, int64_t h, int64_t vocab_start,
                   const int64_t *ids, const void *table, void *out, void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */
const char *tp_status_string(int status);   /* static string; never NULL */
const char *tp_last_error(void);            /* detail of this thread's last error */
int tp_abi_version(void);                   /* TP_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* TPSHARD_H */
