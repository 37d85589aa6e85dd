/*
 * oracle.c -- plain fp64 CPU checker for one tensor-parallel shard of a
 * transformer layer.  TEST INFRASTRUCTURE ONLY: the GPU library never links,
 * loads or calls this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do.
 *
 * Every routine is the written-out definition of what the shard computes,
 * evaluated in double precision with no intermediate rounding and no
 * blocking: sums run over k in increasing order.  OpenMP only spreads the
 * independent output rows over host threads; it changes no arithmetic.
 *
 * Sources (the pages' notation is kept):
 *  - column split X[s,h] . W(i)[h,h'/t] and row split X(i)[s,h'/t] . W(i)[h'/t,h]:
 *    "7.3 模型并行与张量并行" (LLM internals book) §7.3.2, and the CMU 11-868
 *    lecture 16 notes §5.1;
 *  - MLP Z = act(X.A).B with A column-split, B row-split, one sum of partials:
 *    lecture 16 notes §5.2, book §7.3.2 worked example;
 *  - backward dY.W2^T, activation mask, .W1^T per card, partial dX summed:
 *    book §7.3.3;
 *  - head-split Q/K/V and row-split W_O, SwiGLU gate/up column split with an
 *    elementwise product and row-split down projection: book §7.3.4;
 *  - vocab-split embedding (zero vector for tokens outside the shard) and
 *    vocab-parallel cross entropy (max, sum of exponentials, target logit):
 *    book §7.3.4 and lecture 16 notes §5.5.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <stddef.h>

/* ---------------------------------------------------------------------- */
/* dense product                                                           */
/* ---------------------------------------------------------------------- */

/* C[i,j] = sum_{k=0}^{K-1} A[i,k] * B[k,j], summed over k in increasing
 * order.  A is row-major [M,K]; the right operand is passed transposed, Bt =
 * B^T row-major [N,K], so every dot product reads two contiguous rows.  The
 * caller makes transposed views contiguous first: a copy, no arithmetic. */
void or_gemm(int64_t M, int64_t N, int64_t K,
             const double *A, const double *Bt, double *C)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double *a = A + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const double *b = Bt + j * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += a[k] * b[k];
            C[i * N + j] = acc;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* element-wise activations                                                */
/* ---------------------------------------------------------------------- */
enum { OR_RELU = 0, OR_GELU = 1, OR_SILU = 2 };

static double act_f(int kind, double z)
{
    switch (kind) {
    case OR_RELU: return z > 0.0 ? z : 0.0;
    /* GeLU, exact form: z * Phi(z), Phi the standard normal CDF */
    case OR_GELU: return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
    /* SiLU (swish with beta = 1): z * sigmoid(z) */
    case OR_SILU: return z / (1.0 + exp(-z));
    }
    return NAN;
}

static double act_df(int kind, double z)
{
    switch (kind) {
    /* derivative 0 wherever the pre-activation is not positive (z = 0 included) */
    case OR_RELU: return z > 0.0 ? 1.0 : 0.0;
    case OR_GELU: {
        double Phi = 0.5 * (1.0 + erf(z / sqrt(2.0)));
        double phi = exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
        return Phi + z * phi;
    }
    case OR_SILU: {
        double sg = 1.0 / (1.0 + exp(-z));
        return sg * (1.0 + z * (1.0 - sg));
    }
    }
    return NAN;
}

void or_act(int kind, int64_t n, const double *z, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = act_f(kind, z[i]);
}

void or_act_grad(int kind, int64_t n, const double *z, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = act_df(kind, z[i]);
}

/* ---------------------------------------------------------------------- */
/* vocab-parallel cross entropy, one shard's statistics                    */
/* ---------------------------------------------------------------------- */

/* For every position r of the [s, Vs] logit slice held by the shard that
 * owns global vocab rows [start, start+Vs):
 *   m[r]  = max_j z[r,j]                       (-inf when Vs = 0)
 *   se[r] = sum_j exp(z[r,j] - m[r])           (0 when Vs = 0)
 *   tl[r] = z[r, y_r - start] if start <= y_r < start+Vs, else 0.
 * The sum of exponentials is taken against the shard's own maximum; the
 * combine below rescales it by exp(m_i - M) to the global maximum M. */
void or_ce_stats(int64_t s, int64_t Vs, int64_t start,
                 const double *z, const int64_t *target,
                 double *m, double *se, double *tl)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < s; ++r) {
        const double *row = z + r * Vs;
        double mx = -INFINITY;
        for (int64_t j = 0; j < Vs; ++j)
            if (row[j] > mx) mx = row[j];
        double acc = 0.0;
        for (int64_t j = 0; j < Vs; ++j)
            acc += exp(row[j] - mx);
        int64_t y = target[r];
        m[r] = mx;
        se[r] = acc;
        tl[r] = (y >= start && y < start + Vs) ? row[y - start] : 0.0;
    }
}

/* Combine the t shards' statistics into the per-position loss
 *   M = max_i m_i,  S = sum_i se_i * exp(m_i - M),  loss = M + ln S - sum_i tl_i.
 * Arrays are [t, s] row-major. */
void or_ce_combine(int64_t t, int64_t s, const double *m, const double *se,
                   const double *tl, double *loss)
{
    for (int64_t r = 0; r < s; ++r) {
        double M = -INFINITY;
        for (int64_t i = 0; i < t; ++i)
            if (m[i * s + r] > M) M = m[i * s + r];
        double S = 0.0, T = 0.0;
        for (int64_t i = 0; i < t; ++i) {
            if (se[i * s + r] > 0.0) S += se[i * s + r] * exp(m[i * s + r] - M);
            T += tl[i * s + r];
        }
        loss[r] = M + log(S) - T;
    }
}

/* Gradient of the loss with respect to the shard's logits: the derivative of
 * loss_r = logsumexp_j z[r,j] - z[r,y_r] is softmax minus the one-hot target,
 *   dz[r,j] = g_r * (exp(z[r,j] - M_r) / S_r - [start + j == y_r]),
 * where M_r and S_r are the combined maximum and sum of exponentials over the
 * whole vocabulary (what the combine above reduces across shards) and g_r is
 * the gradient arriving at loss_r. */
void or_ce_bwd(int64_t s, int64_t Vs, int64_t start, const double *z, const int64_t *target,
               const double *M, const double *S, const double *g, double *dz)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < s; ++r) {
        for (int64_t j = 0; j < Vs; ++j) {
            double p = exp(z[r * Vs + j] - M[r]) / S[r];
            double onehot = (start + j == target[r]) ? 1.0 : 0.0;
            dz[r * Vs + j] = g[r] * (p - onehot);
        }
    }
}

/* The unsharded definition: loss_r = logsumexp_j z[r,j] - z[r, y_r] over the
 * whole vocabulary [s, V]. */
void or_ce_direct(int64_t s, int64_t V, const double *z, const int64_t *target,
                  double *loss)
{
    for (int64_t r = 0; r < s; ++r) {
        const double *row = z + r * V;
        double mx = -INFINITY;
        for (int64_t j = 0; j < V; ++j)
            if (row[j] > mx) mx = row[j];
        double acc = 0.0;
        for (int64_t j = 0; j < V; ++j) acc += exp(row[j] - mx);
        loss[r] = mx + log(acc) - row[target[r]];
    }
}

/* ---------------------------------------------------------------------- */
/* vocab-sharded embedding lookup                                          */
/* ---------------------------------------------------------------------- */

/* out[r,:] = table[id_r - start, :] when start <= id_r < start+Vs, else the
 * zero vector.  The rows are copied as raw 16-bit patterns (bfloat16 or any
 * other 2-byte type): a lookup moves bits, it does no arithmetic. */
void or_embed_u16(int64_t n, int64_t Vs, int64_t h, int64_t start,
                  const int64_t *ids, const uint16_t *table, uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        int64_t id = ids[r];
        int in = (id >= start && id < start + Vs);
        for (int64_t c = 0; c < h; ++c)
            out[r * h + c] = in ? table[(id - start) * h + c] : (uint16_t)0;
    }
}

/* the same with 4-byte elements (fp32 tables) */
void or_embed_u32(int64_t n, int64_t Vs, int64_t h, int64_t start,
                  const int64_t *ids, const uint32_t *table, uint32_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        int64_t id = ids[r];
        int in = (id >= start && id < start + Vs);
        for (int64_t c = 0; c < h; ++c)
            out[r * h + c] = in ? table[(id - start) * h + c] : 0u;
    }
}

int or_version(void) { return 1; }

/* ---------------------------------------------------------------------- */
/* attention core on the shard's heads                                     */
/* ---------------------------------------------------------------------- */

/* Causal scaled dot-product attention of the nq query heads a shard holds,
 * sharing nkv key/value heads (query head j reads KV head j / (nq / nkv)).
 * Q [s][nq*d], K and V [s][nkv*d], row-major with head j in columns
 * [j*d, (j+1)*d).  For every head j and each of the nr positions r = rows[i]:
 *   S[c]   = (Q_j[r] . K_g[c]) / sqrt(d)          for c = 0..r (causal)
 *   lse    = m + ln sum_c exp(S[c] - m),  m = max_c S[c]
 *   O_j[r] = sum_c exp(S[c] - lse) V_g[c]
 * written to O [nr][nq*d] and lse [nq][nr].  With causal = 0 every c in
 * 0..s-1 is visible. */
void or_attn_fwd(int64_t s, int64_t nq, int64_t nkv, int64_t d, int causal, const double *Q,
                 const double *K, const double *V, int64_t nr, const int64_t *rows, double *O,
                 double *lse)
{
    const int64_t grp = nq / nkv, lq = nq * d, lk = nkv * d;
    const double scale = 1.0 / sqrt((double)d);
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t j = 0; j < nq; ++j) {
        for (int64_t i = 0; i < nr; ++i) {
            const int64_t r = rows[i], g = j / grp;
            const int64_t n = causal ? r + 1 : s;
            double *S = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
            double m = -INFINITY;
            for (int64_t c = 0; c < n; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < d; ++k) acc += Q[r * lq + j * d + k] * K[c * lk + g * d + k];
                S[c] = acc * scale;
                if (S[c] > m) m = S[c];
            }
            double sum = 0.0;
            for (int64_t c = 0; c < n; ++c) sum += exp(S[c] - m);
            const double L = m + log(sum);
            lse[j * nr + i] = L;
            for (int64_t k = 0; k < d; ++k) {
                double acc = 0.0;
                for (int64_t c = 0; c < n; ++c) acc += exp(S[c] - L) * V[c * lk + g * d + k];
                O[i * lq + j * d + k] = acc;
            }
            free(S);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* sequence-parallel region: residual add, dropout and LayerNorm           */
/* ---------------------------------------------------------------------- */

/* One shard's [n, h] slice of positions (n = s/t) in the region outside the
 * tensor-parallel sublayers.  y is the sublayer output after the
 * reduce-scatter, x the residual stream, mask the dropout mask (1 keep, 0
 * drop) drawn for drop probability p, gamma/beta the LayerNorm parameters:
 *   u[r]  = x[r] + y[r] * mask[r] / (1 - p)
 *   mu    = mean_c u[r][c],  var = mean_c (u[r][c] - mu)^2,  rstd = 1/sqrt(var + eps)
 *   z[r]  = (u[r] - mu) * rstd * gamma + beta
 * u, z [n][h]; mean, rstd [n]. */
void or_sp_ln_fwd(int64_t n, int64_t h, double p, double eps, const double *y, const double *x,
                  const uint8_t *mask, const double *gamma, const double *beta, double *u, double *z,
                  double *mean, double *rstd)
{
    const double keep = 1.0 / (1.0 - p);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double mu = 0.0;
        for (int64_t c = 0; c < h; ++c) {
            const double v = x[r * h + c] + y[r * h + c] * (double)mask[r * h + c] * keep;
            u[r * h + c] = v;
            mu += v;
        }
        mu /= (double)h;
        double var = 0.0;
        for (int64_t c = 0; c < h; ++c) {
            const double dv = u[r * h + c] - mu;
            var += dv * dv;
        }
        var /= (double)h;
        const double rs = 1.0 / sqrt(var + eps);
        mean[r] = mu;
        rstd[r] = rs;
        for (int64_t c = 0; c < h; ++c) z[r * h + c] = (u[r * h + c] - mu) * rs * gamma[c] + beta[c];
    }
}

/* Backward of the above: dz is the gradient of z, dun the gradient reaching u
 * along the residual stream from the layer above.  With xh = (u - mu) rstd and
 * g = dz * gamma:
 *   du     = dun + rstd * (g - mean_c g - xh * mean_c (g xh))     (LayerNorm backward)
 *   dx     = du                       (the residual input)
 *   dy     = du * mask / (1 - p)      (the sublayer output, before the all-gather)
 *   dgamma = sum_r dz * xh,  dbeta = sum_r dz   (this slice's share) */
void or_sp_ln_bwd(int64_t n, int64_t h, double p, const double *dz, const double *dun, const double *u,
                  const double *mean, const double *rstd, const double *gamma, const uint8_t *mask,
                  double *dx, double *dy, double *dgamma, double *dbeta)
{
    const double keep = 1.0 / (1.0 - p);
    for (int64_t c = 0; c < h; ++c) dgamma[c] = dbeta[c] = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        double mg = 0.0, mgx = 0.0;
        for (int64_t c = 0; c < h; ++c) {
            const double xh = (u[r * h + c] - mean[r]) * rstd[r];
            const double g = dz[r * h + c] * gamma[c];
            mg += g;
            mgx += g * xh;
            dgamma[c] += dz[r * h + c] * xh;
            dbeta[c] += dz[r * h + c];
        }
        mg /= (double)h;
        mgx /= (double)h;
        for (int64_t c = 0; c < h; ++c) {
            const double xh = (u[r * h + c] - mean[r]) * rstd[r];
            const double g = dz[r * h + c] * gamma[c];
            const double du = dun[r * h + c] + rstd[r] * (g - mg - xh * mgx);
            dx[r * h + c] = du;
            dy[r * h + c] = du * (double)mask[r * h + c] * keep;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* attention core on the shard's heads: backward                           */
/* ---------------------------------------------------------------------- */

/* Gradients of or_attn_fwd's O with respect to Q, K and V, given dO, the
 * gradient arriving at O (same layout as O).  Differentiating
 * O_j[r] = sum_c P[r][c] V_g[c] with P[r][.] = softmax_c(S[r][.]) and
 * S[r][c] = Q_j[r] . K_g[c] / sqrt(d), for each head j (KV head g = j / (nq/nkv)):
 *   dP[r][c] = dO_j[r] . V_g[c]
 *   D[r]     = sum_c P[r][c] dP[r][c]            (softmax Jacobian: dS = P (dP - D))
 *   dS[r][c] = P[r][c] (dP[r][c] - D[r])
 *   dQ_j[r]  = sum_c dS[r][c] K_g[c] / sqrt(d)
 *   dK_g[c]  = sum over the heads j of group g, then over r, of dS[r][c] Q_j[r] / sqrt(d)
 *   dV_g[c]  = sum over the heads j of group g, then over r, of P[r][c] dO_j[r]
 * with c <= r when causal.  The query heads of a group share their key/value
 * head, so its gradient is the sum of theirs (heads in increasing order, rows
 * in increasing order).
 * Outputs are taken at nr sampled positions rows[] (dQ [nr][nq*d]) and nc
 * sampled key positions cols[] (dK, dV [nc][nkv*d]); all positions give the
 * whole backward.  P and D are first evaluated for every (head, position),
 * since a key's gradient needs every later query's softmax. */
void or_attn_bwd(int64_t s, int64_t nq, int64_t nkv, int64_t d, int causal, const double *Q,
                 const double *K, const double *V, const double *dO, int64_t nr, const int64_t *rows,
                 int64_t nc, const int64_t *cols, double *dQ, double *dK, double *dV)
{
    const int64_t grp = nq / nkv, lq = nq * d, lk = nkv * d;
    const double scale = 1.0 / sqrt((double)d);
    double *lse = (double *)malloc((size_t)(nq * s > 0 ? nq * s : 1) * sizeof(double));
    double *Dv = (double *)malloc((size_t)(nq * s > 0 ? nq * s : 1) * sizeof(double));

    /* log-sum-exp of every score row and D of every (head, position) */
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t j = 0; j < nq; ++j) {
        for (int64_t r = 0; r < s; ++r) {
            const int64_t g = j / grp, n = causal ? r + 1 : s;
            double *S = (double *)malloc((size_t)n * sizeof(double));
            double m = -INFINITY;
            for (int64_t c = 0; c < n; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < d; ++k) acc += Q[r * lq + j * d + k] * K[c * lk + g * d + k];
                S[c] = acc * scale;
                if (S[c] > m) m = S[c];
            }
            double sum = 0.0;
            for (int64_t c = 0; c < n; ++c) sum += exp(S[c] - m);
            const double L = m + log(sum);
            double Dr = 0.0;
            for (int64_t c = 0; c < n; ++c) {
                double dp = 0.0;
                for (int64_t k = 0; k < d; ++k) dp += dO[r * lq + j * d + k] * V[c * lk + g * d + k];
                Dr += exp(S[c] - L) * dp;
            }
            lse[j * s + r] = L;
            Dv[j * s + r] = Dr;
            free(S);
        }
    }

    /* dQ at the sampled positions */
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t j = 0; j < nq; ++j) {
        for (int64_t i = 0; i < nr; ++i) {
            const int64_t r = rows[i], g = j / grp, n = causal ? r + 1 : s;
            double *out = dQ + i * lq + j * d;
            for (int64_t k = 0; k < d; ++k) out[k] = 0.0;
            for (int64_t c = 0; c < n; ++c) {
                double sc = 0.0, dp = 0.0;
                for (int64_t k = 0; k < d; ++k) {
                    sc += Q[r * lq + j * d + k] * K[c * lk + g * d + k];
                    dp += dO[r * lq + j * d + k] * V[c * lk + g * d + k];
                }
                const double p = exp(sc * scale - lse[j * s + r]);
                const double ds = p * (dp - Dv[j * s + r]);
                for (int64_t k = 0; k < d; ++k) out[k] += ds * K[c * lk + g * d + k] * scale;
            }
        }
    }

    /* dK and dV at the sampled key positions */
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t g = 0; g < nkv; ++g) {
        for (int64_t i = 0; i < nc; ++i) {
            const int64_t c = cols[i];
            double *ok = dK + i * lk + g * d, *ov = dV + i * lk + g * d;
            for (int64_t k = 0; k < d; ++k) ok[k] = ov[k] = 0.0;
            for (int64_t j = g * grp; j < (g + 1) * grp; ++j) {
                for (int64_t r = causal ? c : 0; r < s; ++r) {
                    double sc = 0.0, dp = 0.0;
                    for (int64_t k = 0; k < d; ++k) {
                        sc += Q[r * lq + j * d + k] * K[c * lk + g * d + k];
                        dp += dO[r * lq + j * d + k] * V[c * lk + g * d + k];
                    }
                    const double p = exp(sc * scale - lse[j * s + r]);
                    const double ds = p * (dp - Dv[j * s + r]);
                    for (int64_t k = 0; k < d; ++k) {
                        ok[k] += ds * Q[r * lq + j * d + k] * scale;
                        ov[k] += p * dO[r * lq + j * d + k];
                    }
                }
            }
        }
    }
    free(lse);
    free(Dv);
}
