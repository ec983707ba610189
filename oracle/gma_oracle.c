/*
 * gma_oracle.c -- plain fp64 CPU oracle of the Gaussian Mixture Attention
 * (GMA) mixer: forward, and its backward (gma_oracle_backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * Source of every formula: the page "Attention par Melange Gaussien (GMA)"
 * (gist.science, paper 2606.18283), section "Methodologie: Attention par
 * Melange Gaussien (GMA)", sub-section "Mecanisme Central":
 *   item 1 "Routage Latent Probabiliste"  -> gma_oracle_responsibilities
 *   item 2 "Routage de Memoire Latente"   -> gma_oracle_forward (write phase,
 *                                            read phase equation)
 *   item 3 "Variantes et Entrainement"    -> gma_oracle_params (softplus
 *                                            variances, softmax priors) and
 *                                            the causal prefix-sum variant.
 *
 * Everything is the plain definition, in fp64, in the pages' order:
 *   sigma2_kd = softplus(rho_kd) = log(1 + e^rho)
 *   log pi_k  = lambda_k - log sum_j e^lambda_j
 *   l_k(x)    = log pi_k - 1/2 sum_d [ log(2 pi sigma2_kd) + (x_d - mu_kd)^2 / sigma2_kd ]
 *   gamma_k   = e^{l_k} / sum_j e^{l_j}           (posterior p(z = k | x))
 *   Vt = Gamma_K^T V, Z = Gamma_K^T 1             (bidirectional write)
 *   O  = Gamma_Q Vt / (Gamma_Q Z + eps)           (read; one scalar per row)
 *   causal: Vt and Z are running sums over j <= i (the diagonal included).
 *
 * The Gaussian is taken in its direct form (x - mu)^2 / sigma2, not the
 * expanded quadratic the GPU uses.  Sums over n run sequentially in n; each
 * output element is produced by one thread in a fixed order, so results are
 * bitwise independent of the OpenMP thread count.
 *
 * Memory: Gamma rows are produced one block of rows at a time and consumed
 * in row order.  Rows are independent, so this only bounds memory (a head of
 * one million tokens would need gigabytes of Gamma otherwise); the arithmetic
 * of every element is unchanged.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ROW_BLOCK 4096

static const double TWO_PI = 6.283185307179586476925286766559;

/* softplus(r) = log(1 + e^r), written so that it neither overflows nor loses
 * the small-r tail: max(r, 0) + log1p(e^{-|r|}). */
static double softplus(double r) { return fmax(r, 0.0) + log1p(exp(-fabs(r))); }

void gma_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int gma_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Reparameterisation ("Variantes et Entrainement"): variances by softplus,
 * priors by softmax (returned as log pi).  Shapes: raw_var, var [H, K, d_r];
 * prior_logits, log_prior [H, K]. */
void gma_oracle_params(int64_t H, int32_t K, int32_t dr, const double* raw_var,
                       const double* prior_logits, double* var, double* log_prior) {
    for (int64_t i = 0; i < H * K * dr; ++i) var[i] = softplus(raw_var[i]);
    for (int64_t h = 0; h < H; ++h) {
        const double* lam = prior_logits + h * K;
        double m = lam[0];
        for (int k = 1; k < K; ++k) m = fmax(m, lam[k]);
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += exp(lam[k] - m);
        double lse = m + log(s);
        for (int k = 0; k < K; ++k) log_prior[h * K + k] = lam[k] - lse;
    }
}

/* Posterior responsibilities of one row x[d_r] under one head's mixture
 * ("Routage Latent Probabiliste").  mu, var [K, d_r]; log_prior [K];
 * logdet[k] = sum_d log(2 pi var_kd) (a per-component constant).
 * gamma[K] receives p(z = k | x). */
static void row_responsibilities(int32_t K, int32_t dr, const double* x, const double* mu,
                                 const double* var, const double* log_prior,
                                 const double* logdet, double* gamma) {
    double m = -INFINITY;
    for (int k = 0; k < K; ++k) {
        double q = 0.0;
        for (int d = 0; d < dr; ++d) {
            double diff = x[d] - mu[(int64_t)k * dr + d];
            q += diff * diff / var[(int64_t)k * dr + d];
        }
        double l = log_prior[k] - 0.5 * (logdet[k] + q);
        gamma[k] = l;
        if (l > m) m = l;
    }
    double s = 0.0;
    for (int k = 0; k < K; ++k) {
        gamma[k] = exp(gamma[k] - m);
        s += gamma[k];
    }
    for (int k = 0; k < K; ++k) gamma[k] /= s;
}

static void head_logdet(int32_t K, int32_t dr, const double* var, double* logdet) {
    for (int k = 0; k < K; ++k) {
        double s = 0.0;
        for (int d = 0; d < dr; ++d) s += log(TWO_PI * var[(int64_t)k * dr + d]);
        logdet[k] = s;
    }
}

/* Responsibilities of every row of x [B, H, N, d_r] -> gamma [B, H, N, K].
 * Parameters are the raw learned ones: mu, raw_var [H, K, d_r], prior_logits [H, K]. */
int gma_oracle_responsibilities(int64_t B, int64_t H, int64_t N, int32_t dr, int32_t K,
                                const double* x, const double* mu, const double* raw_var,
                                const double* prior_logits, double* gamma) {
    double* var = (double*)malloc(sizeof(double) * H * K * dr);
    double* logp = (double*)malloc(sizeof(double) * H * K);
    double* logdet = (double*)malloc(sizeof(double) * H * K);
    if (!var || !logp || !logdet) { free(var); free(logp); free(logdet); return 1; }
    gma_oracle_params(H, K, dr, raw_var, prior_logits, var, logp);
    for (int64_t h = 0; h < H; ++h) head_logdet(K, dr, var + h * K * dr, logdet + h * K);
    int64_t rows = B * H * N;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t h = (r / N) % H;
        row_responsibilities(K, dr, x + r * dr, mu + h * K * dr, var + h * K * dr, logp + h * K,
                             logdet + h * K, gamma + r * K);
    }
    free(var); free(logp); free(logdet);
    return 0;
}

/* Forward mixer ("Routage de Memoire Latente" and "Variantes et Entrainement").
 * qx, kx [B, H, N, d_r]; v [B, H, N, d_v]; o [B, H, N, d_v]; causal = 0 or 1.
 * Causal only: state_in (or NULL = zero) is the latent memory before the first token and
 * state_out (or NULL) receives it after the last one, both [B, H, K, d_v + 1]: row k holds
 * Vt[k, 0 .. d_v-1] and then Z[k].  The running sums simply start from state_in.
 * Returns 0, or 1 if memory could not be allocated. */
static int forward_impl(int causal, int64_t B, int64_t H, int64_t N, int32_t dr, int32_t K,
                        int32_t dv, double eps, const double* qx, const double* kx,
                        const double* v, const double* mu, const double* raw_var,
                        const double* prior_logits, const double* state_in, double* state_out,
                        double* o) {
    double* var = (double*)malloc(sizeof(double) * H * K * dr);
    double* logp = (double*)malloc(sizeof(double) * H * K);
    double* logdet = (double*)malloc(sizeof(double) * H * K);
    double* gq = (double*)malloc(sizeof(double) * ORACLE_ROW_BLOCK * K);
    double* gk = (double*)malloc(sizeof(double) * ORACLE_ROW_BLOCK * K);
    double* vt = (double*)malloc(sizeof(double) * (int64_t)K * dv);   /* latent memory Vt [K, d_v] */
    double* z = (double*)malloc(sizeof(double) * K);                  /* normaliser Z [K] */
    double* den = (double*)malloc(sizeof(double) * ORACLE_ROW_BLOCK);
    int rc = 0;
    if (!var || !logp || !logdet || !gq || !gk || !vt || !z || !den) { rc = 1; goto done; }
    gma_oracle_params(H, K, dr, raw_var, prior_logits, var, logp);
    for (int64_t h = 0; h < H; ++h) head_logdet(K, dr, var + h * K * dr, logdet + h * K);

    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t h = bh % H;
        const double* mu_h = mu + h * K * dr;
        const double* var_h = var + h * K * dr;
        const double* lp_h = logp + h * K;
        const double* ld_h = logdet + h * K;
        const double* q_bh = qx + bh * N * dr;
        const double* k_bh = kx + bh * N * dr;
        const double* v_bh = v + bh * N * dv;
        double* o_bh = o + bh * N * dv;
        memset(vt, 0, sizeof(double) * (size_t)K * dv);
        memset(z, 0, sizeof(double) * (size_t)K);
        if (causal && state_in) {
            const double* s = state_in + bh * K * (dv + 1);
            for (int k = 0; k < K; ++k) {
                for (int c = 0; c < dv; ++c) vt[(int64_t)k * dv + c] = s[(int64_t)k * (dv + 1) + c];
                z[k] = s[(int64_t)k * (dv + 1) + dv];
            }
        }

        if (!causal) {
            /* Write phase over the whole sequence: Vt = Gamma_K^T V, Z = Gamma_K^T 1. */
            for (int64_t n0 = 0; n0 < N; n0 += ORACLE_ROW_BLOCK) {
                int64_t nb = (N - n0 < ORACLE_ROW_BLOCK) ? N - n0 : ORACLE_ROW_BLOCK;
#pragma omp parallel for schedule(static)
                for (int64_t r = 0; r < nb; ++r)
                    row_responsibilities(K, dr, k_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, gk + r * K);
                for (int64_t r = 0; r < nb; ++r)
                    for (int k = 0; k < K; ++k) z[k] += gk[r * K + k];
#pragma omp parallel for schedule(static)
                for (int c = 0; c < dv; ++c)
                    for (int64_t r = 0; r < nb; ++r)
                        for (int k = 0; k < K; ++k)
                            vt[(int64_t)k * dv + c] += gk[r * K + k] * v_bh[(n0 + r) * dv + c];
            }
            /* Read phase: O_n = (Gamma_Q[n] Vt) / (Gamma_Q[n] . Z + eps). */
            for (int64_t n0 = 0; n0 < N; n0 += ORACLE_ROW_BLOCK) {
                int64_t nb = (N - n0 < ORACLE_ROW_BLOCK) ? N - n0 : ORACLE_ROW_BLOCK;
#pragma omp parallel for schedule(static)
                for (int64_t r = 0; r < nb; ++r) {
                    double* g = gq + r * K;
                    row_responsibilities(K, dr, q_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, g);
                    double d = 0.0;
                    for (int k = 0; k < K; ++k) d += g[k] * z[k];
                    d += eps;
                    for (int c = 0; c < dv; ++c) {
                        double num = 0.0;
                        for (int k = 0; k < K; ++k) num += g[k] * vt[(int64_t)k * dv + c];
                        o_bh[(n0 + r) * dv + c] = num / d;
                    }
                }
            }
        } else {
            /* Causal: for n = 0 .. N-1 in order, Vt += gamma_K[n] (x) v[n], Z += gamma_K[n],
             * then O_n = (gamma_Q[n] Vt) / (gamma_Q[n] . Z + eps).  Inclusive of j = n. */
            for (int64_t n0 = 0; n0 < N; n0 += ORACLE_ROW_BLOCK) {
                int64_t nb = (N - n0 < ORACLE_ROW_BLOCK) ? N - n0 : ORACLE_ROW_BLOCK;
#pragma omp parallel for schedule(static)
                for (int64_t r = 0; r < nb; ++r) {
                    row_responsibilities(K, dr, q_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, gq + r * K);
                    row_responsibilities(K, dr, k_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, gk + r * K);
                }
                /* Denominators: Z as a running sum, one scalar per row. */
                for (int64_t r = 0; r < nb; ++r) {
                    for (int k = 0; k < K; ++k) z[k] += gk[r * K + k];
                    double d = 0.0;
                    for (int k = 0; k < K; ++k) d += gq[r * K + k] * z[k];
                    den[r] = d + eps;
                }
                /* Numerators: column c of Vt is a running sum of its own. */
#pragma omp parallel for schedule(static)
                for (int c = 0; c < dv; ++c) {
                    for (int64_t r = 0; r < nb; ++r) {
                        const double vc = v_bh[(n0 + r) * dv + c];
                        double num = 0.0;
                        for (int k = 0; k < K; ++k) {
                            vt[(int64_t)k * dv + c] += gk[r * K + k] * vc;
                            num += gq[r * K + k] * vt[(int64_t)k * dv + c];
                        }
                        o_bh[(n0 + r) * dv + c] = num / den[r];
                    }
                }
            }
            if (state_out) {
                double* s = state_out + bh * K * (dv + 1);
                for (int k = 0; k < K; ++k) {
                    for (int c = 0; c < dv; ++c) s[(int64_t)k * (dv + 1) + c] = vt[(int64_t)k * dv + c];
                    s[(int64_t)k * (dv + 1) + dv] = z[k];
                }
            }
        }
    }
done:
    free(var); free(logp); free(logdet); free(gq); free(gk); free(vt); free(z); free(den);
    return rc;
}

int gma_oracle_forward(int causal, int64_t B, int64_t H, int64_t N, int32_t dr, int32_t K,
                       int32_t dv, double eps, const double* qx, const double* kx,
                       const double* v, const double* mu, const double* raw_var,
                       const double* prior_logits, double* o) {
    return forward_impl(causal, B, H, N, dr, K, dv, eps, qx, kx, v, mu, raw_var, prior_logits, NULL, NULL, o);
}

/* Bidirectional forward with separate query and key/value sequences (cross-attention): the write
 * phase runs over the Nk rows of kx [B, H, Nk, d_r] and v [B, H, Nk, d_v], the read phase over the
 * Nq rows of qx [B, H, Nq, d_r]; o [B, H, Nq, d_v].  The same definitions as the bidirectional
 * forward above; one GMM per head routes both sides.  Returns 0, or 1 if memory could not be
 * allocated. */
int gma_oracle_forward_bidir_kv(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int32_t dr, int32_t K,
                                int32_t dv, double eps, const double* qx, const double* kx,
                                const double* v, const double* mu, const double* raw_var,
                                const double* prior_logits, double* o) {
    double* var = (double*)malloc(sizeof(double) * H * K * dr);
    double* logp = (double*)malloc(sizeof(double) * H * K);
    double* logdet = (double*)malloc(sizeof(double) * H * K);
    double* g = (double*)malloc(sizeof(double) * ORACLE_ROW_BLOCK * K);
    double* vt = (double*)malloc(sizeof(double) * (int64_t)K * dv);
    double* z = (double*)malloc(sizeof(double) * K);
    int rc = 0;
    if (!var || !logp || !logdet || !g || !vt || !z) { rc = 1; goto done; }
    gma_oracle_params(H, K, dr, raw_var, prior_logits, var, logp);
    for (int64_t h = 0; h < H; ++h) head_logdet(K, dr, var + h * K * dr, logdet + h * K);
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t h = bh % H;
        const double* mu_h = mu + h * K * dr;
        const double* var_h = var + h * K * dr;
        const double* lp_h = logp + h * K;
        const double* ld_h = logdet + h * K;
        const double* q_bh = qx + bh * Nq * dr;
        const double* k_bh = kx + bh * Nk * dr;
        const double* v_bh = v + bh * Nk * dv;
        double* o_bh = o + bh * Nq * dv;
        memset(vt, 0, sizeof(double) * (size_t)K * dv);
        memset(z, 0, sizeof(double) * (size_t)K);
        /* write phase over the key/value rows: Vt = Gamma_K^T V, Z = Gamma_K^T 1 */
        for (int64_t n0 = 0; n0 < Nk; n0 += ORACLE_ROW_BLOCK) {
            int64_t nb = (Nk - n0 < ORACLE_ROW_BLOCK) ? Nk - n0 : ORACLE_ROW_BLOCK;
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < nb; ++r)
                row_responsibilities(K, dr, k_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, g + r * K);
            for (int64_t r = 0; r < nb; ++r)
                for (int k = 0; k < K; ++k) z[k] += g[r * K + k];
#pragma omp parallel for schedule(static)
            for (int c = 0; c < dv; ++c)
                for (int64_t r = 0; r < nb; ++r)
                    for (int k = 0; k < K; ++k)
                        vt[(int64_t)k * dv + c] += g[r * K + k] * v_bh[(n0 + r) * dv + c];
        }
        /* read phase over the query rows: O_n = (Gamma_Q[n] Vt) / (Gamma_Q[n] . Z + eps) */
        for (int64_t n0 = 0; n0 < Nq; n0 += ORACLE_ROW_BLOCK) {
            int64_t nb = (Nq - n0 < ORACLE_ROW_BLOCK) ? Nq - n0 : ORACLE_ROW_BLOCK;
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < nb; ++r) {
                double* gr = g + r * K;
                row_responsibilities(K, dr, q_bh + (n0 + r) * dr, mu_h, var_h, lp_h, ld_h, gr);
                double d = 0.0;
                for (int k = 0; k < K; ++k) d += gr[k] * z[k];
                d += eps;
                for (int c = 0; c < dv; ++c) {
                    double num = 0.0;
                    for (int k = 0; k < K; ++k) num += gr[k] * vt[(int64_t)k * dv + c];
                    o_bh[(n0 + r) * dv + c] = num / d;
                }
            }
        }
    }
done:
    free(var); free(logp); free(logdet); free(g); free(vt); free(z);
    return rc;
}

/* Causal forward with the latent memory carried in (state_in, NULL = zero) and out (state_out,
 * NULL = not wanted); layouts as above. */
int gma_oracle_forward_causal_state(int64_t B, int64_t H, int64_t N, int32_t dr, int32_t K,
                                    int32_t dv, double eps, const double* qx, const double* kx,
                                    const double* v, const double* mu, const double* raw_var,
                                    const double* prior_logits, const double* state_in,
                                    double* state_out, double* o) {
    return forward_impl(1, B, H, N, dr, K, dv, eps, qx, kx, v, mu, raw_var, prior_logits, state_in, state_out, o);
}

/* ---- Backward of the mixer: gradients of a loss L with respect to every input, given
 * dout = dL/dO.  The pages train the layer end to end ("Variantes et Entrainement"), so the
 * gradient is the chain rule through the definitions above, applied step by step:
 *   read phase   O_i = num_i / den_i, num_i = Gamma_Q[i] Vt_i, den_i = Gamma_Q[i] . Z_i + eps
 *                  g_i = dO_i / den_i                       (dL/dnum_i)
 *                  h_i = -(dO_i . O_i) / den_i              (dL/dden_i)
 *                  dGamma_Q[i][k] = Vt_i[k] . g_i + Z_i[k] h_i
 *   write phase  Vt_i, Z_i = sums of gamma_K[j] (x) v_j and gamma_K[j] over j <= i (causal) or
 *                over all j (bidirectional); every query i that sees key j contributes
 *                  dGamma_K[j][k] = sum_{i sees j} Gamma_Q[i][k] (v_j . g_i + h_i)
 *                  dv_j           = sum_{i sees j} (Gamma_Q[i] . gamma_K[j]) g_i
 *   posterior    gamma = softmax_k(l_k): dl_k = gamma_k (dgamma_k - sum_j gamma_j dgamma_j)
 *   log-density  l_k(x) = log pi_k - 1/2 sum_d [log(2 pi s_kd) + (x_d - mu_kd)^2 / s_kd]:
 *                  dx_d   = sum_k dl_k (mu_kd - x_d) / s_kd
 *                  dmu_kd = sum over rows of dl_k (x_d - mu_kd) / s_kd
 *                  ds_kd  = sum over rows of dl_k ((x_d - mu_kd)^2 / s_kd^2 - 1 / s_kd) / 2
 *                  dlog pi_k = sum over rows of dl_k
 *   parameters   s = softplus(rho): drho = ds * sigmoid(rho);
 *                log pi = lambda - logsumexp(lambda): dlambda_j = G_j - pi_j sum_k G_k with
 *                G = dlog pi.
 * Rows of both Q_X and K_X contribute to the parameter gradients (one mixture per head routes
 * both).  Sums over the sequence run sequentially; the per-(b, h) parameter partials are added
 * over b in order, so the result is independent of the thread count.
 * dqx, dkx [B, H, N, d_r]; dv [B, H, N, d_v]; dmu, draw_var [H, K, d_r]; dprior_logits [H, K].
 * Returns 0, or 1 if memory could not be allocated. */
static void row_logit_backward(int32_t K, int32_t dr, const double* x, const double* mu,
                               const double* var, const double* gamma, const double* dgamma,
                               double* dx, double* dmu_acc, double* dvar_acc, double* dlogp_acc) {
    double dot = 0.0;
    for (int k = 0; k < K; ++k) dot += gamma[k] * dgamma[k];
    for (int d = 0; d < dr; ++d) dx[d] = 0.0;
    for (int k = 0; k < K; ++k) {
        const double dl = gamma[k] * (dgamma[k] - dot);
        dlogp_acc[k] += dl;
        for (int d = 0; d < dr; ++d) {
            const double s = var[(int64_t)k * dr + d];
            const double diff = x[d] - mu[(int64_t)k * dr + d];
            dx[d] += dl * (-diff) / s;
            dmu_acc[(int64_t)k * dr + d] += dl * diff / s;
            dvar_acc[(int64_t)k * dr + d] += dl * 0.5 * (diff * diff / (s * s) - 1.0 / s);
        }
    }
}

int gma_oracle_backward(int causal, int64_t B, int64_t H, int64_t N, int32_t dr, int32_t K,
                        int32_t dv, double eps, const double* qx, const double* kx,
                        const double* v, const double* mu, const double* raw_var,
                        const double* prior_logits, const double* dout, double* dqx,
                        double* dkx, double* dvv, double* dmu, double* draw_var,
                        double* dprior_logits) {
    const int64_t BH = B * H, KD = (int64_t)K * dr;
    double* var = (double*)malloc(sizeof(double) * H * KD);
    double* logp = (double*)malloc(sizeof(double) * H * K);
    double* logdet = (double*)malloc(sizeof(double) * H * K);
    double* pmu = (double*)calloc((size_t)(BH * KD), sizeof(double));    /* per-(b, h) partials */
    double* pvar = (double*)calloc((size_t)(BH * KD), sizeof(double));
    double* plogp = (double*)calloc((size_t)(BH * K), sizeof(double));
    int rc = 0;
    if (!var || !logp || !logdet || !pmu || !pvar || !plogp) { rc = 1; goto done; }
    gma_oracle_params(H, K, dr, raw_var, prior_logits, var, logp);
    for (int64_t h = 0; h < H; ++h) head_logdet(K, dr, var + h * KD, logdet + h * K);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t h = bh % H;
        const double* mu_h = mu + h * KD;
        const double* var_h = var + h * KD;
        const double* q_bh = qx + bh * N * dr;
        const double* k_bh = kx + bh * N * dr;
        const double* v_bh = v + bh * N * dv;
        const double* do_bh = dout + bh * N * dv;
        double* gq = (double*)malloc(sizeof(double) * N * K);
        double* gk = (double*)malloc(sizeof(double) * N * K);
        double* dgq = (double*)malloc(sizeof(double) * N * K);
        double* dgk = (double*)malloc(sizeof(double) * N * K);
        double* gg = (double*)malloc(sizeof(double) * N * dv);   /* g_i */
        double* hh = (double*)malloc(sizeof(double) * N);        /* h_i */
        double* st = (double*)malloc(sizeof(double) * (int64_t)K * dv);
        double* z = (double*)malloc(sizeof(double) * K);
        if (!gq || !gk || !dgq || !dgk || !gg || !hh || !st || !z) {
#pragma omp atomic write
            rc = 1;
            free(gq); free(gk); free(dgq); free(dgk); free(gg); free(hh); free(st); free(z);
            continue;
        }
        for (int64_t n = 0; n < N; ++n) {
            row_responsibilities(K, dr, q_bh + n * dr, mu_h, var_h, logp + h * K, logdet + h * K, gq + n * K);
            row_responsibilities(K, dr, k_bh + n * dr, mu_h, var_h, logp + h * K, logdet + h * K, gk + n * K);
        }
        /* read phase and its gradient, queries in order (the latent memory Vt, Z as of query i) */
        memset(st, 0, sizeof(double) * (size_t)K * dv);
        memset(z, 0, sizeof(double) * (size_t)K);
        if (!causal) {
            for (int64_t j = 0; j < N; ++j)
                for (int k = 0; k < K; ++k) {
                    z[k] += gk[j * K + k];
                    for (int c = 0; c < dv; ++c) st[(int64_t)k * dv + c] += gk[j * K + k] * v_bh[j * dv + c];
                }
        }
        for (int64_t i = 0; i < N; ++i) {
            if (causal) {
                for (int k = 0; k < K; ++k) {
                    z[k] += gk[i * K + k];
                    for (int c = 0; c < dv; ++c) st[(int64_t)k * dv + c] += gk[i * K + k] * v_bh[i * dv + c];
                }
            }
            double den = 0.0;
            for (int k = 0; k < K; ++k) den += gq[i * K + k] * z[k];
            den += eps;
            double dot = 0.0;   /* dO_i . O_i */
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int k = 0; k < K; ++k) num += gq[i * K + k] * st[(int64_t)k * dv + c];
                dot += do_bh[i * dv + c] * (num / den);
                gg[i * dv + c] = do_bh[i * dv + c] / den;
            }
            hh[i] = -dot / den;
            for (int k = 0; k < K; ++k) {
                double s = 0.0;
                for (int c = 0; c < dv; ++c) s += st[(int64_t)k * dv + c] * gg[i * dv + c];
                dgq[i * K + k] = s + z[k] * hh[i];
            }
        }
        /* write phase gradient, keys in reverse order: R = sum over the queries that see key j of
         * Gamma_Q[i] (x) g_i, r = the same sum of Gamma_Q[i] h_i */
        memset(st, 0, sizeof(double) * (size_t)K * dv);
        memset(z, 0, sizeof(double) * (size_t)K);
        if (!causal) {
            for (int64_t i = 0; i < N; ++i)
                for (int k = 0; k < K; ++k) {
                    z[k] += gq[i * K + k] * hh[i];
                    for (int c = 0; c < dv; ++c) st[(int64_t)k * dv + c] += gq[i * K + k] * gg[i * dv + c];
                }
        }
        double* dv_bh = dvv + bh * N * dv;
        for (int64_t j = N - 1; j >= 0; --j) {
            if (causal) {
                for (int k = 0; k < K; ++k) {
                    z[k] += gq[j * K + k] * hh[j];
                    for (int c = 0; c < dv; ++c) st[(int64_t)k * dv + c] += gq[j * K + k] * gg[j * dv + c];
                }
            }
            for (int k = 0; k < K; ++k) {
                double s = 0.0;
                for (int c = 0; c < dv; ++c) s += st[(int64_t)k * dv + c] * v_bh[j * dv + c];
                dgk[j * K + k] = s + z[k];
            }
            for (int c = 0; c < dv; ++c) {
                double s = 0.0;
                for (int k = 0; k < K; ++k) s += gk[j * K + k] * st[(int64_t)k * dv + c];
                dv_bh[j * dv + c] = s;
            }
        }
        /* posterior and log-density gradients of every row of both sides */
        for (int64_t n = 0; n < N; ++n) {
            row_logit_backward(K, dr, q_bh + n * dr, mu_h, var_h, gq + n * K, dgq + n * K,
                               dqx + bh * N * dr + n * dr, pmu + bh * KD, pvar + bh * KD, plogp + bh * K);
            row_logit_backward(K, dr, k_bh + n * dr, mu_h, var_h, gk + n * K, dgk + n * K,
                               dkx + bh * N * dr + n * dr, pmu + bh * KD, pvar + bh * KD, plogp + bh * K);
        }
        free(gq); free(gk); free(dgq); free(dgk); free(gg); free(hh); free(st); free(z);
    }
    if (rc) goto done;
    /* parameter gradients: partials added over b in order, then the reparameterisations */
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t e = 0; e < KD; ++e) {
            double sm = 0.0, sv = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                sm += pmu[(b * H + h) * KD + e];
                sv += pvar[(b * H + h) * KD + e];
            }
            const double r = raw_var[h * KD + e];
            dmu[h * KD + e] = sm;
            draw_var[h * KD + e] = sv / (1.0 + exp(-r));   /* softplus'(r) = sigmoid(r) */
        }
        double tot = 0.0;
        double* gsum = dprior_logits + h * K;
        for (int k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t b = 0; b < B; ++b) s += plogp[(b * H + h) * K + k];
            gsum[k] = s;
            tot += s;
        }
        for (int k = 0; k < K; ++k) gsum[k] -= exp(logp[h * K + k]) * tot;
    }
done:
    free(var); free(logp); free(logdet); free(pmu); free(pvar); free(plogp);
    return rc;
}
