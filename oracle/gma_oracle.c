/*
 * GMA oracle: plain fp64 CPU implementation of the Gaussian Mixture Attention
 * forward pass, written from "Gaussian Mixture Attention: Linear-Time Sequence
 * Mixing via Probabilistic Latent Routing" (Huang & Raza).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the HIP implementation, and the HIP implementation never calls it.
 *
 * Everything is double precision, plain loops, no blocking and no reordering
 * beyond what the equations state.  Parallelism is an OpenMP loop over the
 * independent (batch, head) pairs (Sec. 3, "applies the same computation
 * independently across heads"), so results do not depend on the thread count.
 *
 * Layout (all contiguous, row-major):
 *   X, XQ, XK : [B, H, N, d_r]      routing vectors (query or key projections, Eq. 4)
 *   V         : [B, H, N, d_v]      value projections (Eq. 4)
 *   mu, sigma2: [H, K, d_r]         per-head diagonal Gaussian components (Sec. 3.2),
 *                                   shared by queries and keys (Fig. 1)
 *   pi        : [H, K]              mixture priors, positive, summing to one (Sec. 3.2)
 *   S, Gamma  : [B, H, N, K]        scores / responsibilities
 *   O         : [B, H, N, d_v]      output (Eq. 7-8, or Eq. 8b for the causal variant)
 *
 * Return value: 0 on success, -1 on a bad argument (null pointer, negative size),
 * -2 if a work buffer cannot be allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* log(2*pi) written out; only used for the k-independent constant of Eq. 16. */
static const double LOG_2PI = 1.83787706640934548356065947281;

/*
 * Log-density score of Sec. 4.1, Eq. 16, for one routing vector x against all K
 * components of one head:
 *   s_k = log pi_k - (d_r/2) log(2 pi) - (1/2) log|Sigma_k|
 *         - (1/2) (x - mu_k)^T Sigma_k^{-1} (x - mu_k)
 * with Sigma_k = diag(sigma2_k) (Sec. 3.2), so log|Sigma_k| = sum_d log sigma2_kd
 * and the quadratic form is sum_d (x_d - mu_kd)^2 / sigma2_kd.
 * This is log(pi_k N(x | mu_k, Sigma_k)) with the density of Eq. 2.
 */
static void log_scores_one(const double* x, int64_t dr, const double* mu_h,
                           const double* s2_h, const double* pi_h, int64_t K,
                           double* s) {
    for (int64_t k = 0; k < K; ++k) {
        const double* mu_k = mu_h + k * dr;
        const double* s2_k = s2_h + k * dr;
        double logdet = 0.0, maha = 0.0;
        for (int64_t d = 0; d < dr; ++d) {
            double diff = x[d] - mu_k[d];
            maha += diff * diff / s2_k[d];
            logdet += log(s2_k[d]);
        }
        s[k] = log(pi_h[k]) - 0.5 * (double)dr * LOG_2PI - 0.5 * logdet - 0.5 * maha;
    }
}

/*
 * Responsibilities of Eq. 3 in the softmax form of Eq. 3b: gamma_k = exp(s_k) /
 * sum_l exp(s_l).  The largest score is subtracted before exponentiating; this
 * multiplies numerator and denominator by the same factor and leaves Eq. 3b
 * unchanged while keeping exp() in range.
 */
static void responsibilities_one(const double* x, int64_t dr, const double* mu_h,
                                 const double* s2_h, const double* pi_h, int64_t K,
                                 double* s_scratch, double* gamma) {
    log_scores_one(x, dr, mu_h, s2_h, pi_h, K, s_scratch);
    double m = s_scratch[0];
    for (int64_t k = 1; k < K; ++k)
        if (s_scratch[k] > m) m = s_scratch[k];
    double total = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        gamma[k] = exp(s_scratch[k] - m);
        total += gamma[k];
    }
    for (int64_t k = 0; k < K; ++k) gamma[k] /= total;
}

static int bad_sizes(int64_t B, int64_t H, int64_t N, int64_t dr, int64_t K) {
    return B < 0 || H < 0 || N < 0 || dr < 1 || K < 1;
}

/* S[b,h,n,:] = Eq. 16 scores.  Exposed so tests can compare against a library
 * log-density routine. */
int oracle_log_scores(const double* X, int64_t B, int64_t H, int64_t N, int64_t dr,
                      const double* mu, const double* sigma2, const double* pi,
                      int64_t K, double* S) {
    if (!X || !mu || !sigma2 || !pi || !S || bad_sizes(B, H, N, dr, K)) return -1;
    int64_t P = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < P; ++p) {
        int64_t h = p % H;
        for (int64_t n = 0; n < N; ++n)
            log_scores_one(X + (p * N + n) * dr, dr, mu + h * K * dr, sigma2 + h * K * dr,
                           pi + h * K, K, S + (p * N + n) * K);
    }
    return 0;
}

/* Gamma[b,h,n,:] = Eq. 3 / 3b responsibilities of every routing vector. */
int oracle_responsibilities(const double* X, int64_t B, int64_t H, int64_t N, int64_t dr,
                            const double* mu, const double* sigma2, const double* pi,
                            int64_t K, double* Gamma) {
    if (!X || !mu || !sigma2 || !pi || !Gamma || bad_sizes(B, H, N, dr, K)) return -1;
    int64_t P = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t p = 0; p < P; ++p) {
        int64_t h = p % H;
        double* s = (double*)malloc((size_t)K * sizeof(double));
        if (!s) { failed = 1; continue; }
        for (int64_t n = 0; n < N; ++n)
            responsibilities_one(X + (p * N + n) * dr, dr, mu + h * K * dr,
                                 sigma2 + h * K * dr, pi + h * K, K, s,
                                 Gamma + (p * N + n) * K);
        free(s);
    }
    return failed ? -2 : 0;
}

/*
 * Bidirectional GMA (Sec. 3.3).
 *   Latent aggregation, Eq. 5-6:  Vt_k = sum_j gammaK_jk V_j,   Z_k = sum_j gammaK_jk
 *   Normalised broadcasting, Eq. 7-8:
 *        O_i = sum_k gammaQ_ik Vt_k / (sum_k gammaQ_ik Z_k + eps)
 * eps is added once to the row denominator (footnote 4 of Sec. 3.3).
 */
int oracle_forward_bidir(const double* XQ, const double* XK, const double* V,
                         int64_t B, int64_t H, int64_t N, int64_t dr, int64_t dv, int64_t K,
                         const double* mu, const double* sigma2, const double* pi,
                         double eps, double* O) {
    if (!XQ || !XK || !V || !mu || !sigma2 || !pi || !O || dv < 1 ||
        bad_sizes(B, H, N, dr, K))
        return -1;
    int64_t P = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t p = 0; p < P; ++p) {
        int64_t h = p % H;
        const double* mu_h = mu + h * K * dr;
        const double* s2_h = sigma2 + h * K * dr;
        const double* pi_h = pi + h * K;
        double* s = (double*)malloc((size_t)K * sizeof(double));
        double* g = (double*)malloc((size_t)K * sizeof(double));
        double* Vt = (double*)calloc((size_t)(K * dv), sizeof(double));
        double* Z = (double*)calloc((size_t)K, sizeof(double));
        if (!s || !g || !Vt || !Z) {
            failed = 1;
        } else {
            /* write: Eq. 6 */
            for (int64_t j = 0; j < N; ++j) {
                responsibilities_one(XK + (p * N + j) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                const double* vj = V + (p * N + j) * dv;
                for (int64_t k = 0; k < K; ++k) {
                    for (int64_t c = 0; c < dv; ++c) Vt[k * dv + c] += g[k] * vj[c];
                    Z[k] += g[k];
                }
            }
            /* read: Eq. 8 */
            for (int64_t i = 0; i < N; ++i) {
                responsibilities_one(XQ + (p * N + i) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                double den = 0.0;
                for (int64_t k = 0; k < K; ++k) den += g[k] * Z[k];
                den += eps;
                double* oi = O + (p * N + i) * dv;
                for (int64_t c = 0; c < dv; ++c) {
                    double num = 0.0;
                    for (int64_t k = 0; k < K; ++k) num += g[k] * Vt[k * dv + c];
                    oi[c] = num / den;
                }
            }
        }
        free(s); free(g); free(Vt); free(Z);
    }
    return failed ? -2 : 0;
}

/*
 * Cross-attention GMA (Sec. 3, "Cross-attention"): queries come from a query-side
 * sequence X of length Nq, keys and values from a separate context sequence Y of
 * length Nk, and the routing of Sec. 3.3 is applied with Gamma^Q_X and Gamma^K_Y.
 *   Latent aggregation over the context, Eq. 5-6:  Vt_k = sum_j gammaK_jk V_j,  Z_k = sum_j gammaK_jk
 *   Normalised broadcasting to the queries, Eq. 7-8:
 *        O_i = sum_k gammaQ_ik Vt_k / (sum_k gammaQ_ik Z_k + eps)
 * Layout: XQ [B,H,Nq,d_r], XK [B,H,Nk,d_r], V [B,H,Nk,d_v], O [B,H,Nq,d_v].  An empty
 * context (Nk = 0) leaves Vt = 0 and Z = 0, so every output is 0 / eps = 0.
 */
int oracle_forward_cross(const double* XQ, int64_t Nq, const double* XK, const double* V, int64_t Nk,
                         int64_t B, int64_t H, int64_t dr, int64_t dv, int64_t K,
                         const double* mu, const double* sigma2, const double* pi,
                         double eps, double* O) {
    if (!XQ || !XK || !V || !mu || !sigma2 || !pi || !O || dv < 1 || Nk < 0 ||
        bad_sizes(B, H, Nq, dr, K))
        return -1;
    int64_t P = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t p = 0; p < P; ++p) {
        int64_t h = p % H;
        const double* mu_h = mu + h * K * dr;
        const double* s2_h = sigma2 + h * K * dr;
        const double* pi_h = pi + h * K;
        double* s = (double*)malloc((size_t)K * sizeof(double));
        double* g = (double*)malloc((size_t)K * sizeof(double));
        double* Vt = (double*)calloc((size_t)(K * dv), sizeof(double));
        double* Z = (double*)calloc((size_t)K, sizeof(double));
        if (!s || !g || !Vt || !Z) {
            failed = 1;
        } else {
            /* write: Eq. 6 over the context positions */
            for (int64_t j = 0; j < Nk; ++j) {
                responsibilities_one(XK + (p * Nk + j) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                const double* vj = V + (p * Nk + j) * dv;
                for (int64_t k = 0; k < K; ++k) {
                    for (int64_t c = 0; c < dv; ++c) Vt[k * dv + c] += g[k] * vj[c];
                    Z[k] += g[k];
                }
            }
            /* read: Eq. 8 for every query position */
            for (int64_t i = 0; i < Nq; ++i) {
                responsibilities_one(XQ + (p * Nq + i) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                double den = 0.0;
                for (int64_t k = 0; k < K; ++k) den += g[k] * Z[k];
                den += eps;
                double* oi = O + (p * Nq + i) * dv;
                for (int64_t c = 0; c < dv; ++c) {
                    double num = 0.0;
                    for (int64_t k = 0; k < K; ++k) num += g[k] * Vt[k * dv + c];
                    oi[c] = num / den;
                }
            }
        }
        free(s); free(g); free(Vt); free(Z);
    }
    return failed ? -2 : 0;
}

/*
 * Causal GMA (Sec. 3.5).
 *   Prefix memory, Eq. 6b:  Vt^(i)_k = sum_{j<=i} gammaK_jk V_j,  Z^(i)_k = sum_{j<=i} gammaK_jk
 *   Output, Eq. 8b:         O_i = sum_k gammaQ_ik Vt^(i)_k / (sum_k gammaQ_ik Z^(i)_k + eps)
 * The prefix sums are kept as a running sum along the sequence (the cumulative-sum
 * reading given at the end of Sec. 3.5); position i is included before O_i is read.
 *
 * Carried memory: the running sum is Eq. 6b as a recurrence (memory after i = memory
 * after i-1 + gammaK_i [V_i | 1]), so a sequence may be continued from the memory of the
 * positions before it.  state_in [B,H,K,d_v+1] (row k: Vt_k then Z_k) is that starting
 * memory (NULL: empty); state_out receives the memory after the last position (NULL: not
 * wanted).
 */
int oracle_forward_causal_state(const double* XQ, const double* XK, const double* V,
                                int64_t B, int64_t H, int64_t N, int64_t dr, int64_t dv, int64_t K,
                                const double* mu, const double* sigma2, const double* pi,
                                double eps, const double* state_in, double* O, double* state_out) {
    if (!XQ || !XK || !V || !mu || !sigma2 || !pi || !O || dv < 1 ||
        bad_sizes(B, H, N, dr, K))
        return -1;
    int64_t P = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t p = 0; p < P; ++p) {
        int64_t h = p % H;
        const double* mu_h = mu + h * K * dr;
        const double* s2_h = sigma2 + h * K * dr;
        const double* pi_h = pi + h * K;
        double* s = (double*)malloc((size_t)K * sizeof(double));
        double* g = (double*)malloc((size_t)K * sizeof(double));
        double* Vt = (double*)calloc((size_t)(K * dv), sizeof(double));
        double* Z = (double*)calloc((size_t)K, sizeof(double));
        if (!s || !g || !Vt || !Z) {
            failed = 1;
        } else {
            if (state_in) {
                const double* st = state_in + p * K * (dv + 1);
                for (int64_t k = 0; k < K; ++k) {
                    for (int64_t c = 0; c < dv; ++c) Vt[k * dv + c] = st[k * (dv + 1) + c];
                    Z[k] = st[k * (dv + 1) + dv];
                }
            }
            for (int64_t i = 0; i < N; ++i) {
                /* add token i to the prefix memory (j <= i is inclusive) */
                responsibilities_one(XK + (p * N + i) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                const double* vi = V + (p * N + i) * dv;
                for (int64_t k = 0; k < K; ++k) {
                    for (int64_t c = 0; c < dv; ++c) Vt[k * dv + c] += g[k] * vi[c];
                    Z[k] += g[k];
                }
                /* read position i from its prefix-restricted memory */
                responsibilities_one(XQ + (p * N + i) * dr, dr, mu_h, s2_h, pi_h, K, s, g);
                double den = 0.0;
                for (int64_t k = 0; k < K; ++k) den += g[k] * Z[k];
                den += eps;
                double* oi = O + (p * N + i) * dv;
                for (int64_t c = 0; c < dv; ++c) {
                    double num = 0.0;
                    for (int64_t k = 0; k < K; ++k) num += g[k] * Vt[k * dv + c];
                    oi[c] = num / den;
                }
            }
            if (state_out) {
                double* st = state_out + p * K * (dv + 1);
                for (int64_t k = 0; k < K; ++k) {
                    for (int64_t c = 0; c < dv; ++c) st[k * (dv + 1) + c] = Vt[k * dv + c];
                    st[k * (dv + 1) + dv] = Z[k];
                }
            }
        }
        free(s); free(g); free(Vt); free(Z);
    }
    return failed ? -2 : 0;
}

/* Causal GMA from an empty memory. */
int oracle_forward_causal(const double* XQ, const double* XK, const double* V,
                          int64_t B, int64_t H, int64_t N, int64_t dr, int64_t dv, int64_t K,
                          const double* mu, const double* sigma2, const double* pi,
                          double eps, double* O) {
    return oracle_forward_causal_state(XQ, XK, V, B, H, N, dr, dv, K, mu, sigma2, pi, eps, NULL, O, NULL);
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of threads the parallel loops above will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops above from now on (n >= 1; ignored without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
