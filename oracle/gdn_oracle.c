/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
 * baseline).  The product path never loads it; it shares no code with the
 * HIP library.  Argument meaning and layouts: gdn_oracle.h.
 *
 * The sequential routine is the definition: the five per-token steps of
 * "Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron", section "How It Works",
 * in their printed order.  Expanding those steps gives
 *     S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 * the form the rest of the pages (and the tests) use.
 *
 * The chunked routine restates the same recurrence chunk by chunk, in the
 * order a chunk-parallel kernel takes it (decay cumsum, decay-masked
 * beta K K^T, direct triangular solve, then the state hand-off), following
 * "Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up", sections "Why This
 * Exists" and "Implementation Details".  No blocking or reordering beyond
 * that is done.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* x / max(||x||_2, 1e-6); identity when the flag is off. */
static void normalise(const double* x, int n, int on, double* out) {
    if (!on) {
        memcpy(out, x, (size_t)n * sizeof(double));
        return;
    }
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double nrm = sqrt(ss);
    if (nrm < 1e-6) nrm = 1e-6;
    for (int i = 0; i < n; ++i) out[i] = x[i] / nrm;
}

static int bad_shape(int B, int T, int Hk, int Hv, int dk, int dv) {
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return 1;
    if (Hv % Hk != 0) return 1;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sequential definition                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    int B, T, Hk, Hv, dk, dv, qk_l2norm;
    double q_scale;
    const double *q, *k, *v, *log_g, *beta, *h0;
    double *o, *hT;
    int first, stride; /* this worker's (b, h) pairs: first, first+stride, ... */
    int status;
} seq_job;

static void* seq_worker(void* arg) {
    seq_job* J = (seq_job*)arg;
    const int dk = J->dk, dv = J->dv, Hk = J->Hk, Hv = J->Hv, T = J->T;
    const int r = Hv / Hk;
    double* S = (double*)malloc((size_t)dk * dv * sizeof(double));
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* a = (double*)malloc((size_t)dv * sizeof(double));
    double* delta = (double*)malloc((size_t)dv * sizeof(double));
    if (!S || !qh || !kh || !a || !delta) {
        J->status = -2;
        free(S); free(qh); free(kh); free(a); free(delta);
        return NULL;
    }
    for (int bh = J->first; bh < J->B * Hv; bh += J->stride) {
        const int b = bh / Hv, h = bh % Hv;
        const int hk = h / r;
        const size_t state_off = ((size_t)b * Hv + h) * dk * dv;
        if (J->h0)
            memcpy(S, J->h0 + state_off, (size_t)dk * dv * sizeof(double));
        else
            memset(S, 0, (size_t)dk * dv * sizeof(double));

        for (int t = 0; t < T; ++t) {
            const size_t qk_off = (((size_t)b * T + t) * Hk + hk) * dk;
            const size_t v_off = (((size_t)b * T + t) * Hv + h) * dv;
            const size_t g_off = ((size_t)b * T + t) * Hv + h;
            normalise(J->q + qk_off, dk, J->qk_l2norm, qh);
            normalise(J->k + qk_off, dk, J->qk_l2norm, kh);
            const double g = exp(J->log_g[g_off]);
            const double bt = J->beta[g_off];

            /* 1. decay */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[i * dv + j] *= g;
            /* 2. read: a = S^T k */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
                a[j] = acc;
            }
            /* 3. delta = beta (v - a) */
            for (int j = 0; j < dv; ++j) delta[j] = bt * (J->v[v_off + j] - a[j]);
            /* 4. write: S += k delta^T */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[i * dv + j] += kh[i] * delta[j];
            /* 5. output from the updated state: o = S^T q */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
                J->o[v_off + j] = J->q_scale * acc;
            }
        }
        if (J->hT) memcpy(J->hT + state_off, S, (size_t)dk * dv * sizeof(double));
    }
    free(S); free(qh); free(kh); free(a); free(delta);
    return NULL;
}

int oracle_gdn_sequential(int B, int T, int Hk, int Hv, int dk, int dv,
                          int qk_l2norm, double q_scale,
                          const double* q, const double* k, const double* v,
                          const double* log_g, const double* beta,
                          const double* h0, double* o, double* hT,
                          int nthreads) {
    if (bad_shape(B, T, Hk, Hv, dk, dv)) return -1;
    if (T > 0 && (!q || !k || !v || !log_g || !beta || !o)) return -1;
    const int pairs = B * Hv;
    if (pairs == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = pairs;

    seq_job* jobs = (seq_job*)calloc((size_t)nthreads, sizeof(seq_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return -2; }
    for (int w = 0; w < nthreads; ++w) {
        seq_job* J = &jobs[w];
        J->B = B; J->T = T; J->Hk = Hk; J->Hv = Hv; J->dk = dk; J->dv = dv;
        J->qk_l2norm = qk_l2norm; J->q_scale = q_scale;
        J->q = q; J->k = k; J->v = v; J->log_g = log_g; J->beta = beta;
        J->h0 = h0; J->o = o; J->hT = hT;
        J->first = w; J->stride = nthreads; J->status = 0;
    }
    int status = 0;
    if (nthreads == 1) {
        seq_worker(&jobs[0]);
    } else {
        int started = 0;
        for (int w = 0; w < nthreads; ++w) {
            if (pthread_create(&tids[w], NULL, seq_worker, &jobs[w]) != 0) {
                status = -3;
                break;
            }
            ++started;
        }
        for (int w = 0; w < started; ++w) pthread_join(tids[w], NULL);
        /* pairs of a worker that failed to start were not computed */
    }
    for (int w = 0; w < nthreads; ++w)
        if (jobs[w].status) status = jobs[w].status;
    free(jobs);
    free(tids);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Triangular inverses                                                      */
/* ------------------------------------------------------------------------ */

int oracle_unit_lower_inverse(int n, const double* A, double* Tinv) {
    if (n < 0 || (n > 0 && (!A || !Tinv))) return -1;
    /* Row i of (I + A) T = I reads T_i + sum_{j<i} A_ij T_j = e_i. */
    for (int i = 0; i < n; ++i) {
        for (int c = 0; c < n; ++c) Tinv[i * n + c] = (c == i) ? 1.0 : 0.0;
        for (int j = 0; j < i; ++j) {
            const double aij = A[i * n + j];
            for (int c = 0; c < n; ++c) Tinv[i * n + c] -= aij * Tinv[j * n + c];
        }
    }
    return 0;
}

static void matmul_sq(int n, const double* X, const double* Y, double* Z) {
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int l = 0; l < n; ++l) acc += X[i * n + l] * Y[l * n + j];
            Z[i * n + j] = acc;
        }
}

int oracle_neumann_inverse(int n, const double* A, double* Tinv) {
    if (n < 0 || (n > 0 && (!A || !Tinv))) return -1;
    if (n == 0) return 0;
    const size_t nn = (size_t)n * n;
    double* P = (double*)malloc(nn * sizeof(double));   /* (-A)^(2^j) */
    double* F = (double*)malloc(nn * sizeof(double));   /* I + P */
    double* R = (double*)malloc(nn * sizeof(double));   /* running product */
    double* tmp = (double*)malloc(nn * sizeof(double));
    if (!P || !F || !R || !tmp) { free(P); free(F); free(R); free(tmp); return -2; }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            P[i * n + j] = (j < i) ? -A[i * n + j] : 0.0;
            R[i * n + j] = (i == j) ? 1.0 : 0.0;
        }
    /* (I + A)^-1 = sum_{m<n} (-A)^m = prod_{j} (I + (-A)^(2^j)) */
    for (int span = 1; span < n; span *= 2) {
        for (size_t e = 0; e < nn; ++e) F[e] = P[e];
        for (int i = 0; i < n; ++i) F[i * n + i] += 1.0;
        matmul_sq(n, R, F, tmp);
        memcpy(R, tmp, nn * sizeof(double));
        matmul_sq(n, P, P, tmp);
        memcpy(P, tmp, nn * sizeof(double));
    }
    memcpy(Tinv, R, nn * sizeof(double));
    free(P); free(F); free(R); free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gates from raw projections                                               */
/* ------------------------------------------------------------------------ */

/* log(1 + e^x) without overflow: for x > 0 it is x + log(1 + e^-x). */
static double softplus(double x) {
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

int oracle_qwen_gates(long n, int Hv, const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* log_g, double* beta) {
    if (n < 0 || Hv <= 0) return -1;
    if (n > 0 && (!a || !b || !A_log || !dt_bias || !log_g || !beta)) return -1;
    for (long i = 0; i < n; ++i)
        for (int h = 0; h < Hv; ++h) {
            const long e = i * Hv + h;
            log_g[e] = -exp(A_log[h]) * softplus(a[e] + dt_bias[h]);
            beta[e] = 1.0 / (1.0 + exp(-b[e]));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Chunked (WY) form with a direct right-hand-side solve                    */
/* ------------------------------------------------------------------------ */

int oracle_gdn_chunked(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                       int qk_l2norm, double q_scale,
                       const double* q, const double* k, const double* v,
                       const double* log_g, const double* beta,
                       const double* h0, double* o, double* hT) {
    if (bad_shape(B, T, Hk, Hv, dk, dv) || chunk <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !log_g || !beta || !o)) return -1;
    const int r = Hv / Hk;
    const int C = chunk;
    double* S = (double*)malloc((size_t)dk * dv * sizeof(double));
    double* Qh = (double*)malloc((size_t)C * dk * sizeof(double));
    double* Kh = (double*)malloc((size_t)C * dk * sizeof(double));
    double* gam = (double*)malloc((size_t)C * sizeof(double));
    double* A = (double*)malloc((size_t)C * C * sizeof(double));
    double* R = (double*)malloc((size_t)C * dv * sizeof(double)); /* rhs -> Delta */
    double* S_next = (double*)malloc((size_t)dk * dv * sizeof(double));
    if (!S || !Qh || !Kh || !gam || !A || !R || !S_next) {
        free(S); free(Qh); free(Kh); free(gam); free(A); free(R); free(S_next);
        return -2;
    }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hv; ++h) {
            const int hk = h / r;
            const size_t state_off = ((size_t)b * Hv + h) * dk * dv;
            if (h0)
                memcpy(S, h0 + state_off, (size_t)dk * dv * sizeof(double));
            else
                memset(S, 0, (size_t)dk * dv * sizeof(double));

            for (int t0 = 0; t0 < T; t0 += C) {
                const int L = (T - t0 < C) ? (T - t0) : C;
                /* normalised q, k rows of this chunk; inclusive log-decay cumsum */
                double run = 0.0;
                for (int s = 0; s < L; ++s) {
                    const size_t qk_off = (((size_t)b * T + t0 + s) * Hk + hk) * dk;
                    normalise(q + qk_off, dk, qk_l2norm, Qh + (size_t)s * dk);
                    normalise(k + qk_off, dk, qk_l2norm, Kh + (size_t)s * dk);
                    run += log_g[((size_t)b * T + t0 + s) * Hv + h];
                    gam[s] = run;
                }
                /* A_rs = beta_r exp(gam_r - gam_s) (k_r . k_s), s < r */
                for (int rr = 0; rr < L; ++rr) {
                    const double br = beta[((size_t)b * T + t0 + rr) * Hv + h];
                    for (int s = 0; s < L; ++s) {
                        double val = 0.0;
                        if (s < rr) {
                            double dot = 0.0;
                            for (int i = 0; i < dk; ++i)
                                dot += Kh[(size_t)rr * dk + i] * Kh[(size_t)s * dk + i];
                            val = br * exp(gam[rr] - gam[s]) * dot;
                        }
                        A[(size_t)rr * C + s] = val;
                    }
                }
                /* rhs_r = beta_r (v_r - exp(gam_r) S^T k_r) */
                for (int rr = 0; rr < L; ++rr) {
                    const size_t gb = ((size_t)b * T + t0 + rr) * Hv + h;
                    const double br = beta[gb];
                    const double Gr = exp(gam[rr]);
                    const size_t v_off = (((size_t)b * T + t0 + rr) * Hv + h) * dv;
                    for (int j = 0; j < dv; ++j) {
                        double read = 0.0;
                        for (int i = 0; i < dk; ++i)
                            read += S[(size_t)i * dv + j] * Kh[(size_t)rr * dk + i];
                        R[(size_t)rr * dv + j] = br * (v[v_off + j] - Gr * read);
                    }
                }
                /* direct solve (I + A) Delta = rhs, forward substitution */
                for (int rr = 0; rr < L; ++rr)
                    for (int s = 0; s < rr; ++s) {
                        const double ars = A[(size_t)rr * C + s];
                        for (int j = 0; j < dv; ++j)
                            R[(size_t)rr * dv + j] -= ars * R[(size_t)s * dv + j];
                    }
                /* o_r = exp(gam_r) S^T q_r + sum_{s<=r} exp(gam_r-gam_s)(q_r.k_s) Delta_s */
                for (int rr = 0; rr < L; ++rr) {
                    const double Gr = exp(gam[rr]);
                    const size_t o_off = (((size_t)b * T + t0 + rr) * Hv + h) * dv;
                    for (int j = 0; j < dv; ++j) {
                        double acc = 0.0;
                        for (int i = 0; i < dk; ++i)
                            acc += S[(size_t)i * dv + j] * Qh[(size_t)rr * dk + i];
                        acc *= Gr;
                        for (int s = 0; s <= rr; ++s) {
                            double dot = 0.0;
                            for (int i = 0; i < dk; ++i)
                                dot += Qh[(size_t)rr * dk + i] * Kh[(size_t)s * dk + i];
                            acc += exp(gam[rr] - gam[s]) * dot * R[(size_t)s * dv + j];
                        }
                        o[o_off + j] = q_scale * acc;
                    }
                }
                /* S <- exp(gam_L) S + sum_s exp(gam_L - gam_s) k_s Delta_s^T */
                const double GL = exp(gam[L - 1]);
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) {
                        double acc = GL * S[(size_t)i * dv + j];
                        for (int s = 0; s < L; ++s)
                            acc += exp(gam[L - 1] - gam[s]) * Kh[(size_t)s * dk + i] *
                                   R[(size_t)s * dv + j];
                        S_next[(size_t)i * dv + j] = acc;
                    }
                memcpy(S, S_next, (size_t)dk * dv * sizeof(double));
            }
            if (hT) memcpy(hT + state_off, S, (size_t)dk * dv * sizeof(double));
        }
    free(S); free(Qh); free(Kh); free(gam); free(A); free(R); free(S_next);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Causal conv1d and gated RMS norm (the operations around the recurrence)  */
/* ------------------------------------------------------------------------ */

static double silu(double x) { return x / (1.0 + exp(-x)); }

int oracle_causal_conv1d(int B, int T, int C, int K, const double* x, const double* w,
                         const double* bias, const double* state_in, double* state_out,
                         double* y, int silu_on) {
    if (B < 0 || T < 0 || C <= 0 || K < 1) return -1;
    if ((long)B * T > 0 && (!x || !y)) return -1;
    if (!w) return -1;
    const int P = K - 1;                 /* inputs carried between calls */
    /* the whole input of one sequence with its carried prefix: u[s + P], s = -P .. T-1 */
    double* u = (double*)malloc(sizeof(double) * (size_t)(T + P) * (size_t)C);
    if (!u) return -2;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < P; ++i)
            for (int c = 0; c < C; ++c)
                u[(size_t)i * C + c] = state_in ? state_in[((size_t)b * P + i) * C + c] : 0.0;
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c)
                u[(size_t)(t + P) * C + c] = x[((size_t)b * T + t) * C + c];
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) {
                double acc = bias ? bias[c] : 0.0;
                for (int j = 0; j < K; ++j) acc += w[(size_t)c * K + j] * u[(size_t)(t + j) * C + c];
                y[((size_t)b * T + t) * C + c] = silu_on ? silu(acc) : acc;
            }
        if (state_out)
            for (int i = 0; i < P; ++i)
                for (int c = 0; c < C; ++c)
                    state_out[((size_t)b * P + i) * C + c] = u[(size_t)(T + i) * C + c];
    }
    free(u);
    return 0;
}

int oracle_gated_rmsnorm(long rows, int D, const double* x, const double* z, const double* w,
                         double eps, double* y) {
    if (rows < 0 || D <= 0 || eps < 0.0) return -1;
    if (rows > 0 && (!x || !w || !y)) return -1;
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int i = 0; i < D; ++i) ss += x[r * D + i] * x[r * D + i];
        const double inv = 1.0 / sqrt(ss / D + eps);
        for (int i = 0; i < D; ++i) {
            const double g = z ? silu(z[r * D + i]) : 1.0;
            y[r * D + i] = x[r * D + i] * inv * w[i] * g;
        }
    }
    return 0;
}
