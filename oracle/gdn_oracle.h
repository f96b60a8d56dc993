/*
 * gdn_oracle.h -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this library: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP kernels against an
 * obviously correct definition.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it follows (pages cited by title and section):
 *  - "Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron" (Hugging Face model
 *    card), section "How It Works": the per-token recurrence
 *      decay the state by exp(log g); read a = S^T k; delta = beta (v - a);
 *      write S += k delta^T; output o = S^T q from the updated state.
 *  - same card, section "Correctness Contract": log g <= 0 in Qwen models
 *    (no clamping is applied here either); each (batch, head) is independent.
 *  - "Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up" (comment on the PR
 *    "Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and vLLM serving
 *    path"), sections "Why This Exists" and "Implementation Details": the
 *    chunked form solves the lower-triangular causal system directly
 *    (forward substitution on the right-hand side) instead of the Neumann
 *    power-doubling series.  Both solves are exposed here so that their
 *    equivalence in exact-ish arithmetic can be pinned.
 *
 * Layouts (all row-major, innermost dimension last, fp64, host memory):
 *   q, k   [B, T, Hk, dk]
 *   v      [B, T, Hv, dv]
 *   log_g  [B, T, Hv]        (natural-log decay, g = exp(log_g))
 *   beta   [B, T, Hv]
 *   h0, hT [B, Hv, dk, dv]   (h0 may be NULL = zero state; hT may be NULL)
 *   o      [B, T, Hv, dv]
 * Value head h reads key head h / (Hv / Hk) (contiguous grouping).
 * q/k normalisation when qk_l2norm != 0:  x / max(||x||_2, 1e-6).
 * Every routine returns 0 on success and a negative number on bad arguments.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Token-serial definition, threaded over independent (b, h) pairs. */
int oracle_gdn_sequential(int B, int T, int Hk, int Hv, int dk, int dv,
                          int qk_l2norm, double q_scale,
                          const double* q, const double* k, const double* v,
                          const double* log_g, const double* beta,
                          const double* h0, double* o, double* hT,
                          int nthreads);

/* Chunk-parallel (WY) form with a direct forward-substitution solve of the
 * unit lower-triangular chunk system.  Must agree with the sequential form
 * up to rounding; used only to pin that equivalence. */
int oracle_gdn_chunked(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                       int qk_l2norm, double q_scale,
                       const double* q, const double* k, const double* v,
                       const double* log_g, const double* beta,
                       const double* h0, double* o, double* hT);

/* (I + A)^-1 for strictly lower-triangular A (n x n, row-major) by forward
 * substitution.  Entries of A on or above the diagonal are ignored. */
int oracle_unit_lower_inverse(int n, const double* A, double* Tinv);

/* The same inverse by Neumann power doubling: prod_j (I + (-A)^(2^j)),
 * j = 0 .. ceil(log2 n) - 1.  Exact in real arithmetic because A is
 * nilpotent; kept only to pin the equivalence the pages rely on. */
int oracle_neumann_inverse(int n, const double* A, double* Tinv);

/* Qwen gates from raw projections ("Qwen3.5 Gated Delta Net NKI Kernel for
 * AWS Neuron", section "Correctness Contract": log g = -exp(A_log)
 * softplus(a + dt_bias)); beta = 1 / (1 + exp(-b)), a reading (the pages do
 * not spell beta out).  a, b, log_g, beta hold n rows of Hv values (value head
 * innermost); A_log, dt_bias hold Hv values. */
int oracle_qwen_gates(long n, int Hv, const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* log_g, double* beta);

/* The operations around the recurrence ("Qwen3.5 Gated Delta Net NKI Kernel
 * for AWS Neuron", section "How It Works": projections, causal conv1d,
 * gating, RMS norm run outside the recurrence kernel; "Add Qwen3.6-27B
 * hybrid DeltaNet/GQA contrib model and vLLM serving path", section
 * "Summary": GDN convolution state checkpoints).  The pages give no
 * formula; these are the plain readings:
 *
 * Causal depthwise conv1d over the channel axis, width K, optional bias,
 * optional SiLU (x / (1 + e^-x)):
 *   y[b,t,c] = act(bias[c] + sum_{j=0}^{K-1} w[c,j] * u[b, t-(K-1)+j, c])
 * where u[b, s, c] = x[b, s, c] for s >= 0 and state_in[b, K-1+s, c] for
 * s < 0 (zeros when state_in is NULL).  The carried state is the last K-1
 * inputs: state_out[b, i, c] = u[b, T-(K-1)+i, c], i = 0 .. K-2 (it may be
 * state_in itself).  Layouts: x, y [B, T, C]; w [C, K]; bias [C] or NULL;
 * states [B, K-1, C]. */
int oracle_causal_conv1d(int B, int T, int C, int K, const double* x, const double* w,
                         const double* bias, const double* state_in, double* state_out,
                         double* y, int silu);

/* Gated RMS norm over the last axis of `rows` rows of D values:
 *   y[r, i] = x[r, i] / sqrt(mean_i(x[r, i]^2) + eps) * w[i] * silu(z[r, i])
 * (z NULL: no gate).  y may be x itself. */
int oracle_gated_rmsnorm(long rows, int D, const double* x, const double* z, const double* w,
                         double eps, double* y);

#ifdef __cplusplus
}
#endif
#endif
