/*
 * lrs_oracle.c -- plain sequential fp64 oracle for the seven RL
 * credit-assignment estimators.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * Also the generic segmented affine scan those estimators reduce to.
 *
 * Sources (cited by title and section; no other text is relied on):
 *   [P1] "rl-triton: High-Performance Triton GPU Kernels for Reinforcement
 *        Learning Credit Assignment", gist.science summary page, Technical
 *        Summary: Problem Statement; Methodology 1 (Unified Algebraic
 *        Framework) and 3 (Explicit Boundary Semantics).
 *   [P2] the same paper's abstract (arXiv 2608.17641v1 digest page).
 *   [P3] rl-triton GitHub README: Kernels table and Usage section.
 * Standard definitions named by [P3]'s Kernels table:
 *   GAE      -- Schulman et al. 2016, "High-Dimensional Continuous Control
 *               Using Generalized Advantage Estimation", eq. (16) (recursive).
 *   V-trace  -- Espeholt et al. 2018, "IMPALA", sec. 4.1, eq. (1), with the
 *               lambda-weighted trace c_i = lambda*min(cbar, pi/mu) of sec. 4.2.
 *   Retrace  -- Munos et al. 2016, "Safe and Efficient Off-Policy
 *               Reinforcement Learning", eq. (3)/(4), c_s = lambda*min(cbar, pi/mu).
 *   TD(l)    -- Sutton & Barto 2018, sec. 12.1, recursive lambda-return.
 *
 * Conventions (the readings that the pages leave open; see the design notes):
 *   * Arrays are [N, T] row-major (row = environment, column = time step),
 *     exactly the fp32 / uint8 / int32 buffers the GPU reads; every float is
 *     widened to double before use.  Outputs are double (int32 for the
 *     integer prefix sum).
 *   * Masks are uint8, nonzero = true.  term = terminated (tau), trunc =
 *     truncated (kappa), done = d for the two forward estimators.
 *   * Successor value at step t, [P1] Methodology 3:
 *       tau_t            -> 0                         (natural episode end)
 *       else kappa_t     -> trunc_val[t]              (supplied bootstrap)
 *       else t == T-1    -> boot[n] (0 if boot NULL)  (rollout-window end)
 *       else             -> values[t+1]
 *     The window bootstrap enters the local term at t = T-1 only, never also
 *     as a carry, so it is counted once.
 *   * end_t = tau_t or kappa_t or (t == T-1): the backward recursion does not
 *     continue past end_t.
 *   * Forward estimators reset at step t when t == 0 or done[t-1] ([P3]
 *     Kernels table, eligibility-trace formula).
 *   * The integer prefix sum accumulates in int64 and stores the low 32 bits
 *     (two's-complement wrap), i.e. the exact sum whenever it fits in int32.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC lrs_oracle.c -o liblrs_oracle.so
 * Rows are independent, so an OpenMP loop runs over environments; the
 * recursion along time inside each row is the plain sequential one.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>

#define IDX(n, t) ((size_t)(n) * (size_t)T + (size_t)(t))

/* Successor value of step t in row n ([P1] Methodology 3).  `values` may be
 * NULL for estimators that never read values[t+1] (discounted returns). */
static double successor_value(int64_t n, int64_t t, int64_t T,
                              const float* values, const uint8_t* term,
                              const uint8_t* trunc, const float* trunc_val,
                              const float* boot)
{
    size_t i = IDX(n, t);
    if (term[i]) return 0.0;
    if (trunc && trunc[i]) return (double)trunc_val[i];
    if (t == T - 1) return boot ? (double)boot[n] : 0.0;
    return values ? (double)values[i + 1] : 0.0;
}

static int is_end(int64_t n, int64_t t, int64_t T,
                  const uint8_t* term, const uint8_t* trunc)
{
    size_t i = IDX(n, t);
    return term[i] || (trunc && trunc[i]) || t == T - 1;
}

/* GAE ([P3] Kernels table: backward scan over delta + gamma*lambda*A;
 * Schulman et al. 2016 eq. 16):
 *   delta_t = r_t + gamma*Vnext_t - V_t
 *   A_t     = delta_t + (end_t ? 0 : gamma*lambda*A_{t+1})                   */
void lrs_oracle_gae(int64_t N, int64_t T, const float* rewards,
                    const float* values, const uint8_t* term,
                    const uint8_t* trunc, const float* trunc_val,
                    const float* boot, double gamma, double lambda,
                    double* adv)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double next_a = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = IDX(n, t);
            double vn = successor_value(n, t, T, values, term, trunc, trunc_val, boot);
            double delta = (double)rewards[i] + gamma * vn - (double)values[i];
            double a = delta;
            if (!is_end(n, t, T, term, trunc)) a += gamma * lambda * next_a;
            adv[i] = a;
            next_a = a;
        }
    }
}

/* TD(lambda) returns ([P3] Kernels table: lambda-return mixing one-step TD
 * and Monte Carlo; Sutton & Barto sec. 12.1, recursive form):
 *   G_t = r_t + gamma * (end_t ? Vnext_t
 *                              : (1-lambda)*V_{t+1} + lambda*G_{t+1})        */
void lrs_oracle_lambda_returns(int64_t N, int64_t T, const float* rewards,
                               const float* values, const uint8_t* term,
                               const uint8_t* trunc, const float* trunc_val,
                               const float* boot, double gamma, double lambda,
                               double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double next_g = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = IDX(n, t);
            double g;
            if (is_end(n, t, T, term, trunc)) {
                double vn = successor_value(n, t, T, values, term, trunc, trunc_val, boot);
                g = (double)rewards[i] + gamma * vn;
            } else {
                double v1 = (double)values[i + 1];
                g = (double)rewards[i] + gamma * ((1.0 - lambda) * v1 + lambda * next_g);
            }
            out[i] = g;
            next_g = g;
        }
    }
}

/* Discounted returns ([P3] Kernels table: discounted reward-to-go):
 *   G_t = r_t + gamma * (end_t ? Vnext_t : G_{t+1})
 * Vnext here never reads values[] (0 at tau, trunc_val at kappa, boot at the
 * window end).                                                              */
void lrs_oracle_discounted_returns(int64_t N, int64_t T, const float* rewards,
                                   const uint8_t* term, const uint8_t* trunc,
                                   const float* trunc_val, const float* boot,
                                   double gamma, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double next_g = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = IDX(n, t);
            double g;
            if (is_end(n, t, T, term, trunc))
                g = (double)rewards[i]
                    + gamma * successor_value(n, t, T, NULL, term, trunc, trunc_val, boot);
            else
                g = (double)rewards[i] + gamma * next_g;
            out[i] = g;
            next_g = g;
        }
    }
}

/* V-trace ([P3] Kernels table: IS-weighted targets and advantages; Espeholt
 * et al. 2018 sec. 4.1 eq. (1), lambda-trace of sec. 4.2).  With
 * w_t = exp(log_rho_t) = pi/mu at step t:
 *   rho_t = min(rho_bar, w_t),  c_t = lambda * min(c_bar, w_t)
 *   A_t   = rho_t*(r_t + gamma*Vnext_t - V_t) + (end_t ? 0 : gamma*c_t*A_{t+1})
 *   vs_t  = V_t + A_t
 *   pg_t  = min(pg_rho_bar, w_t) * (r_t + gamma*(end_t ? Vnext_t : vs_{t+1}) - V_t)
 * Passing +INFINITY for a clip threshold means no clipping.                 */
void lrs_oracle_vtrace(int64_t N, int64_t T, const float* log_rhos,
                       const float* rewards, const float* values,
                       const uint8_t* term, const uint8_t* trunc,
                       const float* trunc_val, const float* boot,
                       double gamma, double lambda, double rho_bar,
                       double c_bar, double pg_rho_bar,
                       double* vs, double* pg_adv)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double next_a = 0.0;   /* A_{t+1} = vs_{t+1} - V_{t+1} */
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = IDX(n, t);
            double w = exp((double)log_rhos[i]);
            double rho = fmin(rho_bar, w);
            double c = lambda * fmin(c_bar, w);
            double rho_pg = fmin(pg_rho_bar, w);
            double r = (double)rewards[i], v = (double)values[i];
            double vn = successor_value(n, t, T, values, term, trunc, trunc_val, boot);
            int end = is_end(n, t, T, term, trunc);
            double a = rho * (r + gamma * vn - v);
            double target_next;
            if (end) {
                target_next = vn;
            } else {
                a += gamma * c * next_a;
                target_next = (double)values[i + 1] + next_a;   /* vs_{t+1} */
            }
            vs[i] = v + a;
            pg_adv[i] = rho_pg * (r + gamma * target_next - v);
            next_a = a;
        }
    }
}

/* Retrace(lambda) ([P3] Kernels table: off-policy return with truncated IS
 * ratios; Munos et al. 2016).  q = Q(s_t, a_t); values = E_pi Q(s_t, .);
 * the trace uses the ratio of the NEXT step, c_{t+1} = lambda*min(c_bar, w_{t+1}):
 *   G_t = r_t + gamma * (end_t ? Vnext_t
 *                              : V_{t+1} + c_{t+1}*(G_{t+1} - Q_{t+1}))       */
void lrs_oracle_retrace(int64_t N, int64_t T, const float* log_rhos,
                        const float* rewards, const float* q_values,
                        const float* values, const uint8_t* term,
                        const uint8_t* trunc, const float* trunc_val,
                        const float* boot, double gamma, double lambda,
                        double c_bar, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double next_g = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            size_t i = IDX(n, t);
            double g;
            if (is_end(n, t, T, term, trunc)) {
                double vn = successor_value(n, t, T, values, term, trunc, trunc_val, boot);
                g = (double)rewards[i] + gamma * vn;
            } else {
                double c1 = lambda * fmin(c_bar, exp((double)log_rhos[i + 1]));
                g = (double)rewards[i]
                    + gamma * ((double)values[i + 1]
                               + c1 * (next_g - (double)q_values[i + 1]));
            }
            out[i] = g;
            next_g = g;
        }
    }
}

/* Eligibility traces, forward in time ([P3] Kernels table formula):
 *   e_t = x_t + (t == 0 or d_{t-1} ? 0 : gamma*lambda*e_{t-1})               */
void lrs_oracle_eligibility_traces(int64_t N, int64_t T, const float* x,
                                   const uint8_t* done, double gamma,
                                   double lambda, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double prev = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            size_t i = IDX(n, t);
            double e = (double)x[i];
            if (t > 0 && !done[i - 1]) e += gamma * lambda * prev;
            out[i] = e;
            prev = e;
        }
    }
}

/* Episodic prefix sum, inclusive, forward ([P3] Kernels table: cumulative
 * sum with done-mask resets; same reset rule as the traces):
 *   S_t = x_t + (t == 0 or d_{t-1} ? 0 : S_{t-1})                            */
void lrs_oracle_prefix_sum_f32(int64_t N, int64_t T, const float* x,
                               const uint8_t* done, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            size_t i = IDX(n, t);
            if (t == 0 || done[i - 1]) s = 0.0;
            s += (double)x[i];
            out[i] = s;
        }
    }
}

/* Integer variant: exact int64 accumulation, stored modulo 2^32. */
void lrs_oracle_prefix_sum_i32(int64_t N, int64_t T, const int32_t* x,
                               const uint8_t* done, int32_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int64_t s = 0;
        for (int64_t t = 0; t < T; ++t) {
            size_t i = IDX(n, t);
            if (t == 0 || done[i - 1]) s = 0;
            s += (int64_t)x[i];
            out[i] = (int32_t)(uint32_t)(uint64_t)s;
        }
    }
}

/* Generic segmented first-order linear recurrence, the operator all seven
 * estimators reduce to ([P1] Methodology 1, Unified Algebraic Framework; the
 * same page's Significance and Claims section names other segmented affine
 * recurrences as further users).  Scan order runs along t (reverse = 0) or
 * against it (reverse = 1); "previous" means the neighbour earlier in scan
 * order:
 *   reverse = 0:  y_t = alpha_t + beta_t * y_{t-1}
 *   reverse = 1:  y_t = alpha_t + beta_t * y_{t+1}
 * The step before the first one in scan order is carry[n] (0 if carry is
 * NULL).  Where reset[t] is nonzero (reset may be NULL), y_t = alpha_t: the
 * recursion does not read the previous step, as if beta_t were 0.           */
void lrs_oracle_affine_scan(int64_t N, int64_t T, const float* alpha,
                            const float* beta, const uint8_t* reset,
                            const float* carry, int reverse, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double y = carry ? (double)carry[n] : 0.0;
        for (int64_t k = 0; k < T; ++k) {
            int64_t t = reverse ? T - 1 - k : k;
            size_t i = IDX(n, t);
            double next = (double)alpha[i];
            if (!(reset && reset[i])) next += (double)beta[i] * y;
            out[i] = next;
            y = next;
        }
    }
}

/* Number of OpenMP threads a parallel region would use (0 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int lrs_oracle_threads(void) { return omp_get_max_threads(); }
#else
int lrs_oracle_threads(void) { return 1; }
#endif
