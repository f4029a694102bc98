/*
 * sk_oracle.c -- plain CPU float64 reference for dense log-domain Sinkhorn
 * between point clouds under squared-Euclidean cost.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the solver library never calls it and
 * shares no code, header, table or helper with it.
 *
 * Everything is written the slow, obvious way: the cost is the difference form
 * C_ij = sum_t (x_it - y_jt)^2, every log-sum-exp is a max pass followed by a
 * sum pass with natural exp/log, and there is no tiling, no expanded form, no
 * centring and no base-2 arithmetic.  OpenMP only splits independent rows (or
 * columns) across threads; each row's reduction runs sequentially in index
 * order, so results do not depend on the thread count.
 *
 * Inputs are float64 arrays (the Python wrapper promotes the float32 problem
 * exactly).  Weights are used as given: log 0 = -inf, and such a point adds
 * nothing to any sum.
 *
 * Sources (the pages, by title and section):
 *  - "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (technical
 *    summary), Methodology 1: the stabilised log-domain update
 *    f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j]; the g update is its
 *    transpose with f and log a.  Methodology 2: the LSE is an exact running
 *    max / sum-exp statistic (an exact reduction, not an approximation).
 *    Methodology 3: the gradient is a barycentric (weighted-average)
 *    projection through the transport plan, no backprop through iterations.
 *  - SinkSLOT README, Tensor Contract: C_ij = |x_i - y_j|^2 sets the scale of
 *    eps; weights are nonnegative, used exactly as given, zeros are legal.
 *  - SinkSLOT README, API Reference: variant "alternating" (Gauss-Seidel:
 *    each half-step uses the other potential's newest value), stop_mode
 *    "fixed" (exactly n_iters), and the "marginal" residual: the infinity
 *    norm of (P1 - a, P^T 1 - b).  The same section's "symmetric" (Jacobi)
 *    variant with blend alpha, the "marginal" and "potential" stop modes with
 *    their iteration cap, tolerance and check interval; Low-Level Solver API
 *    for iters_run, converged and final_viol.
 *  - SinkSLOT README, opening section: entropic OT is not zero at (x, x), so
 *    a divergence built from it subtracts the two self-terms.
 *  - SinkSLOT README, Gradient Flow: plain descent x <- x - lr * grad on the
 *    analytic gradient, with a fresh solve at every step.
 * Readings where the pages are silent: g starts at 0 and each iteration is an
 * f half-step followed by a g half-step; the cost is the entropic dual
 * objective D(f,g) = <a,f> + <b,g> - eps * sum_ij a_i b_j (e^{(f_i+g_j-C_ij)/eps} - 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Squared Euclidean distance, difference form. */
static double sq_dist(const double *p, const double *q, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) {
        double diff = p[t] - q[t];
        s += diff * diff;
    }
    return s;
}

/* log of a weight, with log 0 = -inf. */
static double log_weight(double w)
{
    return w > 0.0 ? log(w) : -INFINITY;
}

/*
 * One half-step (c-transform) for a single query point p:
 *   out = -eps * log sum_j exp((pot_j - C(p, key_j)) / eps + logw_j)
 * computed as -eps * (M + log sum_j exp(z_j - M)), M = max_j z_j.
 * Returns +inf when every key has zero weight.
 */
static double c_transform_one(const double *p, const double *key, int64_t nk, int d,
                              const double *logw, const double *pot, double eps)
{
    double zmax = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        double z = (pot[j] - sq_dist(p, key + j * d, d)) / eps + logw[j];
        if (z > zmax)
            zmax = z;
    }
    if (zmax == -INFINITY)
        return INFINITY;
    double s = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        double z = (pot[j] - sq_dist(p, key + j * d, d)) / eps + logw[j];
        s += exp(z - zmax);
    }
    return -eps * (zmax + log(s));
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Half-step over a set of query points.  out[r] is the c-transform for query
 * idx[r] (or query r when idx == NULL, with nidx = nq).
 * Row half-step:    (qry, key, logw, pot) = (x, y, log b, g) -> f
 * Column half-step: (qry, key, logw, pot) = (y, x, log a, f) -> g
 */
void oracle_half_step(const double *qry, int64_t nq, const double *key, int64_t nk, int d,
                      const double *w_key, const double *pot_key, double eps,
                      const int64_t *idx, int64_t nidx, double *out)
{
    double *logw = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    for (int64_t j = 0; j < nk; ++j)
        logw[j] = log_weight(w_key[j]);
    int64_t cnt = idx ? nidx : nq;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cnt; ++r) {
        int64_t i = idx ? idx[r] : r;
        out[r] = c_transform_one(qry + i * d, key, nk, d, logw, pot_key, eps);
    }
    free(logw);
}

/*
 * Row and column sums of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps).
 * Each sum is formed in index order by one thread.
 */
void oracle_marginals(const double *x, const double *y, const double *a, const double *b,
                      int64_t n, int64_t m, int d, double eps, const double *f, const double *g,
                      double *row_sum, double *col_sum)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            if (a[i] == 0.0 || b[j] == 0.0)
                continue;
            s += a[i] * b[j] * exp((f[i] + g[j] - sq_dist(x + i * d, y + j * d, d)) / eps);
        }
        row_sum[i] = s;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < m; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            if (a[i] == 0.0 || b[j] == 0.0)
                continue;
            s += a[i] * b[j] * exp((f[i] + g[j] - sq_dist(x + i * d, y + j * d, d)) / eps);
        }
        col_sum[j] = s;
    }
}

/*
 * Marginal residual of the plan at (f, g):
 *   out[0] = max_i |(P1)_i - a_i|,   out[1] = max_j |(P^T 1)_j - b_j|,
 *   out[2] = sum_i |(P1)_i - a_i|,   out[3] = sum_j |(P^T 1)_j - b_j|.
 */
void oracle_residual(const double *x, const double *y, const double *a, const double *b,
                     int64_t n, int64_t m, int d, double eps, const double *f, const double *g,
                     double *out)
{
    double *rs = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *cs = (double *)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    oracle_marginals(x, y, a, b, n, m, d, eps, f, g, rs, cs);
    double linf_r = 0.0, linf_c = 0.0, l1_r = 0.0, l1_c = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double e = fabs(rs[i] - a[i]);
        linf_r = e > linf_r ? e : linf_r;
        l1_r += e;
    }
    for (int64_t j = 0; j < m; ++j) {
        double e = fabs(cs[j] - b[j]);
        linf_c = e > linf_c ? e : linf_c;
        l1_c += e;
    }
    out[0] = linf_r;
    out[1] = linf_c;
    out[2] = l1_r;
    out[3] = l1_c;
    free(rs);
    free(cs);
}

/*
 * Fixed-count alternating Sinkhorn.  g starts from g_init (zeros when NULL).
 * Iteration k: f <- c-transform of g over the columns, then g <- c-transform
 * of the new f over the rows.  When check_every > 0, after iteration k with
 * k % check_every == 0 the residual max(out[0], out[1]) of oracle_residual at
 * (f, g) is stored in resid_trace[k / check_every - 1].
 */
void oracle_sinkhorn(const double *x, const double *y, const double *a, const double *b,
                     int64_t n, int64_t m, int d, double eps, int n_iters, int check_every,
                     const double *g_init, double *f, double *g, double *resid_trace)
{
    for (int64_t j = 0; j < m; ++j)
        g[j] = g_init ? g_init[j] : 0.0;
    for (int64_t i = 0; i < n; ++i)
        f[i] = 0.0;
    for (int k = 1; k <= n_iters; ++k) {
        oracle_half_step(x, n, y, m, d, b, g, eps, NULL, n, f);
        oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, g);
        if (check_every > 0 && k % check_every == 0 && resid_trace) {
            double r[4];
            oracle_residual(x, y, a, b, n, m, d, eps, f, g, r);
            resid_trace[k / check_every - 1] = r[0] > r[1] ? r[0] : r[1];
        }
    }
}

/*
 * Sinkhorn with a choice of update variant and stop rule (SinkSLOT README, API
 * Reference: variant "alternating" | "symmetric" with blend alpha; stop_mode
 * "fixed" | "marginal" | "potential" with stop_max_iter, stop_tol and
 * stop_check_every; Low-Level Solver API: iters_run, converged, final_viol).
 *   variant 0 (alternating, Gauss-Seidel): f <- T_row(g), then g <- T_col(new f).
 *   variant 1 (symmetric, Jacobi): from the old (f, g) compute T_row(g) and
 *     T_col(f), then f <- (1 - alpha) f + alpha T_row(g), g likewise.
 *   Both potentials start at 0.
 *   stop_mode 0: exactly max_iter iterations, *converged = -1, *final_viol = NaN.
 *   stop_mode 1: check after every check_every-th iteration and after the last
 *     one; the check value is max(|P1 - a|_inf, |P^T 1 - b|_inf) at (f, g);
 *     stop at the first check with value <= tol.
 *   stop_mode 2: same checks; the value is max(max_i |f_i - f'_i|, max_j
 *     |g_j - g'_j|) with (f', g') the potentials at the previous check (0 before
 *     the first), i.e. eps times the change of the absorbed potentials f/eps;
 *     stop at the first check with value < tol.
 * *iters_run is the number of iterations performed; *final_viol the value of
 * the last check.
 */
double oracle_dual_cost(const double *x, const double *y, const double *a, const double *b,
                        int64_t n, int64_t m, int d, double eps, const double *f, const double *g);

void oracle_sinkhorn_ex(const double *x, const double *y, const double *a, const double *b,
                        int64_t n, int64_t m, int d, double eps, int variant, double alpha,
                        int stop_mode, double tol, int max_iter, int check_every,
                        double *f, double *g, int *iters_run, int *converged, double *final_viol)
{
    double *fn = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *gn = (double *)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    double *fp = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    double *gp = (double *)calloc((size_t)(m > 0 ? m : 1), sizeof(double));
    for (int64_t i = 0; i < n; ++i)
        f[i] = 0.0;
    for (int64_t j = 0; j < m; ++j)
        g[j] = 0.0;
    *converged = stop_mode == 0 ? -1 : 0;
    *final_viol = NAN;
    int k = 0;
    while (k < max_iter) {
        ++k;
        if (variant == 0) {
            oracle_half_step(x, n, y, m, d, b, g, eps, NULL, n, f);
            oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, g);
        } else {
            oracle_half_step(x, n, y, m, d, b, g, eps, NULL, n, fn);
            oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, gn);
            for (int64_t i = 0; i < n; ++i)
                f[i] = (1.0 - alpha) * f[i] + alpha * fn[i];
            for (int64_t j = 0; j < m; ++j)
                g[j] = (1.0 - alpha) * g[j] + alpha * gn[j];
        }
        if (stop_mode == 0 || (k % check_every != 0 && k != max_iter))
            continue;
        double viol;
        if (stop_mode == 1) {
            double r[4];
            oracle_residual(x, y, a, b, n, m, d, eps, f, g, r);
            viol = r[0] > r[1] ? r[0] : r[1];
        } else {
            viol = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                double e = fabs(f[i] - fp[i]);
                viol = e > viol ? e : viol;
                fp[i] = f[i];
            }
            for (int64_t j = 0; j < m; ++j) {
                double e = fabs(g[j] - gp[j]);
                viol = e > viol ? e : viol;
                gp[j] = g[j];
            }
        }
        *final_viol = viol;
        if ((stop_mode == 1 && viol <= tol) || (stop_mode == 2 && viol < tol)) {
            *converged = 1;
            break;
        }
    }
    *iters_run = k;
    free(fn);
    free(gn);
    free(fp);
    free(gp);
}

/*
 * Barycentric gradient with respect to x at fixed g:
 *   grad_i = 2 a_i (x_i - sum_j w_ij y_j),
 *   w_ij = exp(z_ij) / sum_j exp(z_ij),  z_ij = (g_j - C_ij)/eps + log b_j.
 * The weights are the row of the plan normalised to sum 1 (the plan's row
 * once f is the c-transform of g).  Optionally restricted to rows idx.
 */
void oracle_grad_x(const double *x, const double *y, const double *a, const double *b,
                   int64_t n, int64_t m, int d, double eps, const double *g,
                   const int64_t *idx, int64_t nidx, double *grad)
{
    double *logw = (double *)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    for (int64_t j = 0; j < m; ++j)
        logw[j] = log_weight(b[j]);
    int64_t cnt = idx ? nidx : n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < cnt; ++r) {
        int64_t i = idx ? idx[r] : r;
        const double *xi = x + i * d;
        double zmax = -INFINITY;
        for (int64_t j = 0; j < m; ++j) {
            double z = (g[j] - sq_dist(xi, y + j * d, d)) / eps + logw[j];
            if (z > zmax)
                zmax = z;
        }
        double s = 0.0;
        double bary[256];
        for (int t = 0; t < d; ++t)
            bary[t] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double z = (g[j] - sq_dist(xi, y + j * d, d)) / eps + logw[j];
            double e = exp(z - zmax);
            s += e;
            for (int t = 0; t < d; ++t)
                bary[t] += e * y[j * d + t];
        }
        for (int t = 0; t < d; ++t)
            grad[r * d + t] = 2.0 * a[i] * (xi[t] - bary[t] / s);
    }
    free(logw);
}

/*
 * Entropic dual objective at (f, g):
 *   D = <a,f> + <b,g> - eps * (sum_ij P_ij - sum_i a_i * sum_j b_j).
 * Terms with a_i = 0 (or b_j = 0) are dropped from <a,f> (<b,g>).
 */
double oracle_dual_cost(const double *x, const double *y, const double *a, const double *b,
                        int64_t n, int64_t m, int d, double eps, const double *f, const double *g)
{
    double *rs = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *cs = (double *)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    oracle_marginals(x, y, a, b, n, m, d, eps, f, g, rs, cs);
    double af = 0.0, bg = 0.0, mass_p = 0.0, sa = 0.0, sb = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (a[i] > 0.0)
            af += a[i] * f[i];
        mass_p += rs[i];
        sa += a[i];
    }
    for (int64_t j = 0; j < m; ++j) {
        if (b[j] > 0.0)
            bg += b[j] * g[j];
        sb += b[j];
    }
    free(rs);
    free(cs);
    return af + bg - eps * (mass_p - sa * sb);
}

/*
 * Primal value of the plan at potentials (f, g),
 *   P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps),
 * out[0] = <P, C> + eps KL(P | a x b) with the generalised KL
 *          KL(P | Q) = sum_ij P_ij log(P_ij / Q_ij) - P_ij + Q_ij,
 * out[1] = <P, C>, the transport cost of the plan.
 * Each entry of P is formed and used as written (0 log 0 = 0 where a weight
 * is zero or an entry underflows); rows are summed in index order.  Reading:
 * the SinkSLOT README (Basic Usage) has its loss return the primal value of
 * the achieved plan; for entropic OT that is this objective, which equals the
 * dual objective at the optimum.
 */
void oracle_primal(const double *x, const double *y, const double *a, const double *b,
                   int64_t n, int64_t m, int d, double eps, const double *f, const double *g,
                   double *out)
{
    double *row_obj = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *row_pc = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        double obj = 0.0, pc = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double q = a[i] * b[j];
            double c = sq_dist(x + i * d, y + j * d, d);
            double p = q > 0.0 ? q * exp((f[i] + g[j] - c) / eps) : 0.0;
            double kl = p > 0.0 ? p * log(p / q) - p + q : q;
            pc += p * c;
            obj += p * c + eps * kl;
        }
        row_obj[i] = obj;
        row_pc[i] = pc;
    }
    double so = 0.0, sp = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        so += row_obj[i];
        sp += row_pc[i];
    }
    out[0] = so;
    out[1] = sp;
    free(row_obj);
    free(row_pc);
}

/*
 * Debiased entropic divergence S = OT(x,y) - OT(x,x)/2 - OT(y,y)/2, each term
 * the dual objective after n_iters iterations of the chosen variant (fixed
 * stop).  out[0] = S, out[1..3] = OT(x,y), OT(x,x), OT(y,y).  Reading: the
 * SinkSLOT README (opening section) contrasts its own objective, which is zero
 * at (x, x), with entropic OT, whose value at (x, x) is not zero and must be
 * subtracted; the three terms use the same solver and settings.
 */
void oracle_divergence(const double *x, const double *y, const double *a, const double *b,
                       int64_t n, int64_t m, int d, double eps, int variant, double alpha, int n_iters,
                       double *out)
{
    int64_t mx = n > m ? n : m;
    double *f = (double *)malloc((size_t)mx * sizeof(double));
    double *g = (double *)malloc((size_t)mx * sizeof(double));
    int it, conv;
    double viol;
    oracle_sinkhorn_ex(x, y, a, b, n, m, d, eps, variant, alpha, 0, 0.0, n_iters, 1, f, g, &it, &conv, &viol);
    double t_xy = oracle_dual_cost(x, y, a, b, n, m, d, eps, f, g);
    oracle_sinkhorn_ex(x, x, a, a, n, n, d, eps, variant, alpha, 0, 0.0, n_iters, 1, f, g, &it, &conv, &viol);
    double t_xx = oracle_dual_cost(x, x, a, a, n, n, d, eps, f, g);
    oracle_sinkhorn_ex(y, y, b, b, m, m, d, eps, variant, alpha, 0, 0.0, n_iters, 1, f, g, &it, &conv, &viol);
    double t_yy = oracle_dual_cost(y, y, b, b, m, m, d, eps, f, g);
    out[0] = t_xy - 0.5 * t_xx - 0.5 * t_yy;
    out[1] = t_xy;
    out[2] = t_xx;
    out[3] = t_yy;
    free(f);
    free(g);
}

/*
 * Gradient flow of the entropic cost in x (SinkSLOT README, Gradient Flow: an
 * explicit descent loop on the analytic gradient).  Each of the n_steps steps
 * solves afresh from g = 0 with n_iters alternating iterations at the current
 * x, takes the barycentric gradient at the final g, and moves
 * x <- x - lr * grad.  x (n x d) is updated in place; f, g and grad are those
 * of the last step (at the x before its move); cost_trace[k] (if not NULL) is
 * the dual cost at step k's potentials.
 */
void oracle_gradient_flow(double *x, const double *y, const double *a, const double *b,
                          int64_t n, int64_t m, int d, double eps, int n_iters, int n_steps, double lr,
                          double *cost_trace, double *f, double *g, double *grad)
{
    for (int k = 0; k < n_steps; ++k) {
        oracle_sinkhorn(x, y, a, b, n, m, d, eps, n_iters, 0, NULL, f, g, NULL);
        if (cost_trace)
            cost_trace[k] = oracle_dual_cost(x, y, a, b, n, m, d, eps, f, g);
        oracle_grad_x(x, y, a, b, n, m, d, eps, g, NULL, n, grad);
        for (int64_t e = 0; e < n * d; ++e)
            x[e] -= lr * grad[e];
    }
}

/* max_ij C_ij over all pairs (the scale of the parity tolerance). */
double oracle_max_cost(const double *x, const double *y, int64_t n, int64_t m, int d)
{
    double best = 0.0;
#pragma omp parallel for reduction(max : best) schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < m; ++j) {
            double c = sq_dist(x + i * d, y + j * d, d);
            if (c > best)
                best = c;
        }
    return best;
}
