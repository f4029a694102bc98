/*
 * sk.h -- C ABI of the streaming log-domain Sinkhorn library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library solves entropic optimal transport between two weighted point
 * clouds under squared-Euclidean cost, C_ij = |x_i - y_j|^2, without ever
 * forming the n x m cost or kernel matrix: every half-step is a streamed,
 * tiled log-sum-exp with a running maximum, computed on the GPU.
 *
 * Conventions shared by every entry point
 *  - Arrays are float32, row-major and contiguous, and live in device memory
 *    of the current HIP device unless stated otherwise.  x is (n, d), y is
 *    (m, d), a is (n), b is (m), f is (n), g is (m).  They are owned by the
 *    caller; the library never allocates, frees or retains them.
 *  - The library never allocates device memory (sk_solve_ex with a stop rule
 *    keeps a few pinned host bytes for its check values; the code object holds
 *    the static scratch of sk_solve_noalloc, one per GPU).  Entry points that need
 *    scratch space take a workspace `ws` of at least sk_workspace_bytes(n, m, d)
 *    bytes, 256-byte aligned, owned by the caller.  A workspace may be reused
 *    by later calls once the calls that used it have completed in stream order.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Compute entry
 *    points only enqueue work and return; results are ready when the stream
 *    reaches that point.  Only sk_check_inputs, and sk_solve_ex with a stop
 *    rule (at each check), wait for the stream.  The other compute entry points allocate
 *    nothing, synchronise nothing and use no memset, so they may be captured
 *    into a HIP graph and replayed (inputs, outputs and workspace at the
 *    captured addresses).
 *  - Weights are used exactly as given (not normalised); zeros are legal and
 *    such points contribute nothing.  Data-dependent validity (negative or
 *    non-finite values, unequal masses) is checked by sk_check_inputs, not by
 *    the compute entry points, which assume valid data.
 *  - Argument errors (NULL pointers, bad sizes, eps, iteration counts,
 *    unsupported d, short workspace) are detected on the host before anything
 *    is enqueued and are returned as an sk_status; nothing is launched then.
 *    A failed launch returns SK_ERR_HIP.
 *  - Supported dimensions: 1 <= d <= 256.  d <= 8 runs on the vector ALUs;
 *    9 <= d <= 256 computes the x.y cross term of the solver passes on matrix
 *    cores as three fp16 products of a two-part split of each fp32
 *    coordinate, scaled per cloud by a power of two and accumulated in fp32
 *    (the error per term lies within 2^-22 of |x_t y_t|, a few roundings of
 *    an fp32 dot product).  The workspace then also holds the keys' fp16
 *    parts, 4 bytes per padded coordinate, and each cloud's largest
 *    |coordinate|.
 *
 * Sources (page title and section):
 *  FS   = "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
 *         technical summary, Methodology 1-3.
 *  FS2  = "FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport", abstract.
 *  SLOT = SinkSLOT README: opening section, Tensor Contract, Gradient Flow,
 *         API Reference, Low-Level Solver API.
 */
#ifndef SK_H
#define SK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sk_status {
    SK_OK = 0,
    SK_ERR_NULL = 1,           /* a required pointer is NULL */
    SK_ERR_SHAPE = 2,          /* n < 1, m < 1 or d < 1, or n, m beyond 2^31 - 1; also a payload
                                  width, block size or block-pair count outside an entry
                                  point's limits (see sk_transport, sk_fs2_solve) */
    SK_ERR_UNSUPPORTED_D = 3,  /* d > 256 */
    SK_ERR_EPS = 4,            /* eps not finite or eps <= 0 */
    SK_ERR_ITERS = 5,          /* an iteration or step count out of range (n_iters < 0, ...) */
    SK_ERR_CHECK_EVERY = 6,    /* check_every < 0, or > 0 with resid_trace == NULL */
    SK_ERR_NEG_WEIGHT = 7,     /* some a_i or b_j < 0 */
    SK_ERR_MASS_MISMATCH = 8,  /* |sum a - sum b| > 1e-5 * max(sum a, sum b) */
    SK_ERR_EMPTY_MEASURE = 9,  /* sum a == 0 or sum b == 0 */
    SK_ERR_NONFINITE = 10,     /* NaN or Inf in x, y, a or b */
    SK_ERR_WORKSPACE = 11,     /* ws NULL, misaligned, or ws_bytes too small */
    SK_ERR_HIP = 12,           /* a HIP runtime call or kernel launch failed */
    SK_ERR_VARIANT = 13,       /* variant not 0 or 1, or symmetric with alpha outside (0, 1] */
    SK_ERR_STOP = 14,          /* stop_mode not 0, 1 or 2; or a stop rule with stop_tol < 0,
                                  non-finite, or check_every < 1; or a negative or non-finite
                                  threshold of sk_fs2_solve */
    SK_ERR_CAPTURE = 15,       /* a host-synchronous call (a stop rule, sk_fs2_solve) on a
                                  stream under graph capture */
    SK_ERR_LR = 16,            /* the gradient-flow step size is not finite */
    SK_ERR_SCRATCH = 17        /* sk_solve_noalloc: sk_workspace_bytes(n, m, d) exceeds
                                  SK_NOALLOC_SCRATCH_BYTES */
} sk_status;

/* Bytes of the static device scratch that sk_solve_noalloc works in (64 MiB). */
#define SK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Version of this ABI (incremented on any signature change). */
int sk_abi_version(void);

/* Human-readable name of a status code; never NULL, static storage. */
const char *sk_status_string(int status);

/*
 * Bytes of workspace needed by every entry point below for a problem of n
 * source points, m target points in dimension d (0 for invalid sizes).  The
 * size is O((n + m) d): the library keeps the clouds, potentials and per-row
 * partial statistics, never an n x m array (FS, Methodology 3: linear memory).
 */
size_t sk_workspace_bytes(int64_t n, int64_t m, int32_t d);

/*
 * Validates the data of a problem (SLOT, Tensor Contract): x and y finite,
 * a and b finite and nonnegative, sum(a) > 0, sum(b) > 0 and
 * |sum(a) - sum(b)| <= 1e-5 * max(sum(a), sum(b)) with the sums taken in
 * float64.  Synchronises `stream`.  Returns SK_OK or the first failing check
 * in the order NONFINITE, NEG_WEIGHT, EMPTY_MEASURE, MASS_MISMATCH.
 */
int sk_check_inputs(const float *x, const float *y, const float *a, const float *b,
                    int64_t n, int64_t m, int32_t d,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * Fixed-count alternating log-domain Sinkhorn (FS, Methodology 1; SLOT, API
 * Reference: variant "alternating", stop_mode "fixed").  Starting from g = 0,
 * each of the n_iters iterations computes
 *     f_i <- -eps * LSE_j[(g_j - C_ij)/eps + log b_j]      (row half-step)
 *     g_j <- -eps * LSE_i[(f_i - C_ij)/eps + log a_i]      (column half-step,
 *                                                           with the new f)
 * each as one streamed pass with an on-chip running max / sum-exp (FS,
 * Methodology 2).  On return f (n) and g (m) hold the potentials after the
 * last iteration, in cost units (f, not f/eps); n_iters = 0 gives f = g = 0.
 *
 * Residual trace: when check_every > 0, resid_trace (device, n_iters /
 * check_every floats) receives, for k = check_every, 2*check_every, ...,
 * the marginal residual max(|P1 - a|_inf, |P^T 1 - b|_inf) of the plan
 * P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) at the potentials after
 * iteration k (SLOT, API Reference, stop_mode "marginal" norm).  No early
 * stop is taken.  check_every = 0 disables the trace (resid_trace may be NULL).
 */
int sk_solve(const float *x, const float *y, const float *a, const float *b,
             int64_t n, int64_t m, int32_t d, float eps, int32_t n_iters,
             float *f, float *g, int32_t check_every, float *resid_trace,
             void *ws, size_t ws_bytes, void *stream);

/*
 * sk_solve started from a given g instead of 0 (SLOT, Low-Level Solver API:
 * the solver state is the pair of potentials, so a solve can continue from
 * one).  The first row half-step reads g_init (m, device, cost units); it may
 * alias g, which is then updated in place.  Running k1 iterations and then
 * k2 more from the resulting g is the (k1 + k2)-iteration trajectory up to
 * float32 rounding of the state handed over.  n_iters = 0 gives f = 0 and
 * g = g_init.  Everything else (trace, workspace, errors, capture) as
 * sk_solve.
 */
int sk_solve_warm(const float *x, const float *y, const float *a, const float *b,
                  int64_t n, int64_t m, int32_t d, float eps, int32_t n_iters,
                  const float *g_init, float *f, float *g, int32_t check_every,
                  float *resid_trace, void *ws, size_t ws_bytes, void *stream);

/*
 * sk_solve without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels, results and errors as
 * sk_solve, bit for bit; the workspace is instead a static device array of
 * SK_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held from the first
 * call on that GPU until the process ends.  Problems whose
 * sk_workspace_bytes(n, m, d) exceeds it return SK_ERR_SCRATCH before
 * anything is enqueued (64 MiB holds, e.g., n = m = 50,000 at d = 3 and
 * n = m = 16,384 at d = 64).  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine) and enqueues only.  The scratch keeps
 * the last call's contents; the solve writes every part of it before reading
 * it, so nothing is cleared.  All calls on one GPU share the one array: calls
 * whose work overlaps on that GPU (other streams, other threads, or the same
 * stream captured into graphs replayed concurrently) race and give undefined
 * results; serialise them.  The caller still passes inputs and outputs.
 */
int sk_solve_noalloc(const float *x, const float *y, const float *a, const float *b,
                     int64_t n, int64_t m, int32_t d, float eps, int32_t n_iters,
                     float *f, float *g, int32_t check_every, float *resid_trace,
                     void *stream);

/*
 * Entropic OT cost at potentials (f, g) that come out of a column half-step
 * (so the plan's column sums equal b): the dual objective
 *     <a, f> + <b, g> - eps * sum(b) * (1 - sum(a)),
 * accumulated in float64 in a fixed order (deterministic).  Terms with a zero
 * weight are skipped.  `out` is one device double.  For unit mass this is
 * <a, f> + <b, g>.
 */
int sk_cost(const float *a, const float *b, const float *f, const float *g,
            int64_t n, int64_t m, float eps, double *out, void *stream);

/*
 * Marginal residual of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) at
 * arbitrary potentials (f, g) (SLOT, API Reference: the "marginal" stop norm).
 * Two streamed passes (row sums and column sums of P, never stored).  `out`
 * is 4 device floats: [max_i |(P1)_i - a_i|, max_j |(P^T 1)_j - b_j|,
 * sum_i |(P1)_i - a_i|, sum_j |(P^T 1)_j - b_j|].
 */
int sk_marginal_residual(const float *x, const float *y, const float *a, const float *b,
                         int64_t n, int64_t m, int32_t d, float eps,
                         const float *f, const float *g, float *out,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Analytic gradient with respect to x at fixed g (FS, Methodology 3:
 * barycentric projection as a weighted average; no differentiation through
 * the iterations):
 *     grad_i = 2 a_i (x_i - sum_j w_ij y_j),
 *     w_ij = softmax_j((g_j - C_ij)/eps + log b_j),
 * one streamed pass with an on-chip running max and rescaled weighted sums.
 * `grad` is (n, d) device memory.
 */
int sk_grad_x(const float *x, const float *y, const float *a, const float *b,
              int64_t n, int64_t m, int32_t d, float eps, const float *g,
              float *grad, void *ws, size_t ws_bytes, void *stream);

/*
 * Sinkhorn with a choice of update variant and stop rule (SLOT, API
 * Reference: `variant`, `alpha`, `stop_mode`, `stop_max_iter`, `stop_tol`,
 * `stop_check_every`; Low-Level Solver API: iters_run, converged,
 * final_viol).  Both potentials start at 0.
 *
 * variant 0, alternating (Gauss-Seidel): each iteration is the row half-step
 *   from the current g, then the column half-step from the new f, exactly as
 *   sk_solve.
 * variant 1, symmetric (Jacobi): each iteration computes both half-steps from
 *   the potentials before it and blends, f <- (1 - alpha) f + alpha T_row(g),
 *   g <- (1 - alpha) g + alpha T_col(f), with 0 < alpha <= 1 (alpha is
 *   ignored for variant 0).
 * stop_mode 0, fixed: exactly max_iter iterations, no check; *converged = -1
 *   and *final_viol = NaN (the API's None).  Enqueues only, like sk_solve.
 * stop_mode 1, marginal, and 2, potential: a check follows every
 *   check_every-th iteration and the last one (max_iter is the cap).  The
 *   marginal value is max(|P1 - a|_inf, |P^T 1 - b|_inf) at the current
 *   potentials (for variant 0 the column term is zero by construction and is
 *   not evaluated); the run stops at the first check with value <= stop_tol.
 *   The potential value is max(max_i |f_i - f'_i|, max_j |g_j - g'_j|) against
 *   the potentials at the previous check (zero before the first), i.e. eps
 *   times the change of the absorbed potentials f/eps; the run stops at the
 *   first check with value < stop_tol.  A check value taken from a NaN
 *   state is NaN and never meets the tolerance.  At each check the host waits until
 *   `stream` has produced that check's value: the GPU stores it straight into
 *   pinned, mapped host memory and raises a flag there, which the host polls
 *   (a 64-byte slot per call in flight, allocated with hipHostMalloc on first
 *   need and kept by the library for the life of the process).  Work the
 *   caller enqueued on `stream` before the call is waited for as well.  On
 *   small problems (at most 4.2e6 pairs per pass, except the symmetric
 *   variant's marginal rule) a check's value is read only when the next check
 *   is due, so the GPU never waits for the host; the checked iteration's state
 *   is kept until then and a stop returns exactly the same outputs, after the
 *   iterations already enqueued past it have run.
 *   Calling with a stop rule on a stream under graph capture returns
 *   SK_ERR_CAPTURE before anything is enqueued.  The
 *   marginal value of iteration k is produced by the passes of iteration
 *   k + 1, so a check costs no extra pass except after the last iteration.
 * Outputs: f, g (device) hold the potentials after *iters_run iterations;
 *   iters_run, converged (1 met the tolerance, 0 hit the cap) and final_viol
 *   (value of the last check) are host pointers, written on SK_OK.
 * max_iter = 0 gives f = g = 0, *iters_run = 0 and no check.
 */
int sk_solve_ex(const float *x, const float *y, const float *a, const float *b,
                int64_t n, int64_t m, int32_t d, float eps,
                int32_t variant, float alpha, int32_t stop_mode, float stop_tol,
                int32_t max_iter, int32_t check_every,
                float *f, float *g, int32_t *iters_run, int32_t *converged,
                float *final_viol, void *ws, size_t ws_bytes, void *stream);

/*
 * Entropic dual objective at arbitrary potentials (f, g):
 *     <a, f> + <b, g> - eps * (sum_ij P_ij - sum(a) sum(b)),
 *     P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps),
 * with the plan mass from one streamed row pass (the row sums of P, never
 * stored) and every sum in float64 in a fixed order.  Unlike sk_cost it holds
 * for any potentials, e.g. those of the symmetric variant.  `out` is one
 * device double; ws as for sk_workspace_bytes(n, m, d).
 */
int sk_dual_cost(const float *x, const float *y, const float *a, const float *b,
                 int64_t n, int64_t m, int32_t d, float eps,
                 const float *f, const float *g, double *out,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Primal value of the plan at potentials (f, g) (SLOT, Basic Usage: the loss
 * reports the primal value of the plan it reached),
 *     P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps),
 *     out[0] = <P, C> + eps KL(P | a x b),
 *              KL(P | Q) = sum_ij P_ij log(P_ij / Q_ij) - P_ij + Q_ij,
 *     out[1] = <P, C>, the transport cost of the plan.
 * With log(P_ij / (a_i b_j)) = (f_i + g_j - C_ij)/eps, out[0] is computed as
 * <P1, f> + <P^T 1, g> - eps (sum P - sum(a) sum(b)); it equals the dual
 * objective (sk_dual_cost) at the optimum.  <P, C> comes from the per-row
 * sums of P [y, |y|^2] in the centred expanded form.  Three streamed passes
 * (for d > 8 four: a log-sum-exp pass first), P never stored; float64 sums in
 * a fixed order.  `out` is 2 device doubles; ws of at least
 * sk_transport_workspace_bytes(n, m, d) bytes.  Enqueues only.
 */
int sk_primal_cost(const float *x, const float *y, const float *a, const float *b,
                   int64_t n, int64_t m, int32_t d, float eps,
                   const float *f, const float *g, double *out,
                   void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of sk_divergence (0 for invalid sizes). */
size_t sk_divergence_workspace_bytes(int64_t n, int64_t m, int32_t d);

/*
 * Debiased entropic divergence S = OT(x, y) - OT(x, x)/2 - OT(y, y)/2 (SLOT,
 * opening section: entropic OT is not zero at (x, x), so a divergence built
 * from it subtracts the self-terms).  Each term is the dual objective
 * (sk_dual_cost) after n_iters iterations of the given variant and alpha
 * (fixed stop) on that pair of clouds.  `out` is 4 device doubles:
 * [S, OT(x,y), OT(x,x), OT(y,y)].  ws of at least
 * sk_divergence_workspace_bytes(n, m, d) bytes, 256-byte aligned.  Enqueues
 * only.
 */
int sk_divergence(const float *x, const float *y, const float *a, const float *b,
                  int64_t n, int64_t m, int32_t d, float eps,
                  int32_t variant, float alpha, int32_t n_iters, double *out,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * Gradient flow of the entropic cost in x (SLOT, Gradient Flow: explicit
 * descent on the analytic gradient).  Each of the n_steps steps enqueues a
 * fresh sk_solve of n_iters iterations at the current x (from g = 0), the
 * gradient sk_grad_x at the resulting g, and the move x <- x - lr * grad.
 * x (n, d, device) is updated in place.  On return f, g and grad (n, d) hold
 * the last step's potentials and gradient, taken at the x before its move;
 * cost_trace (device doubles, n_steps entries, or NULL) receives each step's
 * sk_cost.  n_steps = 0 leaves everything untouched.  ws as for
 * sk_workspace_bytes(n, m, d).  Enqueues only (capturable into a graph).
 */
int sk_gradient_flow(float *x, const float *y, const float *a, const float *b,
                     int64_t n, int64_t m, int32_t d, float eps,
                     int32_t n_iters, int32_t n_steps, float lr,
                     float *f, float *g, float *grad, double *cost_trace,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Workspace bytes of sk_transport and sk_hvp (0 for invalid sizes).  It is
 * larger than sk_workspace_bytes: it adds the split partials of the transport
 * passes and the vectors of the Hessian-vector product, all O((n + m) d).
 */
size_t sk_transport_workspace_bytes(int64_t n, int64_t m, int32_t d);

/*
 * Transport product with the plan at potentials (f, g) (FS, Methodology 3:
 * the transport matrix applied by the same streamed traversal as the
 * half-steps, never stored):
 *     P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps),
 *     transpose = 0:  out (n, k) = P v,    v (m, k);
 *     transpose = 1:  out (m, k) = P^T v,  v (n, k).
 * Row-major, device memory; k >= 1 (columns are processed 9 per pass for
 * d <= 8, 16 or 64 per pass on the matrix cores).  For d <= 8 each row runs
 * an on-chip running maximum; for d > 8 a first pass stores each row's
 * log-sum-exp of the scores so that every weight is at most 1; either way the
 * result is exact up to float32 rounding for any potentials.  ws of at least
 * sk_transport_workspace_bytes(n, m, d).  Enqueues only.
 */
int sk_transport(const float *x, const float *y, const float *a, const float *b,
                 int64_t n, int64_t m, int32_t d, float eps,
                 const float *f, const float *g, int32_t transpose,
                 const float *v, int32_t k, float *out,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Hessian-vector product of the entropic OT cost OT_eps(x, y) in the source
 * points x, at the plan of (f, g) (FS, Methodology 3: a streamed product built
 * from transport-vector and transport-matrix products, O((n + m) d) memory).
 * By implicit differentiation at the plan, with r = P 1, c = P^T 1 and
 * Cdot_ij = 2 <x_i - y_j, v_i>, the potential derivatives (phi, psi) solve
 *     r_i phi_i + (P psi)_i = sum_j P_ij Cdot_ij,
 *     (P^T phi)_j + c_j psi_j = sum_i P_ij Cdot_ij,
 * and out_i = 2 r_i v_i - (2/eps) sum_j P_ij (phi_i + psi_j - Cdot_ij) y_j.
 * At the optimal (f, g) this is the exact Hessian of the entropic cost; for
 * other potentials it is the same formula at their plan.  The system is
 * solved by cg_iters steps of conjugate gradients preconditioned by
 * diag(r, c)^-1 (two streamed passes each), with the residual kept
 * orthogonal to the gauge direction (1, -1), on which the system is
 * singular; the iterate with the smallest residual is used, so extra steps
 * never make the result worse.  cg_resid (one device float, or NULL)
 * receives that iterate's preconditioned residual relative to the start.
 * v and out are (n, d) device arrays.  For d > 8 the two log-sum-exp passes
 * that the matrix-core products need are taken once, the plan being fixed.
 * ws of at least sk_transport_workspace_bytes(n, m, d).  Enqueues only.
 */
int sk_hvp(const float *x, const float *y, const float *a, const float *b,
           int64_t n, int64_t m, int32_t d, float eps,
           const float *f, const float *g, const float *v, int32_t cg_iters,
           float *out, float *cg_resid, void *ws, size_t ws_bytes, void *stream);

/*
 * Workspace bytes of sk_fs2_solve for the given block size and sample count
 * (0 for invalid arguments, or when the radix sort's scratch size cannot be
 * queried because no device is present).  The size does not depend on the
 * thresholds; the kept-tile lists take at most 2^28 entries per side, so it
 * stays O(n + m + NBx + NBy).
 */
size_t sk_fs2_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t block, int32_t n_sample);

/*
 * Two-stage block-sparse solver (FS2): a coarse stage on block centroids, then
 * block-sparse point-level iterations, for low-dimensional clouds (1 <= d <= 8).
 * The pages describe it only in outline; the steps taken are:
 *  1. Morton order of each cloud in the bounding box of both (float32
 *     quantisation to 30 / d bits per coordinate, at most 10; a stable radix
 *     sort of (code, index)), and blocks of `block` consecutive points
 *     (1 <= block <= 512) with their mass, weighted centroid and box;
 *  2. coarse stage: alternating Sinkhorn on the centroid measures (from G = 0,
 *     then continuing) in rounds of coarse_iters; after each round both
 *     potentials are lifted to the points by one c-transform against the
 *     other side's centroids, and the check value is the largest row
 *     deviation |(P1)_i - a_i| of the lifted plan over n_sample evenly spaced
 *     rows (P over all points).  The coarse stage ends when the check value
 *     is <= tol, or fell by less than the fraction coarse_gain since the last
 *     round, or after max_rounds rounds.  These comparisons are made on the
 *     base-2 logarithm of the check value, which stays finite when the value
 *     itself (a far-off lift at small eps) is beyond float32 range;
 *  3. fine stage from the lifted potentials: before every screen_every-th
 *     iteration each block pair (I, J) gets the bound
 *       (max_I f + max_J g - dmin_IJ^2)/eps + log max(B_J NBy, A_I NBx)
 *     (dmin the distance between the blocks' boxes; maxima over points of
 *     positive weight; NBx, NBy the block counts) and is kept iff it exceeds
 *     log delta (every pair when delta = 0), so that the omitted pairs add at
 *     most delta a_i to any row's and delta b_j to any column's mass; each
 *     block also keeps its pair of largest bound.  Each iteration is a row
 *     and a column half-step over kept pairs only (the kept pairs shared out
 *     evenly over the workgroups); after every check_every-th
 *     iteration and the last, the row residual of the kept-pair plan (its
 *     column sums are exact) is checked and the stage stops at <= tol.
 * Outputs f, g (device, caller's order).  info_i (host, 4): coarse rounds,
 * fine iterations, kept block pairs at the last screening, converged (0/1);
 * info_f (host, 2): last fine residual (NaN without a check), last coarse
 * check value (+inf when beyond float32 range).  perm_x, perm_y (device, n and m ints, or NULL) receive the
 * Morton order (original index of each sorted point).  Host-synchronous
 * (the checks are read back); refuses graph capture (SK_ERR_CAPTURE).
 * Also SK_ERR_SHAPE for a block outside [1, 512], more than 2^36 block pairs,
 * delta = 0 (every pair kept) with more than 2^28 block pairs, or -- during
 * the solve, returned at the screening that found it -- more than 2^28 kept
 * pairs (raise delta or the block size), SK_ERR_STOP for a negative or non-finite tol, delta or coarse_gain,
 * SK_ERR_ITERS for counts below 1 (max_iters may be 0).
 */
int sk_fs2_solve(const float *x, const float *y, const float *a, const float *b,
                 int64_t n, int64_t m, int32_t d, float eps, int32_t block,
                 float tol, float delta, int32_t coarse_iters, int32_t max_rounds,
                 float coarse_gain, int32_t n_sample, int32_t max_iters,
                 int32_t check_every, int32_t screen_every,
                 float *f, float *g, int32_t *info_i, float *info_f,
                 int32_t *perm_x, int32_t *perm_y,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Kernel timing of the streamed log-sum-exp passes (benchmark diagnostics).
 * sk_timing_enable(k) with k >= 1 resets the counters and from then on times
 * every k-th streamed-pass kernel that the entry points enqueue with a HIP
 * event pair recorded with the kernel's own dispatch (hipExtLaunchKernel: the
 * pair spans the kernel alone) (k = 1: every one; a larger k keeps the host
 * cost of the events off small problems); the split merge and the other
 * kernels are not timed.  Auxiliary passes are left out so that the
 * timed launches are of one kernel: the store-lse passes of the transport
 * products and the Hessian-vector product, the HVP's products outside its
 * conjugate-gradient steps, and the coarse stage of sk_fs2_solve (whose timed
 * launches are the block-sparse passes of the fine stage, counted by the
 * point pairs of the kept blocks).  sk_timing_enable(0)
 * stops recording.  sk_timing_read waits for the recorded events and returns
 * the total kernel milliseconds, the number of timed launches and the number
 * of (query, key) pairs those launches evaluated.  Launches enqueued while the
 * stream is being captured into a graph are not timed (nor counted).  Events
 * come from a process-wide pool that grows on demand; calls from several
 * threads at once are serialised.  Returns SK_ERR_NULL for NULL outputs,
 * SK_ERR_HIP on a HIP failure.
 */
int sk_timing_enable(int enable);
int sk_timing_read(double *total_ms, int64_t *launches, double *pairs);

#ifdef __cplusplus
}
#endif

#endif /* SK_H */
