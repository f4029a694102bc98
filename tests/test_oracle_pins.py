"""Pins for the CPU oracle: each oracle function is checked against something
other than itself -- a closed form, a textbook route, a library routine, brute
force or an exact invariant -- and every planted mistake in the oracle source
must trip at least one pin (mutation check at the bottom).

Sources: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
(Methodology 1-3), SinkSLOT README (Tensor Contract, API Reference), and
"Sinkhorn Distances: Lightspeed Computation of Optimal Transportation
Distances" (named in the FlashSinkhorn 2 reference list) for the matrix-scaling
form used as the brute-force route.
"""
import itertools
import math
import os
import re

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment
from scipy.spatial.distance import cdist
from scipy.special import logsumexp

import oracle
from sk_inputs import random_problem

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _problem(n, m, d, seed, scale=1.0):
    x, y, a, b = random_problem(n, m, d, seed, scale=scale)
    return (x.astype(np.float64), y.astype(np.float64), a.astype(np.float64) / a.astype(np.float64).sum(),
            b.astype(np.float64) / b.astype(np.float64).sum())


def _scaling_form(x, y, a, b, eps, n_iters):
    """Matrix scaling u = a / (K v), v = b / (K^T u), K = exp(-C/eps), started at v = b
    (the scaling-form image of g = 0); returns (f, g, P) with f = eps log(u/a),
    g = eps log(v/b) and P = diag(u) K diag(v)."""
    K = np.exp(-cdist(x, y, "sqeuclidean") / eps)
    v = b.copy()
    u = None
    for _ in range(n_iters):
        u = a / (K @ v)
        v = b / (K.T @ u)
    return eps * np.log(u / a), eps * np.log(v / b), u[:, None] * K * v[None, :]


# --------------------------------------------------------------------------- pins
def pin_scaling_form_trajectory(lib):
    """Log-domain iterates equal the matrix-scaling iterates (tiny, moderate eps)."""
    for (n, m, d, seed, eps, iters) in [(7, 5, 2, 11, 0.5, 1), (7, 5, 2, 11, 0.5, 2), (6, 9, 3, 12, 2.0, 15),
                                        (8, 8, 1, 13, 0.3, 40), (5, 11, 4, 14, 1.0, 7)]:
        x, y, a, b = _problem(n, m, d, seed)
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters, lib=lib)
        fs, gs, _ = _scaling_form(x, y, a, b, eps, iters)
        scale = cdist(x, y, "sqeuclidean").max()
        assert np.max(np.abs(f - fs)) <= 1e-11 * scale, (n, m, d, iters)
        assert np.max(np.abs(g - gs)) <= 1e-11 * scale, (n, m, d, iters)


def pin_scaling_form_warm_start(lib):
    """From a given g_init the log-domain iterates equal the matrix-scaling iterates started at
    v = b exp(g_init / eps), the scaling-form image of g_init."""
    for (n, m, d, seed, eps, iters) in [(7, 5, 2, 51, 0.5, 1), (6, 9, 3, 52, 2.0, 6), (8, 8, 1, 53, 0.3, 12)]:
        x, y, a, b = _problem(n, m, d, seed)
        g0 = np.random.default_rng(seed + 1).normal(size=m) * eps
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters, g_init=g0, lib=lib)
        K = np.exp(-cdist(x, y, "sqeuclidean") / eps)
        v = b * np.exp(g0 / eps)
        for _ in range(iters):
            u = a / (K @ v)
            v = b / (K.T @ u)
        scale = cdist(x, y, "sqeuclidean").max()
        assert np.max(np.abs(f - eps * np.log(u / a))) <= 1e-11 * scale, (n, m, d, iters)
        assert np.max(np.abs(g - eps * np.log(v / b))) <= 1e-11 * scale, (n, m, d, iters)


def pin_marginals_scaling_form(lib):
    """Plan marginals and residual norms equal those of the explicit scaled plan."""
    for (n, m, d, seed, eps, iters) in [(7, 5, 2, 21, 0.5, 3), (9, 6, 3, 22, 0.8, 1)]:
        x, y, a, b = _problem(n, m, d, seed)
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters, lib=lib)
        _, _, P = _scaling_form(x, y, a, b, eps, iters)
        rs, cs = oracle.marginals(x, y, a, b, f, g, eps, lib=lib)
        assert np.allclose(rs, P.sum(1), rtol=1e-11, atol=0)
        assert np.allclose(cs, P.sum(0), rtol=1e-11, atol=0)
        r = oracle.residual(x, y, a, b, f, g, eps, lib=lib)
        er, ec = P.sum(1) - a, P.sum(0) - b
        want = [np.abs(er).max(), np.abs(ec).max(), np.abs(er).sum(), np.abs(ec).sum()]
        assert np.allclose(r, want, rtol=1e-8, atol=1e-15)
        assert want[0] > 1e-6  # a non-trivial residual was compared


def pin_m1_closed_form(lib):
    """m = 1: after one iteration f_i = C_i1 - eps log b_1 (b_1 = sum a), g = 0,
    grad_i = 2 a_i (x_i - y_1), cost = sum_i a_i C_i1 (unit mass)."""
    x, y, a, b = _problem(6, 1, 2, 31)
    eps = 0.37
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 1, lib=lib)
    C = ((x - y[0]) ** 2).sum(1)
    assert np.allclose(f, C - eps * np.log(b[0]), rtol=0, atol=1e-13)
    assert abs(g[0]) <= 1e-13
    grad = oracle.grad_x(x, y, a, b, g, eps, lib=lib)
    assert np.allclose(grad, 2 * a[:, None] * (x - y[0]), rtol=0, atol=1e-13)
    assert abs(oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib) - (a * C).sum()) <= 1e-13
    # n = 1 (the transpose): f_1 = C_1j-weighted LSE, g_j = C_1j - f_1 + ... ; the plan is b itself
    x1, y1, a1, b1 = _problem(1, 5, 2, 32)
    f1, g1, _ = oracle.sinkhorn(x1, y1, a1, b1, eps, 1, lib=lib)
    C1 = ((y1 - x1[0]) ** 2).sum(1)
    assert np.allclose(f1 + g1, C1, rtol=0, atol=1e-13)
    assert abs(oracle.dual_cost(x1, y1, a1, b1, f1, g1, eps, lib=lib) - (b1 * C1).sum()) <= 1e-13


def pin_grad_finite_difference(lib):
    """grad equals the derivative of x -> sum_i a_i f~_i(x) at fixed g (envelope theorem)."""
    x, y, a, b = _problem(5, 7, 3, 41)
    rng = np.random.default_rng(42)
    g = rng.normal(size=7)
    eps = 0.3
    grad = oracle.grad_x(x, y, a, b, g, eps, lib=lib)
    h = 1e-5
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for t in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[i, t] += h
            xm[i, t] -= h
            fp = (a * oracle.half_step(xp, y, b, g, eps, lib=lib)).sum()
            fm = (a * oracle.half_step(xm, y, b, g, eps, lib=lib)).sum()
            fd[i, t] = (fp - fm) / (2 * h)
    assert np.allclose(grad, fd, rtol=1e-7, atol=1e-9)
    # restricted rows agree with the full computation
    sub = oracle.grad_x(x, y, a, b, g, eps, idx=[4, 0, 2], lib=lib)
    assert np.array_equal(sub, grad[[4, 0, 2]])


def pin_column_marginal_exact(lib):
    """After the g half-step the plan's column sums equal b (to rounding)."""
    x, y, a, b = _problem(9, 13, 2, 51)
    f, g, _ = oracle.sinkhorn(x, y, a, b, 0.05, 4, lib=lib)
    _, cs = oracle.marginals(x, y, a, b, f, g, 0.05, lib=lib)
    assert np.allclose(cs, b, rtol=1e-12, atol=0)


def pin_dual_cost_identity(lib):
    """With exact column marginals, D(f,g) = <a,f> + <b,g> - eps * M (1 - M), M = sum a = sum b."""
    for scale_mass in (1.0, 2.5):
        x, y, a, b = _problem(8, 6, 2, 52)
        a, b = a * scale_mass, b * scale_mass
        eps = 0.2
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 5, lib=lib)
        M = a.sum()
        want = (a * f).sum() + (b * g).sum() - eps * M * (1 - M)
        assert abs(oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib) - want) <= 1e-12 * max(1.0, abs(want))


def pin_gauge_invariance(lib):
    """Plan, residual, grad and cost are unchanged under (f + c, g - c) with balanced mass."""
    x, y, a, b = _problem(7, 9, 2, 61)
    eps = 0.4
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 3, lib=lib)
    c = 0.731
    r0, r1 = oracle.residual(x, y, a, b, f, g, eps, lib=lib), oracle.residual(x, y, a, b, f + c, g - c, eps, lib=lib)
    assert np.allclose(r0, r1, rtol=1e-10, atol=1e-16)
    g0, g1 = oracle.grad_x(x, y, a, b, g, eps, lib=lib), oracle.grad_x(x, y, a, b, g - c, eps, lib=lib)
    assert np.allclose(g0, g1, rtol=1e-12, atol=1e-15)
    c0 = oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib)
    c1 = oracle.dual_cost(x, y, a, b, f + c, g - c, eps, lib=lib)
    assert abs(c0 - c1) <= 1e-12


def pin_translation_covariance(lib):
    """Shifting y by t adds alpha_i = |t|^2 - 2<t,x_i> to f and beta_j = 2<t,y_j> to g
    along the whole trajectory when g starts at beta."""
    x, y, a, b = _problem(6, 8, 3, 71)
    t = np.array([0.7, -1.3, 2.1])
    eps = 0.25
    alpha = t @ t - 2 * x @ t
    beta = 2 * y @ t
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 6, lib=lib)
    f2, g2, _ = oracle.sinkhorn(x, y + t, a, b, eps, 6, g_init=beta, lib=lib)
    assert np.allclose(f2, f + alpha, rtol=0, atol=1e-10)
    assert np.allclose(g2, g + beta, rtol=0, atol=1e-10)


def pin_strong_duality(lib):
    """At convergence the dual cost equals the primal <P,C> + eps KL(P | a x b) of the scaled plan."""
    x, y, a, b = _problem(6, 5, 2, 81)
    eps = 0.5
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 3000, lib=lib)
    _, _, P = _scaling_form(x, y, a, b, eps, 3000)
    C = cdist(x, y, "sqeuclidean")
    ab = a[:, None] * b[None, :]
    primal = (P * C).sum() + eps * ((P * np.log(P / ab)).sum() - P.sum() + ab.sum())
    assert abs(oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib) - primal) <= 1e-10 * max(1.0, abs(primal))
    assert oracle.residual(x, y, a, b, f, g, eps, lib=lib)[0] < 1e-12


def pin_primal_explicit_plan(lib):
    """The primal value and <P,C> at potentials off the optimum equal those of the explicit matrix-scaling plan
    with the generalised KL written out: the scaling plan diag(u) K diag(v) after a few iterations, with v
    rescaled by exp(delta_j / eps), is the plan of (f, g + delta), whose mass differs from sum(a) sum(b)."""
    for (n, m, d, seed, eps, iters) in [(7, 5, 2, 61, 0.5, 2), (6, 9, 3, 62, 0.8, 1), (5, 5, 1, 63, 0.3, 4)]:
        x, y, a, b = _problem(n, m, d, seed)
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters, lib=lib)
        delta = 0.3 * eps * np.random.default_rng(seed).normal(size=m)
        g = g + delta
        _, _, P = _scaling_form(x, y, a, b, eps, iters)
        P = P * np.exp(delta / eps)[None, :]
        C = cdist(x, y, "sqeuclidean")
        ab = a[:, None] * b[None, :]
        want = (P * C).sum() + eps * ((P * np.log(P / ab)).sum() - P.sum() + ab.sum())
        assert abs(P.sum() - 1.0) > 1e-6  # the mass terms of the KL matter here
        got, pc = oracle.primal(x, y, a, b, f, g, eps, lib=lib)
        assert abs(got - want) <= 1e-11 * max(1.0, abs(want)), (n, m, d)
        assert abs(pc - (P * C).sum()) <= 1e-11 * max(1.0, (P * C).sum()), (n, m, d)


def pin_primal_duality_and_closed_forms(lib):
    """At convergence the primal value equals the dual cost; with one target point after one iteration the
    plan is a itself, so <P,C> = sum_i a_i C_i1 and the KL vanishes (unit mass); zero-weight points add nothing."""
    x, y, a, b = _problem(6, 5, 2, 81)
    eps = 0.5
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 3000, lib=lib)
    pr, pc = oracle.primal(x, y, a, b, f, g, eps, lib=lib)
    assert abs(pr - oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib)) <= 1e-10 * max(1.0, abs(pr))
    assert pc < pr  # the entropic term is positive here
    x1, y1, a1, b1 = _problem(6, 1, 2, 31)
    f1, g1, _ = oracle.sinkhorn(x1, y1, a1, b1, 0.37, 1, lib=lib)
    pr1, pc1 = oracle.primal(x1, y1, a1, b1, f1, g1, 0.37, lib=lib)
    C1 = ((x1 - y1[0]) ** 2).sum(1)
    assert abs(pc1 - (a1 * C1).sum()) <= 1e-13 and abs(pr1 - pc1) <= 1e-13
    # zero weights: dropping the weightless points changes neither value
    xz, yz, az, bz = _problem(9, 7, 2, 64)
    az[[1, 4]] = 0.0
    bz[2] = 0.0
    az, bz = az / az.sum(), bz / bz.sum()
    fz, gz, _ = oracle.sinkhorn(xz, yz, az, bz, 0.4, 5, lib=lib)
    keep_a, keep_b = az > 0, bz > 0
    full = oracle.primal(xz, yz, az, bz, fz, gz, 0.4, lib=lib)
    part = oracle.primal(xz[keep_a], yz[keep_b], az[keep_a], bz[keep_b], fz[keep_a], gz[keep_b], 0.4, lib=lib)
    assert np.allclose(full, part, rtol=1e-13, atol=0)


def pin_large_eps_limit(lib):
    """As eps grows the plan tends to a x b and the cost to sum_ij a_i b_j C_ij."""
    x, y, a, b = _problem(7, 6, 2, 91)
    eps = 1e6
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 5, lib=lib)
    want = (a[:, None] * b[None, :] * cdist(x, y, "sqeuclidean")).sum()
    assert abs(oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib) - want) <= 1e-5 * want


def pin_small_eps_bruteforce(lib):
    """Uniform n = m: OT_0 <= D <= OT_0 + eps log n at convergence, OT_0 by enumerating permutations."""
    x, y, a, b = _problem(6, 6, 2, 101)
    a, b = np.full(6, 1 / 6), np.full(6, 1 / 6)
    C = cdist(x, y, "sqeuclidean")
    ot0 = min(C[np.arange(6), list(p)].mean() for p in itertools.permutations(range(6)))
    r, c = linear_sum_assignment(C)
    assert abs(C[r, c].mean() - ot0) <= 1e-12
    # converged: both bounds; OT_0 <= OT_eps <= OT_0 + eps log n (permutation plan)
    f, g, _ = oracle.sinkhorn(x, y, a, b, 0.2, 20000, lib=lib)
    assert oracle.residual(x, y, a, b, f, g, 0.2, lib=lib)[0] < 1e-12
    D = oracle.dual_cost(x, y, a, b, f, g, 0.2, lib=lib)
    assert ot0 - 1e-9 <= D <= ot0 + 0.2 * math.log(6) + 1e-9
    # any iterate: weak duality, D(f, g) <= OT_eps <= OT_0 + eps log n
    for eps in (0.05, 0.01):
        for k in (1, 10, 300):
            f, g, _ = oracle.sinkhorn(x, y, a, b, eps, k, lib=lib)
            assert oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib) <= ot0 + eps * math.log(6) + 1e-9


def pin_1d_sorting(lib):
    """1-D uniform measures: OT_0 is the cost of the sorted (monotone) matching."""
    rng = np.random.default_rng(111)
    x = rng.normal(size=(40, 1))
    y = rng.normal(size=(40, 1)) * 0.7 + 0.4
    a = np.full(40, 1 / 40)
    ot0 = ((np.sort(x[:, 0]) - np.sort(y[:, 0])) ** 2).mean()
    eps = 0.05
    f, g, _ = oracle.sinkhorn(x, y, a, a, eps, 30000, lib=lib)
    assert oracle.residual(x, y, a, a, f, g, eps, lib=lib)[0] < 1e-6
    D = oracle.dual_cost(x, y, a, a, f, g, eps, lib=lib)
    assert ot0 - 1e-6 <= D <= ot0 + eps * math.log(40) + 1e-9


def pin_self_term(lib):
    """(x, x, a, a) at convergence: f - g is constant and 0 <= OT_eps(x,x) <= eps H(a)
    (the diagonal plan bounds it), unlike a divergence that vanishes at (x, x)."""
    x, _, a, _ = _problem(9, 9, 2, 121)
    eps = 0.3
    f, g, _ = oracle.sinkhorn(x, x, a, a, eps, 4000, lib=lib)
    assert np.ptp(f - g) < 1e-7
    D = oracle.dual_cost(x, x, a, a, f, g, eps, lib=lib)
    H = -(a * np.log(a)).sum()
    assert 0.0 < D <= eps * H


def pin_zero_weights(lib):
    """Zero-weight points change nothing for the others: the problem with them removed
    gives the same f, g, cost and gradient on the remaining points; grad is 0 where a_i = 0."""
    x, y, a, b = _problem(10, 8, 2, 131)
    a[[1, 4, 7]] = 0.0
    b[[0, 5]] = 0.0
    a, b = a / a.sum(), b / b.sum()
    eps = 0.15
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 6, lib=lib)
    ka, kb = a > 0, b > 0
    fr, gr, _ = oracle.sinkhorn(x[ka], y[kb], a[ka], b[kb], eps, 6, lib=lib)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    assert np.allclose(f[ka], fr, rtol=0, atol=1e-12)
    assert np.allclose(g[kb], gr, rtol=0, atol=1e-12)
    assert abs(oracle.dual_cost(x, y, a, b, f, g, eps, lib=lib)
               - oracle.dual_cost(x[ka], y[kb], a[ka], b[kb], fr, gr, eps, lib=lib)) <= 1e-12
    gx = oracle.grad_x(x, y, a, b, g, eps, lib=lib)
    assert np.all(gx[~ka] == 0.0)
    assert np.allclose(gx[ka], oracle.grad_x(x[ka], y[kb], a[ka], b[kb], gr, eps, lib=lib), rtol=0, atol=1e-12)


def pin_half_step_vs_logsumexp(lib):
    """The c-transform equals -eps * scipy.special.logsumexp((g - C_i.)/eps, b=w), also at tiny eps."""
    x, y, a, b = _problem(12, 30, 3, 141)
    rng = np.random.default_rng(142)
    g = rng.normal(size=30)
    C = cdist(x, y, "sqeuclidean")
    for eps in (1.0, 1e-2, 1e-4):
        want = -eps * logsumexp((g[None, :] - C) / eps, b=b[None, :], axis=1)
        got = oracle.half_step(x, y, b, g, eps, lib=lib)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * C.max())
        sub = oracle.half_step(x, y, b, g, eps, idx=[3, 11], lib=lib)
        assert np.array_equal(sub, got[[3, 11]])


def pin_max_cost(lib):
    """Exhaustive max cost equals scipy's cdist maximum; the hull shortcut equals the exhaustive scan."""
    rng = np.random.default_rng(151)
    x, y = rng.random((300, 3)), rng.random((400, 3)) * 1.3
    want = cdist(x, y, "sqeuclidean").max()
    assert oracle.max_cost(x, y, lib=lib) == pytest.approx(want, rel=1e-14)
    assert oracle.max_cost_hull(x, y) == pytest.approx(want, rel=1e-14)


def pin_residual_trace(lib):
    """The residual trace holds the residual at (f_k, g_k) for k = c, 2c, ...; the run with
    fewer iterations is a prefix of the longer one."""
    x, y, a, b = _problem(8, 7, 2, 161)
    eps = 0.2
    f, g, tr = oracle.sinkhorn(x, y, a, b, eps, 9, check_every=3, lib=lib)
    assert tr.shape == (3,)
    for k, r in zip((3, 6, 9), tr):
        fk, gk, _ = oracle.sinkhorn(x, y, a, b, eps, k, lib=lib)
        res = oracle.residual(x, y, a, b, fk, gk, eps, lib=lib)
        assert r == pytest.approx(max(res[0], res[1]), rel=1e-12, abs=1e-18)
    assert np.array_equal(f, oracle.sinkhorn(x, y, a, b, eps, 9, lib=lib)[0])


# ---- update variants, stop rules and the debiased divergence (SinkSLOT README, API Reference,
# Low-Level Solver API, opening section)
def _plan(x, y, a, b, f, g, eps):
    C = cdist(x, y, "sqeuclidean")
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)


def pin_jacobi_first_steps(lib):
    """Symmetric variant from zero potentials: one step gives alpha * T(0) on each side; the second
    blends the first with the c-transforms of the OTHER side's first-step potential (both from old
    values).  T is the c-transform written with scipy's logsumexp."""
    x, y, a, b = _problem(9, 7, 2, 171)
    eps, alpha = 0.3, 0.3
    C = cdist(x, y, "sqeuclidean")
    T_row = lambda g: -eps * logsumexp((g[None, :] - C) / eps, b=b[None, :], axis=1)
    T_col = lambda f: -eps * logsumexp((f[:, None] - C) / eps, b=a[:, None], axis=0)
    f1, g1, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=alpha, max_iter=1, lib=lib)
    assert it == 1 and conv is None and math.isnan(viol)
    assert np.allclose(f1, alpha * T_row(np.zeros(7)), rtol=0, atol=1e-12)
    assert np.allclose(g1, alpha * T_col(np.zeros(9)), rtol=0, atol=1e-12)
    f2, g2, *_ = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=alpha, max_iter=2, lib=lib)
    assert np.allclose(f2, (1 - alpha) * f1 + alpha * T_row(g1), rtol=0, atol=1e-12)
    assert np.allclose(g2, (1 - alpha) * g1 + alpha * T_col(f1), rtol=0, atol=1e-12)


def pin_jacobi_alpha1_interleaves(lib):
    """With alpha = 1 the Jacobi sequence holds the alternating one at every other step:
    Jacobi f after 2k-1 steps is alternating f after k, Jacobi g after 2k is alternating g after k."""
    x, y, a, b = _problem(8, 6, 3, 181)
    eps = 0.4
    for k in (1, 2, 5):
        fa, ga, _ = oracle.sinkhorn(x, y, a, b, eps, k, lib=lib)
        fj, _, *_ = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=1.0, max_iter=2 * k - 1, lib=lib)
        _, gj, *_ = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=1.0, max_iter=2 * k, lib=lib)
        assert np.allclose(fj, fa, rtol=0, atol=1e-12), k
        assert np.allclose(gj, ga, rtol=0, atol=1e-12), k


def pin_jacobi_fixed_point(lib):
    """Blended Jacobi converges to the matrix-scaling plan (the fixed point does not depend on alpha)."""
    x, y, a, b = _problem(7, 9, 2, 191)
    eps = 0.5
    _, _, P = _scaling_form(x, y, a, b, eps, 4000)
    for alpha in (0.5, 0.3, 0.8):
        f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=alpha,
                                                  stop_mode="marginal", stop_tol=1e-13, max_iter=20000,
                                                  check_every=10, lib=lib)
        assert conv and viol <= 1e-13
        assert np.max(np.abs(_plan(x, y, a, b, f, g, eps) - P)) <= 1e-12, alpha


def pin_jacobi_symmetric_problem(lib):
    """On (x, x, a, a) both Jacobi updates are the same computation, so f equals g exactly."""
    x, _, a, _ = _problem(11, 11, 2, 201)
    for k in (1, 4, 17):
        f, g, *_ = oracle.sinkhorn_ex(x, x, a, a, 0.2, variant="symmetric", alpha=0.5, max_iter=k, lib=lib)
        assert np.array_equal(f, g)


def pin_stop_fixed(lib):
    """Fixed stop: exactly max_iter alternating iterations, no check values."""
    x, y, a, b = _problem(8, 7, 2, 211)
    f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, 0.2, max_iter=13, lib=lib)
    f0, g0, _ = oracle.sinkhorn(x, y, a, b, 0.2, 13, lib=lib)
    assert it == 13 and conv is None and math.isnan(viol)
    assert np.array_equal(f, f0) and np.array_equal(g, g0)


def pin_stop_marginal(lib):
    """Marginal stop: the first check (every c-th iteration, and the last) whose residual is <= tol,
    judged against the residual trace of the fixed-count run (pinned above)."""
    x, y, a, b = _problem(9, 8, 2, 221)
    eps, c = 0.2, 4
    _, _, tr = oracle.sinkhorn(x, y, a, b, eps, 60, check_every=c, lib=lib)
    assert np.all(np.diff(tr) < 0)
    for k_star in (1, 3, 12):
        tol = math.sqrt(tr[k_star - 1] * tr[k_star - 2]) if k_star > 1 else tr[0] * 1.5
        f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, stop_mode="marginal", stop_tol=tol,
                                                  max_iter=400, check_every=c, lib=lib)
        assert conv and it == c * k_star, (k_star, it)
        assert viol == pytest.approx(tr[k_star - 1], rel=1e-12)
        f0, g0, _ = oracle.sinkhorn(x, y, a, b, eps, it, lib=lib)
        assert np.array_equal(f, f0) and np.array_equal(g, g0)
    # unreachable tolerance: runs to the cap, checking after the last iteration as well
    f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, stop_mode="marginal", stop_tol=0.0,
                                              max_iter=10, check_every=c, lib=lib)
    f0, g0, _ = oracle.sinkhorn(x, y, a, b, eps, 10, lib=lib)
    r = oracle.residual(x, y, a, b, f0, g0, eps, lib=lib)
    assert it == 10 and conv is False and viol == pytest.approx(max(r[0], r[1]), rel=1e-12)


def pin_stop_potential(lib):
    """Potential stop: the change max(|f - f'|, |g - g'|) since the previous check (zero potentials
    before the first) falls strictly below tol."""
    x, y, a, b = _problem(9, 8, 2, 231)
    eps, c = 0.2, 3
    runs = [oracle.sinkhorn(x, y, a, b, eps, k, lib=lib)[:2] for k in range(0, 61, c)]
    runs[0] = (np.zeros(9), np.zeros(8))
    delta = [max(np.abs(runs[i][0] - runs[i - 1][0]).max(), np.abs(runs[i][1] - runs[i - 1][1]).max())
             for i in range(1, len(runs))]
    assert np.all(np.diff(delta[1:]) < 0)
    for k_star in (2, 5, 11):
        tol = math.sqrt(delta[k_star - 1] * delta[k_star - 2])
        f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, stop_mode="potential", stop_tol=tol,
                                                  max_iter=60, check_every=c, lib=lib)
        assert conv and it == c * k_star, (k_star, it)
        assert viol == pytest.approx(delta[k_star - 1], rel=1e-12)
    # max_iter not a multiple of the interval: the last check compares against iteration 6
    f, g, it, conv, viol = oracle.sinkhorn_ex(x, y, a, b, eps, stop_mode="potential", stop_tol=0.0,
                                              max_iter=8, check_every=c, lib=lib)
    f8, g8, _ = oracle.sinkhorn(x, y, a, b, eps, 8, lib=lib)
    want = max(np.abs(f8 - runs[2][0]).max(), np.abs(g8 - runs[2][1]).max())
    assert it == 8 and conv is False and viol == pytest.approx(want, rel=1e-12)


def pin_divergence_dirac(lib):
    """One point each: OT(x,y) = |x - y|^2 after one iteration, the self-terms vanish."""
    x = np.array([[0.3, -1.2, 0.5]])
    y = np.array([[1.1, 0.4, -0.7]])
    one = np.ones(1)
    for variant in ("alternating", "symmetric"):
        S, (txy, txx, tyy) = oracle.divergence(x, y, one, one, 0.7, 1 if variant == "alternating" else 200,
                                               variant=variant, alpha=0.5, lib=lib)
        want = float(((x - y) ** 2).sum())
        assert abs(txx) <= 1e-12 and abs(tyy) <= 1e-12
        assert S == pytest.approx(want, rel=1e-12, abs=1e-12)


def pin_divergence_translation(lib):
    """S(x, x + t) = |t|^2 for unit mass: the translated cost differs by a separable term whose
    integral is |t|^2, the self-terms are translation invariant; S(x, x) = 0 exactly."""
    x, _, a, _ = _problem(12, 12, 2, 241)
    t = np.array([0.35, -0.2])
    for variant in ("alternating", "symmetric"):
        S, _ = oracle.divergence(x, x + t, a, a, 1.0, 3000, variant=variant, lib=lib)
        assert S == pytest.approx(t @ t, abs=1e-10), variant
        S0, _ = oracle.divergence(x, x, a, a, 0.3, 50, variant=variant, lib=lib)
        assert S0 == 0.0


def pin_divergence_symmetric_positive(lib):
    """At convergence S(x,y) = S(y,x) and S > 0 for distinct measures (different sizes)."""
    x, y, a, b = _problem(10, 7, 2, 251)
    Sxy, (txy, _, _) = oracle.divergence(x, y, a, b, 0.25, 4000, lib=lib)
    Syx, (tyx, _, _) = oracle.divergence(y, x, b, a, 0.25, 4000, lib=lib)
    assert abs(txy - tyx) <= 1e-10 and abs(Sxy - Syx) <= 1e-10
    assert Sxy > 0.0


# ---- gradient flow (SinkSLOT README, Gradient Flow)
def pin_flow_single_target(lib):
    """One target point: w_i1 = 1, so grad_i = 2 a_i (x_i - y) and each point decays geometrically,
    x_i^K - y = (1 - 2 lr a_i)^K (x_i^0 - y); the cost at step k is sum_i a_i |x_i^k - y|^2."""
    rng = np.random.default_rng(261)
    x0 = rng.normal(size=(7, 3))
    y = np.array([[0.4, -0.2, 1.1]])
    a = rng.exponential(size=7)
    a /= a.sum()
    lr, K = 0.3, 6
    xK, trace, f, g, grad = oracle.gradient_flow(x0, y, a, np.ones(1), 0.2, 4, K, lr, lib=lib)
    decay = (1.0 - 2.0 * lr * a)[:, None]
    assert np.allclose(xK - y, decay ** K * (x0 - y), rtol=0, atol=1e-13)
    for k in range(K):
        xk = y + decay ** k * (x0 - y)
        assert trace[k] == pytest.approx((a * ((xk - y) ** 2).sum(axis=1)).sum(), rel=1e-12)
    x_last = y + decay ** (K - 1) * (x0 - y)
    assert np.allclose(grad, 2 * a[:, None] * (x_last - y), rtol=0, atol=1e-13)


def pin_flow_steps_compose(lib):
    """Two steps equal two explicit moves, each with its own solve from g = 0 (no warm start);
    the returned f, g, grad are the last step's."""
    x0, y, a, b = _problem(8, 6, 2, 271)
    eps, iters, lr = 0.3, 3, 0.7
    x = x0.copy()
    for _ in range(2):
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters, lib=lib)
        grad = oracle.grad_x(x, y, a, b, g, eps, lib=lib)
        x_prev, x = x, x - lr * grad
    xK, trace, fK, gK, gradK = oracle.gradient_flow(x0, y, a, b, eps, iters, 2, lr, lib=lib)
    assert np.allclose(xK, x, rtol=0, atol=1e-13)
    assert np.allclose(fK, f, rtol=0, atol=1e-13) and np.allclose(gK, g, rtol=0, atol=1e-13)
    assert np.allclose(gradK, grad, rtol=0, atol=1e-13)
    assert trace[1] == pytest.approx(oracle.dual_cost(x_prev, y, a, b, f, g, eps, lib=lib), rel=1e-12)


def pin_flow_mean_converged(lib):
    """Uniform weights and converged solves: the plan's column sums are b, so the gradients sum to
    2 (mean x - mean y) and the mean gap shrinks by exactly (1 - 2 lr / n) per step."""
    rng = np.random.default_rng(281)
    n, m = 6, 5
    x0 = rng.normal(size=(n, 2))
    y = rng.normal(size=(m, 2)) + 1.5
    a, b = np.full(n, 1 / n), np.full(m, 1 / m)
    lr, K = 0.5, 4
    xK, *_ = oracle.gradient_flow(x0, y, a, b, 2.0, 3000, K, lr, lib=lib)
    gap0 = x0.mean(axis=0) - y.mean(axis=0)
    assert np.allclose(xK.mean(axis=0) - y.mean(axis=0), (1 - 2 * lr / n) ** K * gap0, rtol=0, atol=1e-12)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


def test_sampled_rows_match_full():
    """Restricting the half-step to a row subset gives bit-identical values (rows are
    reduced independently and in index order, whatever the threading)."""
    x, y, a, b = _problem(33, 29, 2, 171)
    f, g, _ = oracle.sinkhorn(x, y, a, b, 0.1, 5)
    g4 = oracle.sinkhorn(x, y, a, b, 0.1, 4)[1]
    f_rows = np.array([oracle.half_step(x, y, b, g4, 0.1, idx=[i])[0] for i in range(33)])
    assert np.array_equal(f_rows, f)
    g_cols = oracle.half_step(y, x, a, f, 0.1, idx=np.arange(29)[::-1])
    assert np.array_equal(g_cols[::-1], g)


# --------------------------------------------------------------------------- mutation check
ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "sk_oracle.c")

MUTANTS = {
    "g_init_ignored": ("g[j] = g_init ? g_init[j] : 0.0;", "g[j] = 0.0;", 1),
    "primal_kl_no_mass": ("double kl = p > 0.0 ? p * log(p / q) - p + q : q;",
                          "double kl = p > 0.0 ? p * log(p / q) : 0.0;", 1),
    "primal_kl_sign": ("obj += p * c + eps * kl;", "obj += p * c - eps * kl;", 1),
    "l1_cost": ("s += diff * diff;", "s += fabs(diff);", 1),
    "cost_sign": ("(pot[j] - sq_dist(p, key + j * d, d)) / eps", "(pot[j] + sq_dist(p, key + j * d, d)) / eps", 2),
    "weight_sign": ("/ eps + logw[j];", "/ eps - logw[j];", 4),
    "eps_times": ("/ eps + logw[j];", "* eps + logw[j];", 4),
    "dropped_max": ("return -eps * (zmax + log(s));", "return -eps * log(s);", 1),
    "raw_weight": ("return w > 0.0 ? log(w) : -INFINITY;", "return w;", 1),
    "wrong_coord": ("double diff = p[t] - q[t];", "double diff = p[t] - q[0];", 1),
    "g_first": ("        oracle_half_step(x, n, y, m, d, b, g, eps, NULL, n, f);\n"
                "        oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, g);",
                "        oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, g);\n"
                "        oracle_half_step(x, n, y, m, d, b, g, eps, NULL, n, f);", 1),
    "grad_no_weight": ("2.0 * a[i] * (xi[t] - bary[t] / s)", "2.0 * (xi[t] - bary[t] / s)", 1),
    "grad_sign": ("2.0 * a[i] * (xi[t] - bary[t] / s)", "2.0 * a[i] * (bary[t] / s - xi[t])", 1),
    "grad_unnormalised": ("2.0 * a[i] * (xi[t] - bary[t] / s)", "2.0 * a[i] * (xi[t] - bary[t])", 1),
    "grad_half": ("2.0 * a[i] * (xi[t] - bary[t] / s)", "a[i] * (xi[t] - bary[t] / s)", 1),
    "marginal_drop_a": ("            s += a[i] * b[j] * exp(", "            s += b[j] * exp(", 2, 1),
    "dual_sign": ("return af + bg - eps * (mass_p - sa * sb);", "return af + bg + eps * (mass_p - sa * sb);", 1),
    "dual_no_mass": ("return af + bg - eps * (mass_p - sa * sb);", "return af + bg - eps * mass_p;", 1),
    "resid_no_abs": ("double e = fabs(rs[i] - a[i]);", "double e = rs[i] - a[i];", 1),
    "jacobi_new_f": ("oracle_half_step(y, m, x, n, d, a, f, eps, NULL, m, gn);",
                     "oracle_half_step(y, m, x, n, d, a, fn, eps, NULL, m, gn);", 1),
    "alpha_swap": ("f[i] = (1.0 - alpha) * f[i] + alpha * fn[i];", "f[i] = alpha * f[i] + (1.0 - alpha) * fn[i];", 1),
    "potential_no_snapshot": ("                fp[i] = f[i];\n", "", 1),
    "check_phase": ("k % check_every != 0", "(k + 1) % check_every != 0", 1),
    "no_last_check": (" && k != max_iter", "", 1),
    "marginal_col_only": ("viol = r[0] > r[1] ? r[0] : r[1];", "viol = r[1];", 1),
    "div_full_self": ("out[0] = t_xy - 0.5 * t_xx - 0.5 * t_yy;", "out[0] = t_xy - t_xx - t_yy;", 1),
    "div_self_x_twice": ("oracle_sinkhorn_ex(y, y, b, b, m, m,", "oracle_sinkhorn_ex(x, x, a, a, n, n,", 1),
    "flow_warm_start": ("oracle_sinkhorn(x, y, a, b, n, m, d, eps, n_iters, 0, NULL, f, g, NULL);",
                        "oracle_sinkhorn(x, y, a, b, n, m, d, eps, n_iters, 0, k ? g : NULL, f, g, NULL);", 1),
    "flow_ascent": ("x[e] -= lr * grad[e];", "x[e] += lr * grad[e];", 1),
    "flow_cost_after_move": ("        if (cost_trace)\n            cost_trace[k] = oracle_dual_cost(x, y, a, b, n, m, d, eps, f, g);\n"
                             "        oracle_grad_x(x, y, a, b, n, m, d, eps, g, NULL, n, grad);\n"
                             "        for (int64_t e = 0; e < n * d; ++e)\n            x[e] -= lr * grad[e];",
                             "        oracle_grad_x(x, y, a, b, n, m, d, eps, g, NULL, n, grad);\n"
                             "        for (int64_t e = 0; e < n * d; ++e)\n            x[e] -= lr * grad[e];\n"
                             "        if (cost_trace)\n            cost_trace[k] = oracle_dual_cost(x, y, a, b, n, m, d, eps, f, g);", 1),
    "trace_row_only": ("resid_trace[k / check_every - 1] = r[0] > r[1] ? r[0] : r[1];",
                       "resid_trace[k / check_every - 1] = r[1];", 1),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new, count, *n_replace = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == count, f"mutation site for {name} not found exactly {count} time(s)"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, *n_replace))
    lib = oracle.load(oracle.build(str(mutated), str(tmp_path / "libmutant.so")))
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
