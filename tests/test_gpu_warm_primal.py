"""GPU parity of the warm-started solve (SinkSLOT README, Low-Level Solver API:
the solver state is the pair of potentials) and of the plan's primal value
(SinkSLOT README, Basic Usage: the loss reports the primal value of its plan)
against the CPU float64 oracle, through the C ABI.

Tolerances
  * warm-started potentials after the same iterations from the same float32
    g_init: max|f - f*|, max|g - g*| <= 1e-4 max C, the solve's bar;
  * primal value at identical float32 potentials: each plan entry carries the
    float32 error of its exponent, at most 32 kappa relative (kappa = 2^-24
    (max|f| + max|g| + max C) / eps, as for the residual and the transport
    products), so |D - D*| <= 32 kappa (sum_i |f_i| r_i + sum_j |g_j| c_j +
    eps sum P) for <P,C> + eps KL = <r, f> + <c, g> - eps (sum P - mass^2), and
    |<P,C> - <P,C>*| <= 32 kappa sum_ij P_ij (|x~_i| + |y~_j|)^2 for the
    transport cost summed in the centred expanded form (x~, y~ shifted by the
    common centre), with r, c, P the oracle's.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from sk_inputs import eps32, random_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U32 = 2.0 ** -24


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in arrs]


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


WARM_CASES = [
    # n, m, d, eps, iters, seed, zero_frac, check_every
    (1, 7, 2, 0.2, 3, 1, 0.0, 0),
    (1100, 900, 2, 0.05, 12, 2, 0.0, 4),
    (2000, 1700, 3, 0.02, 9, 3, 0.1, 3),
    (900, 1300, 5, 0.3, 5, 4, 0.0, 0),
    (700, 600, 64, 0.5, 6, 5, 0.05, 2),
    (300, 500, 130, 0.5, 4, 6, 0.0, 0),
]


@pytest.mark.parametrize("case", WARM_CASES, ids=["%dx%dd%d" % c[:3] for c in WARM_CASES])
def test_warm_start_matches_oracle(case):
    n, m, d, eps, iters, seed, zf, ce = case
    say("warm", case)
    x, y, a, b = random_problem(n, m, d, seed, zero_frac=zf)
    eps = eps32(eps)
    g0 = (eps * np.random.default_rng(seed + 100).normal(size=m) * 3.0).astype(np.float32)
    X, Y, A, B, G0 = dev(x, y, a, b, g0)
    f_t, g_t, tr_t = sk.solve_warm(X, Y, A, B, eps=eps, n_iters=iters, g_init=G0, check_every=ce)
    f, g = host(f_t), host(g_t)
    fo, go, tro = oracle.sinkhorn(x, y, a, b, eps, iters, check_every=ce, g_init=g0.astype(np.float64))
    maxc = oracle.max_cost(x, y)
    df, dg = np.max(np.abs(f - fo)), np.max(np.abs(g - go))
    say("warm", case, "df/tol", df / (1e-4 * maxc), "dg/tol", dg / (1e-4 * maxc))
    assert df <= 1e-4 * maxc and dg <= 1e-4 * maxc
    assert torch.equal(G0, torch.from_numpy(g0).to(DEV))  # the start is not written
    if ce:
        tr = host(tr_t)
        kap = U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps
        bound = (a.max() + tro) * (math.expm1(2 * max(df, dg) / eps) + 32 * kap)
        assert tr.shape == tro.shape and np.all(np.abs(tr - tro) <= bound)


@pytest.mark.parametrize("d", [3, 64])
def test_warm_start_continues_in_place(d):
    """k1 iterations, then k2 more from the resulting g updated in place, follow the (k1 + k2)-iteration
    trajectory: both against the oracle's k1 + k2 iterations from 0, to the solve's bar."""
    x, y, a, b = random_problem(1500, 1200, d, 21 + d)
    eps = eps32(0.05 if d == 3 else 0.5)
    X, Y, A, B = dev(x, y, a, b)
    ws = sk.workspace(1500, 1200, d, X.device)
    f_t, g_t, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=7, ws=ws)
    f_t, g_t, _ = sk.solve_warm(X, Y, A, B, eps=eps, n_iters=5, g_init=g_t, ws=ws, f=f_t, g=g_t)
    f12, g12, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=12, ws=ws)
    fo, go, _ = oracle.sinkhorn(x, y, a, b, eps, 12)
    tol = 1e-4 * oracle.max_cost(x, y)
    for ff, gg in ((host(f_t), host(g_t)), (host(f12), host(g12))):
        assert np.max(np.abs(ff - fo)) <= tol and np.max(np.abs(gg - go)) <= tol
    # the hand-over differs from the uninterrupted run only by the float32 rounding of the state
    say("continue d", d, "max|f_warm - f_12| / tol", np.max(np.abs(host(f_t) - host(f12))) / tol)


def test_warm_start_zero_iterations():
    x, y, a, b = random_problem(40, 30, 2, 31)
    g0 = np.linspace(-1.0, 1.0, 30).astype(np.float32)
    X, Y, A, B, G0 = dev(x, y, a, b, g0)
    f, g, _ = sk.solve_warm(X, Y, A, B, eps=0.1, n_iters=0, g_init=G0)
    assert torch.count_nonzero(f) == 0 and torch.equal(g, G0)


PRIMAL_CASES = [
    # n, m, d, eps, iters, seed, zero_frac, perturb (x eps on g: off the optimum, plan mass != 1)
    (1, 5, 2, 0.2, 3, 1, 0.0, 0.3),
    (7, 1, 3, 0.2, 3, 2, 0.0, 0.0),
    (1100, 900, 2, 0.05, 10, 3, 0.0, 0.3),
    (1300, 1000, 3, 0.02, 20, 4, 0.1, 0.5),
    (900, 1300, 5, 0.3, 5, 5, 0.0, 0.2),
    (1300, 700, 8, 0.5, 5, 6, 0.05, 0.3),
    (900, 700, 16, 0.3, 5, 7, 0.0, 0.3),
    (700, 900, 64, 0.5, 5, 8, 0.05, 0.3),
    (300, 500, 130, 0.5, 4, 9, 0.0, 0.3),
]


@pytest.mark.parametrize("case", PRIMAL_CASES, ids=["%dx%dd%d" % c[:3] for c in PRIMAL_CASES])
def test_primal_matches_oracle(case):
    n, m, d, eps, iters, seed, zf, pert = case
    say("primal", case)
    x, y, a, b = random_problem(n, m, d, seed, zero_frac=zf)
    eps = eps32(eps)
    X, Y, A, B = dev(x, y, a, b)
    f_t, g_t, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=iters)
    g_t = g_t + pert * eps * torch.from_numpy(np.random.default_rng(seed).normal(size=m).astype(np.float32)).to(DEV)
    out = host(sk.primal_cost(X, Y, A, B, f_t, g_t, eps=eps))
    f, g = host(f_t), host(g_t)
    want, want_pc = oracle.primal(x, y, a, b, f, g, eps)
    # bounds from the oracle's plan at the same potentials
    x64, y64 = x.astype(np.float64), y.astype(np.float64)
    C = ((x64[:, None, :] - y64[None, :, :]) ** 2).sum(-1)
    with np.errstate(over="ignore", divide="ignore"):
        P = a[:, None].astype(np.float64) * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)
    r, c = P.sum(1), P.sum(0)
    kap = U32 * (np.abs(f).max() + np.abs(g).max() + C.max()) / eps
    b0 = 32 * kap * (np.dot(np.abs(f), r) + np.dot(np.abs(g), c) + eps * P.sum())
    centre = 0.5 * (x64.mean(0) + y64.mean(0))
    nxs, nys = np.linalg.norm(x64 - centre, axis=1), np.linalg.norm(y64 - centre, axis=1)
    b1 = 32 * kap * (P * (nxs[:, None] + nys[None, :]) ** 2).sum()
    say("primal", case, "err/bound", abs(out[0] - want) / b0, abs(out[1] - want_pc) / b1)
    assert abs(out[0] - want) <= b0 and abs(out[1] - want_pc) <= b1


def test_primal_equals_dual_at_convergence():
    """Strong duality: at (near) convergence the primal value equals the dual cost (relative 1e-4, the cost bar),
    and the transport cost is below both by the entropic term."""
    x, y, a, b = random_problem(2000, 1800, 3, 51)
    eps = eps32(0.1)
    X, Y, A, B = dev(x, y, a, b)
    f, g, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=400)
    pr = host(sk.primal_cost(X, Y, A, B, f, g, eps=eps))
    du = float(host(sk.dual_cost(X, Y, A, B, f, g, eps=eps))[0])
    say("duality", pr, du)
    assert abs(pr[0] - du) <= 1e-4 * abs(du)
    assert pr[1] < pr[0]
