"""GPU parity at the full workload sizes.

* Full trajectories (gflow_d2, gauss_d2, gmm8_d3, gauss_d64): the GPU solve
  with the workload's iteration count against the oracle results stored in
  tests/golden/ (written by tests/golden/make_golden.py, which calls only the
  oracle).  The inputs are regenerated from their seeds and checked against the
  stored digest first.
* Sampled single steps (gmm8_d3_sq -- the benchmark workload, in the launch
  configuration bench.py times -- and cluster_d3 with 2^20 points): runs with
  k-1 and k iterations are prefixes of one deterministic trajectory, so the
  oracle can recompute f_k on sampled rows from the GPU's g_{k-1} and g_k on
  sampled columns from the GPU's f_k.  Each half-step is 1-Lipschitz in the
  sup norm, so if every row and column of every step were within
  1e-4 max C / (2K), the K-iteration trajectory would stay within 1e-4 max C.
  This is a statistical, per-step check: it bounds the sampled rows and
  columns of the steps it visits (the last step of gmm8_d3_sq; steps 1, 2, 10,
  25 and 50 of cluster_d3), not every row of every step.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from sk_inputs import WORKLOADS, digest, eps32, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in arrs]


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["gflow_d2", "gauss_d2", "gmm8_d3", "gauss_d64"])
def test_full_trajectory_against_stored_oracle(name):
    w = WORKLOADS[name]
    gold = np.load(os.path.join(GOLDEN, f"{name}.npz"))
    x, y, a, b = make_inputs(name)
    assert str(gold["digest"]) == digest(x, y, a, b), "input generator drifted from the stored oracle run"
    eps = eps32(w.eps)
    assert float(gold["eps"]) == eps and int(gold["n_iters"]) == w.n_iters
    say("full trajectory", name, w.n, w.m, w.d, w.n_iters)
    X, Y, A, B = dev(x, y, a, b)
    f_t, g_t, tr_t = sk.solve(X, Y, A, B, eps=eps, n_iters=w.n_iters, check_every=w.check_every)
    c_t = sk.cost(A, B, f_t, g_t, eps=eps)
    f, g, tr, c = host(f_t), host(g_t), host(tr_t), float(host(c_t)[0])
    maxc = float(gold["max_cost"])
    df, dg = np.max(np.abs(f - gold["f"])), np.max(np.abs(g - gold["g"]))
    say(name, "max|df|/tol", df / (1e-4 * maxc), "max|dg|/tol", dg / (1e-4 * maxc),
        "cost rel", abs(c - float(gold["cost"])) / abs(float(gold["cost"])))
    assert df <= 1e-4 * maxc and dg <= 1e-4 * maxc
    assert abs(c - float(gold["cost"])) <= 1e-4 * abs(float(gold["cost"]))
    if w.check_every:
        want = gold["trace"]
        assert tr.shape == want.shape
        # trajectory difference delta moves each plan exponent by at most 2 delta / eps
        kap = U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps
        bound = (a.max() + want) * (math.expm1(2 * max(df, dg) / eps) + 32 * kap)
        say(name, "trace err/bound", np.max(np.abs(tr - want) / bound))
        assert np.all(np.abs(tr - want) <= bound)
    if w.grad:
        grad = host(sk.grad_x(X, Y, A, B, g_t, eps=eps))
        kap = U32 * (np.abs(g).max() + maxc) / eps
        bound = 2 * a.max() * math.sqrt(maxc) * (16 * kap + 2 * math.expm1(2 * dg / eps))
        say(name, "grad err/bound", np.max(np.abs(grad - gold["grad"])) / bound)
        assert np.max(np.abs(grad - gold["grad"])) <= bound


def _sampled_step_check(name, n_sample, seed):
    w = WORKLOADS[name]
    K = w.n_iters
    x, y, a, b = make_inputs(name)
    eps = eps32(w.eps)
    X, Y, A, B = dev(x, y, a, b)
    ws = sk.workspace(w.n, w.m, w.d, X.device)
    say("sampled step", name, "K-1 =", K - 1)
    _, g_prev, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=K - 1, ws=ws)
    g_prev = host(g_prev)
    say("sampled step", name, "K =", K)
    f_t, g_t, tr_t = sk.solve(X, Y, A, B, eps=eps, n_iters=K, check_every=w.check_every, ws=ws)
    f, g, tr = host(f_t), host(g_t), host(tr_t)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    maxc = oracle.max_cost(x, y) if w.n * w.m <= 4e9 else oracle.max_cost_hull(x, y)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.n, n_sample, replace=False))
    cols = np.sort(rng.choice(w.m, n_sample, replace=False))
    say("oracle rows", name)
    f_or = oracle.half_step(x, y, b, g_prev, eps, idx=rows)
    say("oracle cols", name)
    g_or = oracle.half_step(y, x, a, f, eps, idx=cols)
    tol = 1e-4 * maxc / (2 * K)
    e_f, e_g = np.max(np.abs(f[rows] - f_or)), np.max(np.abs(g[cols] - g_or))
    say(name, "row step err/tol", e_f / tol, "col step err/tol", e_g / tol)
    assert e_f <= tol and e_g <= tol
    return x, y, a, b, f, g, g_t, tr, eps, maxc, rows, X, Y, A, B


def test_sampled_steps_benchmark_workload():
    """n = m = 50,000, d = 3, 100 iterations with the residual every 10 (as bench.py runs it)."""
    x, y, a, b, f, g, g_t, tr, eps, maxc, rows, X, Y, A, B = _sampled_step_check("gmm8_d3_sq", 2048, 7)
    # the fused residual after the last iteration equals the oracle's residual of the GPU's (f, g)
    say("oracle residual 50k x 50k")
    ro = oracle.residual(x, y, a, b, f, g, eps)
    kap = U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps
    assert abs(tr[-1] - max(ro[0], ro[1])) <= 32 * kap * (a.max() + ro[0])
    # gradient at the GPU's g, sampled rows
    grad = host(sk.grad_x(X, Y, A, B, g_t, eps=eps))
    gr = oracle.grad_x(x, y, a, b, g, eps, idx=rows)
    kap_g = U32 * (np.abs(g).max() + maxc) / eps
    assert np.max(np.abs(grad[rows] - gr)) <= 2 * a.max() * 16 * kap_g * math.sqrt(maxc)


def test_sampled_steps_clustered_million():
    """2^20 x 2^20 clustered clouds, eps = (n^(-1/3))^2, 50 iterations, then grad_x and the cost.

    Steps k = 1, 2, 10, 25 and 50 of the 50-iteration trajectory: f_k on 4096 sampled rows from the GPU's
    g_{k-1}, g_k on 4096 sampled columns from the GPU's f_k, each within 1e-4 max C / (2 * 50); the cost of the
    final potentials against a float64 <a, f> + <b, g> of the same potentials; the gradient on sampled rows."""
    name = "cluster_d3"
    w = WORKLOADS[name]
    K, n_sample = w.n_iters, 4096
    x, y, a, b = make_inputs(name)
    eps = eps32(w.eps)
    X, Y, A, B = dev(x, y, a, b)
    ws = sk.workspace(w.n, w.m, w.d, X.device)
    say("cluster max C (hull)")
    maxc = oracle.max_cost_hull(x, y)
    rng = np.random.default_rng(11)
    tol = 1e-4 * maxc / (2 * K)
    g_prev = np.zeros(w.m)
    done = 0
    for k in (1, 2, 10, 25, 50):
        if k - 1 > done:
            say(name, "solve", k - 1)
            _, gp_t, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=k - 1, ws=ws)
            g_prev = host(gp_t)
        say(name, "solve", k)
        f_t, g_t, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=k, ws=ws)
        f, g = host(f_t), host(g_t)
        done = k
        assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
        rows = np.sort(rng.choice(w.n, n_sample, replace=False))
        cols = np.sort(rng.choice(w.m, n_sample, replace=False))
        say(name, "oracle rows and columns of step", k)
        f_or = oracle.half_step(x, y, b, g_prev, eps, idx=rows)
        g_or = oracle.half_step(y, x, a, f, eps, idx=cols)
        e_f, e_g = np.max(np.abs(f[rows] - f_or)), np.max(np.abs(g[cols] - g_or))
        say(name, "step", k, "row err/tol", e_f / tol, "col err/tol", e_g / tol)
        assert e_f <= tol and e_g <= tol, (k, e_f / tol, e_g / tol)
        g_prev = g
    # cost of the final potentials: the float64 dual sum over all 2^21 points
    c = float(host(sk.cost(A, B, f_t, g_t, eps=eps))[0])
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    c_ref = float(np.dot(a64, f) + np.dot(b64, g) - eps * b64.sum() * (1.0 - a64.sum()))
    say(name, "cost rel err", abs(c - c_ref) / abs(c_ref))
    assert abs(c - c_ref) <= 1e-4 * abs(c_ref)
    grad = host(sk.grad_x(X, Y, A, B, g_t, eps=eps))
    assert np.all(np.isfinite(grad))
    say("oracle grad rows")
    gr = oracle.grad_x(x, y, a, b, g, eps, idx=rows)
    kap_g = U32 * (np.abs(g).max() + maxc) / eps
    err = np.max(np.abs(grad[rows] - gr))
    say("cluster grad err/bound", err / (2 * a.max() * 16 * kap_g * math.sqrt(maxc)))
    assert err <= 2 * a.max() * 16 * kap_g * math.sqrt(maxc)
