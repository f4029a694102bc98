"""GPU parity of the gradient flow (SinkSLOT README, Gradient Flow): n_steps of
x <- x - lr grad_x, each at a fresh fixed-count solve, through the C ABI.

Tolerances
  * against the library's own step-by-step composition (sk_solve, sk_grad_x and
    the move done by torch): the only difference is the rounding of the move,
    a few float32 ulps of |x| per step;
  * against the float64 oracle: the potentials and costs of the last step to the
    solve's bounds (1e-4 max C, relative 1e-4); x to the sum over steps of lr
    times the per-step gradient bound, which the observed potential error delta
    sets as in the end-to-end gradient check: 2 max(a) sqrt(max C)
    (16 kappa + 2 expm1(2 delta / eps)) per step, doubled for the propagation
    through later steps (the flow with these step sizes is a contraction up to
    that factor).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from sk_inputs import WORKLOADS, digest, eps32, make_inputs, random_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U32 = 2.0 ** -24
GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "gflow_d2_flow.npz")


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in arrs]


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def x_bound(a, maxc, eps, f, g, delta, lr, steps):
    kappa = U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps
    per_step = 2 * a.max() * math.sqrt(maxc) * (16 * kappa + 2 * math.expm1(2 * delta / eps))
    return 2 * lr * steps * per_step


FLOW_CASES = [
    # n, m, d, eps, n_iters, n_steps, lr, seed
    (300, 257, 2, 0.05, 30, 20, 0.1, 1),
    (700, 900, 3, 0.1, 20, 10, 0.5, 2),
    (400, 300, 64, 0.5, 10, 8, 0.2, 3),
    (1, 5, 2, 0.1, 5, 6, 0.3, 4),
]


@pytest.mark.parametrize("case", FLOW_CASES, ids=[f"{c[0]}x{c[1]}d{c[2]}" for c in FLOW_CASES])
def test_flow_matches_composition_and_oracle(case):
    n, m, d, eps, iters, steps, lr, seed = case
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.5)
    eps = eps32(eps)
    say("flow", case)
    X, Y, A, B = dev(x, y, a, b)
    X0 = X.clone()
    Xf, f_t, g_t, gr_t, tr_t = sk.gradient_flow(X, Y, A, B, eps=eps, n_iters=iters, n_steps=steps, lr=lr)
    assert Xf.data_ptr() == X.data_ptr()
    xg, f, g, grad, trace = host(Xf), host(f_t), host(g_t), host(gr_t), host(tr_t)
    # the library's own composition, step by step
    Xc = X0.clone()
    for _ in range(steps):
        fc, gc, _ = sk.solve(Xc, Y, A, B, eps=eps, n_iters=iters)
        gr = sk.grad_x(Xc, Y, A, B, gc, eps=eps)
        Xc = Xc - lr * gr
    xc = host(Xc)
    ulp_tol = 8 * steps * U32 * max(np.abs(xc).max(), 1.0)
    say("composition diff", np.abs(xg - xc).max(), "tol", ulp_tol)
    assert np.abs(xg - xc).max() <= ulp_tol
    # the oracle
    xo, tro, fo, go, gro = oracle.gradient_flow(x, y, a, b, eps, iters, steps, lr)
    maxc = oracle.max_cost(x, y)
    delta = max(np.abs(f - fo).max(), np.abs(g - go).max())
    tol_x = x_bound(a, maxc, eps, f, g, delta, lr, steps)
    say("x err", np.abs(xg - xo).max(), "bound", tol_x, "delta/maxC", delta / maxc,
        "moved", np.abs(xo - x).max())
    assert delta <= 1e-4 * maxc
    assert np.abs(xg - xo).max() <= tol_x
    assert np.allclose(trace, tro, rtol=1e-4, atol=1e-12)


def test_flow_zero_steps_and_graph_replay():
    x, y, a, b = random_problem(500, 400, 2, 11, shift=0.5)
    eps = eps32(0.05)
    X, Y, A, B = dev(x, y, a, b)
    X0 = X.clone()
    sk.gradient_flow(X, Y, A, B, eps=eps, n_iters=10, n_steps=0, lr=0.1)
    assert torch.equal(X, X0)
    # one flow step captured and replayed equals the eager flow of as many steps
    ws = sk.workspace(500, 400, 2, X.device)
    f, g = torch.empty(500, device=DEV), torch.empty(400, device=DEV)
    gr = torch.empty((500, 2), device=DEV)
    tr = torch.empty(1, dtype=torch.float64, device=DEV)
    Xe = X0.clone()
    sk.gradient_flow(Xe, Y, A, B, eps=eps, n_iters=10, n_steps=4, lr=0.1, ws=ws, f=f, g=g, grad=gr, check=False)
    torch.cuda.synchronize()
    want = Xe.clone()
    Xg = X0.clone()
    sk.gradient_flow(Xg, Y, A, B, eps=eps, n_iters=10, n_steps=1, lr=0.1, ws=ws, f=f, g=g, grad=gr, cost_trace=tr,
                     check=False)  # warm-up outside capture
    Xg.copy_(X0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sk.gradient_flow(Xg, Y, A, B, eps=eps, n_iters=10, n_steps=1, lr=0.1, ws=ws, f=f, g=g, grad=gr,
                         cost_trace=tr, check=False)
    Xg.copy_(X0)
    torch.cuda.synchronize()
    for _ in range(4):
        graph.replay()
        torch.cuda.synchronize()
        _ = (Y * 2.0).sum().item()  # unrelated eager work between replays
    assert torch.equal(Xg, want)


def test_gradient_flow_workload_against_stored_oracle():
    """The 1000-point problem, 200 flow steps of 200 iterations each, lr = 0.1, against the stored
    oracle trajectory (tests/golden/make_golden.py)."""
    gold = np.load(GOLDEN)
    w = WORKLOADS["gflow_d2"]
    x, y, a, b = make_inputs("gflow_d2")
    assert str(gold["digest"]) == digest(x, y, a, b)
    eps = eps32(w.eps)
    assert float(gold["eps"]) == eps
    steps, lr, iters = int(gold["n_steps"]), float(gold["lr"]), int(gold["n_iters"])
    say("gflow_d2 flow", steps, "steps")
    X, Y, A, B = dev(x, y, a, b)
    Xf, f_t, g_t, gr_t, tr_t = sk.gradient_flow(X, Y, A, B, eps=eps, n_iters=iters, n_steps=steps, lr=lr)
    xg, f, g, trace = host(Xf), host(f_t), host(g_t), host(tr_t)
    maxc = float(gold["max_cost"])
    delta = max(np.abs(f - gold["f"]).max(), np.abs(g - gold["g"]).max())
    tol_x = x_bound(a, maxc, eps, f, g, delta, lr, steps)
    say("x err", np.abs(xg - gold["x"]).max(), "bound", tol_x, "delta/maxC", delta / maxc,
        "moved", np.abs(gold["x"] - x).max())
    assert delta <= 1e-4 * maxc
    assert np.abs(xg - gold["x"]).max() <= tol_x
    assert np.allclose(trace, gold["cost_trace"], rtol=1e-4, atol=1e-12)
