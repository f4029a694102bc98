"""A captured HIP graph of the hot path replays to the eager result.

The entry points allocate nothing, synchronise nothing and use no memset, so a
whole step (solve with residual trace, cost, gradient) can be captured and
replayed.  The graph is replayed several times with the program's own eager
work and synchronisations in between, and every replay must equal the eager
result bit for bit.
"""
import numpy as np
import pytest
import torch

import streaming_sinkhorn_solver_amd as sk
from sk_inputs import eps32, make_inputs, random_problem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["gflow_d2", "ragged_d3", "split_d40", "split_d64"])
def test_graph_replay_matches_eager(case):
    if case == "gflow_d2":
        x, y, a, b = make_inputs("gflow_d2")
        eps, iters, ce = eps32(0.01), 40, 10
    elif case == "ragged_d3":
        x, y, a, b = random_problem(2600, 1900, 3, 77)
        eps, iters, ce = eps32(0.05), 12, 4
    else:  # the matrix-core path: scale reduction, key split, split passes, gradient as transport mode 4
        d = 40 if case == "split_d40" else 64
        x, y, a, b = random_problem(1700, 2100, d, 78 + d, scale=1.0 / np.sqrt(d), shift=0.2)
        eps, iters, ce = eps32(0.3), 10, 5
    dev = torch.device("cuda:0")
    X, Y, A, B = (torch.from_numpy(v).to(dev) for v in (x, y, a, b))
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    ws = sk.workspace(n, m, d, dev)
    f = torch.empty(n, device=dev)
    g = torch.empty(m, device=dev)
    tr = torch.empty(iters // ce, device=dev)
    c = torch.empty(1, dtype=torch.float64, device=dev)
    gr = torch.empty((n, d), device=dev)

    def step():
        sk.solve(X, Y, A, B, eps=eps, n_iters=iters, check_every=ce, ws=ws, f=f, g=g, trace=tr, check=False)
        sk.cost(A, B, f, g, eps=eps, out=c)
        sk.grad_x(X, Y, A, B, g, eps=eps, ws=ws, out=gr)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (f, g, tr, c, gr)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (f, g, tr, gr):  # scribble over the outputs with eager work
            t.fill_(float("nan"))
        c.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((f, g, tr, c, gr), want):
            assert torch.equal(got, exp), f"replay {rep} differs from the eager step"
        _ = (X * 2.0).sum().item()  # unrelated eager work between replays


def test_graph_replay_symmetric_dual_cost_and_divergence():
    """Fixed-stop entry points of the other variant, the general dual cost and the
    divergence are capturable too."""
    x, y, a, b = random_problem(1900, 1400, 3, 78, shift=0.3)
    eps, iters = eps32(0.05), 9
    dev = torch.device("cuda:0")
    X, Y, A, B = (torch.from_numpy(v).to(dev) for v in (x, y, a, b))
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    ws = sk.workspace(n, m, d, dev)
    wsd = sk.divergence_workspace(n, m, d, dev)
    f = torch.empty(n, device=dev)
    g = torch.empty(m, device=dev)
    c = torch.empty(1, dtype=torch.float64, device=dev)
    dv = torch.empty(4, dtype=torch.float64, device=dev)

    def step():
        sk.solve_ex(X, Y, A, B, eps=eps, variant="symmetric", alpha=0.5, max_iter=iters, ws=ws, f=f, g=g,
                    check=False)
        sk.dual_cost(X, Y, A, B, f, g, eps=eps, ws=ws, out=c)
        sk.divergence(X, Y, A, B, eps=eps, n_iters=iters, ws=wsd, out=dv, check=False)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (f, g, c, dv)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (f, g):
            t.fill_(float("nan"))
        c.fill_(-1.0)
        dv.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((f, g, c, dv), want):
            assert torch.equal(got, exp), f"replay {rep} differs from the eager step"
        _ = (X * 2.0).sum().item()


@pytest.mark.parametrize("d", [3, 64])
def test_graph_replay_transport_and_hvp(d):
    """The transport product and the Hessian-vector product with a fixed CG step count are
    capturable (the CG's scalars live on the device; nothing synchronises)."""
    x, y, a, b = random_problem(1300, 1100, d, 79 + d, scale=1.0 / np.sqrt(d), shift=0.3)
    eps = eps32(0.2 if d == 3 else 0.5)
    dev = torch.device("cuda:0")
    X, Y, A, B = (torch.from_numpy(v).to(dev) for v in (x, y, a, b))
    n, m = x.shape[0], y.shape[0]
    F, G, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=50)
    wst = sk.transport_workspace(n, m, d, dev)
    v = torch.from_numpy(np.random.default_rng(5).normal(size=(m, 4)).astype(np.float32)).to(dev)
    u = torch.from_numpy(np.random.default_rng(6).normal(size=(n, d)).astype(np.float32)).to(dev)
    pv = torch.empty((n, 4), device=dev)
    hv = torch.empty((n, d), device=dev)
    res = torch.empty(1, device=dev)

    def step():
        sk.transport(X, Y, A, B, F, G, v, eps=eps, ws=wst, out=pv)
        sk.hvp(X, Y, A, B, F, G, u, eps=eps, cg_iters=10, ws=wst, out=hv, cg_resid=res)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (pv, hv, res)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (pv, hv, res):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((pv, hv, res), want):
            assert torch.equal(got, exp), f"replay {rep} differs from the eager step"
        _ = (X * 2.0).sum().item()
