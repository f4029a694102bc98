"""Writes the stored oracle results for the full-size workloads.

Calls only the CPU oracle (``oracle/``) on the seeded inputs of ``sk_inputs``;
nothing here comes from the GPU library.  Each workload gets
``tests/golden/<name>.npz`` holding the float64 potentials after the full
fixed iteration count, the dual cost, the final marginal residual, the
residual trace (when the workload checks it), the gradient (when it asks for
one), max C, the float32 eps used and a SHA-256 digest of the inputs so a test
can tell if the generator ever drifts.

``gflow_d2_flow`` is the gradient flow on the gflow_d2 problem (SinkSLOT
README, Gradient Flow): FLOW_STEPS steps of x <- x - FLOW_LR grad, each at a
fresh solve of the workload's iteration count; it stores the final x, the
per-step cost trace and the last step's f, g and gradient.

Usage: python tests/golden/make_golden.py [name ...]   (default: the four
workloads whose full trajectories the oracle can finish on a CPU, and the
gradient flow).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from sk_inputs import WORKLOADS, digest, eps32, make_inputs  # noqa: E402

DEFAULT = ["gflow_d2", "gauss_d2", "gmm8_d3", "gauss_d64", "gflow_d2_flow"]
FLOW_STEPS, FLOW_LR = 200, 0.1


def make_flow(name: str = "gflow_d2_flow") -> str:
    w = WORKLOADS["gflow_d2"]
    x, y, a, b = make_inputs("gflow_d2")
    eps = eps32(w.eps)
    t0 = time.time()
    xK, trace, f, g, grad = oracle.gradient_flow(x, y, a, b, eps, w.n_iters, FLOW_STEPS, FLOW_LR)
    out = dict(x=xK, cost_trace=trace, f=f, g=g, grad=grad, eps=np.float64(eps), n_iters=np.int64(w.n_iters),
               n_steps=np.int64(FLOW_STEPS), lr=np.float64(FLOW_LR), digest=np.array(digest(x, y, a, b)),
               max_cost=np.float64(oracle.max_cost(x, y)))
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: {time.time() - t0:.1f} s -> {path}", flush=True)
    return path


def make(name: str) -> str:
    w = WORKLOADS[name]
    x, y, a, b = make_inputs(name)
    eps = eps32(w.eps)
    t0 = time.time()
    f, g, trace = oracle.sinkhorn(x, y, a, b, eps, w.n_iters, check_every=w.check_every)
    out = dict(f=f, g=g, trace=trace, eps=np.float64(eps), n_iters=np.int64(w.n_iters),
               check_every=np.int64(w.check_every), digest=np.array(digest(x, y, a, b)),
               cost=np.float64(oracle.dual_cost(x, y, a, b, f, g, eps)),
               residual=oracle.residual(x, y, a, b, f, g, eps),
               max_cost=np.float64(oracle.max_cost(x, y)))
    if w.grad:
        out["grad"] = oracle.grad_x(x, y, a, b, g, eps)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: {time.time() - t0:.1f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for nm in (sys.argv[1:] or DEFAULT):
        make_flow(nm) if nm == "gflow_d2_flow" else make(nm)
