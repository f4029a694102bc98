"""Writes the stored oracle results for the full-size workloads.

Calls only the CPU oracle (``oracle/``) on the seeded inputs of ``sk_inputs``;
nothing here comes from the GPU library.  Each workload gets
``tests/golden/<name>.npz`` holding the float64 potentials after the full
fixed iteration count, the dual cost, the final marginal residual, the
residual trace (when the workload checks it), the gradient (when it asks for
one), max C, the float32 eps used and a SHA-256 digest of the inputs so a test
can tell if the generator ever drifts.

Usage: python tests/golden/make_golden.py [name ...]   (default: the four
workloads whose full trajectories the oracle can finish on a CPU).
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

DEFAULT = ["gflow_d2", "gauss_d2", "gmm8_d3", "gauss_d64"]


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
        make(nm)
