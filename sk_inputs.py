"""Seeded synthetic point clouds for the entropic-OT workloads.

This module only draws inputs.  It holds none of the solver's arithmetic, so it
can feed both the HIP library and the CPU oracle without coupling them.

Each workload is a pair of point clouds x (n, d), y (m, d) with nonnegative
weights a (n,), b (m,), an entropic strength eps measured against the squared
Euclidean cost, and a fixed Sinkhorn iteration count.  Everything is drawn in
float64 with ``numpy.random.default_rng(seed)`` (PCG64) in the order x, y, a, b
and then cast to float32, which is the precision the GPU path computes in.

Workload shapes follow the problems on the pages:

* ``gflow_d2``   -- the gradient-flow toy problem of the SinkSLOT README
  ("Gradient Flow" example): 1000 points, y shifted by +3, eps = 0.01.
* ``gauss_d2``   -- the SinkSLOT README's "Basic Usage" problem: two 10,000-point
  standard Gaussian clouds in 2-D, eps = 0.05, 200 iterations.
* ``gmm8_d3``    -- an 8-Gaussian mixture in the unit cube in 3-D with
  Exponential(1) weights, 50,000 x 40,000 points (the FlashSinkhorn summary's
  largest dense size, n = 50,000; SinkSLOT's "Gaussian d=3" benchmark family).
* ``gmm8_d3_sq`` -- the same recipe at n = m = 50,000 (the throughput headline).
* ``gauss_d64``  -- 16,384-point Gaussian clouds in 64-D, eps = 0.5 (SinkSLOT's
  "Gaussian d=64" grid, eps in [0.1, 1]).
* ``cluster_d3`` -- 2^20-point clustered 3-D clouds standing in for the N-body
  snapshots of the FlashSinkhorn 2 abstract (which are not available here):
  80 % of points around 4096 tight clusters, 20 % uniform background, blur equal
  to the mean interparticle spacing, i.e. eps = (n^(-1/3))^2.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    m: int
    d: int
    eps: float
    n_iters: int
    check_every: int
    grad: bool
    seed: int
    recipe: str
    description: str


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("gflow_d2", 1000, 1000, 2, 0.01, 200, 0, True, 1, "shifted_gauss",
                 "x~N(0,I2), y~N(0,I2)+3, uniform weights, eps=0.01, 200 iterations, f,g,cost,grad_x"),
        Workload("gauss_d2", 10000, 10000, 2, 0.05, 200, 10, False, 2, "gauss",
                 "x,y~N(0,I2), uniform weights, eps=0.05, 200 iterations, residual every 10"),
        Workload("gmm8_d3", 50000, 40000, 3, 0.01, 100, 0, False, 3, "gmm8",
                 "8-component Gaussian mixtures in [0,1]^3 (std 0.05), Exp(1) weights summing to 1, eps=0.01, 100 iterations"),
        Workload("gauss_d64", 16384, 16384, 64, 0.5, 100, 0, False, 4, "shifted_gauss64",
                 "x,y~N(0,I/64), y shifted by 0.5/sqrt(64) per coordinate, uniform weights, eps=0.5, 100 iterations"),
        Workload("cluster_d3", 1 << 20, 1 << 20, 3, float((1 << 20) ** (-2.0 / 3.0)), 50, 0, True, 5, "clusters",
                 "80% of points in 4096 clusters (std 0.002) with uniform centres in the unit cube, 20% uniform background, "
                 "uniform weights, eps=(n^(-1/3))^2, 50 iterations + grad_x"),
        Workload("gmm8_d3_sq", 50000, 50000, 3, 0.01, 100, 10, True, 6, "gmm8",
                 "the gmm8_d3 recipe at n=m=50,000: 100 iterations, residual every 10, cost and grad_x"),
    ]
}


def _uniform(rng: np.random.Generator, k: int) -> np.ndarray:
    del rng
    return np.full(k, 1.0 / k)


def _gmm8(rng: np.random.Generator, k: int, d: int) -> np.ndarray:
    means = rng.uniform(0.0, 1.0, size=(8, d))
    comp = rng.integers(0, 8, size=k)
    return means[comp] + 0.05 * rng.standard_normal((k, d))


def _clusters(rng: np.random.Generator, k: int, d: int) -> np.ndarray:
    centres = rng.uniform(0.0, 1.0, size=(4096, d))
    n_clustered = (8 * k) // 10
    which = rng.integers(0, 4096, size=n_clustered)
    clustered = centres[which] + 0.002 * rng.standard_normal((n_clustered, d))
    background = rng.uniform(0.0, 1.0, size=(k - n_clustered, d))
    pts = np.concatenate([clustered, background], axis=0)
    return pts[rng.permutation(k)]


def _exp_weights(rng: np.random.Generator, k: int) -> np.ndarray:
    w = rng.exponential(1.0, size=k)
    return w / w.sum()


def make_inputs(name: str, n: int | None = None, m: int | None = None, seed: int | None = None,
                d: int | None = None):
    """Draw (x, y, a, b) as contiguous float32 arrays for workload ``name``.

    ``n``/``m`` override the sizes (same recipe, smaller or ragged problem);
    ``seed`` overrides the workload's seed; ``d`` the dimension (same recipe
    in d dimensions).
    """
    w = WORKLOADS[name]
    n = w.n if n is None else int(n)
    m = w.m if m is None else int(m)
    d = w.d if d is None else int(d)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.recipe == "shifted_gauss":
        x = rng.standard_normal((n, d))
        y = rng.standard_normal((m, d)) + 3.0
        a, b = _uniform(rng, n), _uniform(rng, m)
    elif w.recipe == "gauss":
        x = rng.standard_normal((n, d))
        y = rng.standard_normal((m, d))
        a, b = _uniform(rng, n), _uniform(rng, m)
    elif w.recipe == "gmm8":
        x = _gmm8(rng, n, d)
        y = _gmm8(rng, m, d)
        a, b = _exp_weights(rng, n), _exp_weights(rng, m)
    elif w.recipe == "shifted_gauss64":
        s = 1.0 / np.sqrt(d)
        x = s * rng.standard_normal((n, d))
        y = s * rng.standard_normal((m, d)) + 0.5 / np.sqrt(d)
        a, b = _uniform(rng, n), _uniform(rng, m)
    elif w.recipe == "clusters":
        x = _clusters(rng, n, d)
        y = _clusters(rng, m, d)
        a, b = _uniform(rng, n), _uniform(rng, m)
    else:  # pragma: no cover - table above is closed
        raise KeyError(w.recipe)
    f32 = lambda v: np.ascontiguousarray(v, dtype=np.float32)  # noqa: E731
    return f32(x), f32(y), f32(a), f32(b)


def random_problem(n: int, m: int, d: int, seed: int, *, scale: float = 1.0, shift: float = 0.0,
                   weights: str = "exp", zero_frac: float = 0.0):
    """Small generic problem for parity sweeps: Gaussian clouds, optional zero weights.

    weights: "uniform" or "exp" (Exponential(1), normalised so both sum to 1).
    zero_frac: fraction of weights set exactly to zero (then renormalised).
    """
    rng = np.random.default_rng(seed)
    x = scale * rng.standard_normal((n, d))
    y = scale * rng.standard_normal((m, d)) + shift
    if weights == "uniform":
        a, b = np.full(n, 1.0 / n), np.full(m, 1.0 / m)
    else:
        a, b = rng.exponential(1.0, n), rng.exponential(1.0, m)
    if zero_frac > 0.0:
        a[rng.random(n) < zero_frac] = 0.0
        b[rng.random(m) < zero_frac] = 0.0
        if a.sum() == 0.0:
            a[0] = 1.0
        if b.sum() == 0.0:
            b[0] = 1.0
    a, b = a / a.sum(), b / b.sum()
    f32 = lambda v: np.ascontiguousarray(v, dtype=np.float32)  # noqa: E731
    return f32(x), f32(y), f32(a), f32(b)


def eps32(eps: float) -> float:
    """The entropic strength both sides use: the float32 value of eps, as a Python float."""
    return float(np.float32(eps))


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the given arrays (detects generator drift)."""
    h = hashlib.sha256()
    for arr in arrays:
        h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()
