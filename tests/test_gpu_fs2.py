"""GPU parity of the two-stage block-sparse solver ("FlashSinkhorn 2:
Block-Sparse Entropic Optimal Transport", abstract) against its float64
reference (oracle/fs2.py), through the C ABI.

  * The Morton order is integer work decided in float32 on both sides: equal
    bit for bit (ties by index).
  * With every data-dependent decision switched off (tol = 0 and a coarse gain
    that never stops the coarse stage, so exactly max_rounds rounds and
    max_iters fine iterations), the potentials match the reference to
    1e-4 max C, the tolerance of the dense solve: each step is a Sinkhorn
    half-step over the same blocks; a tile whose keep decision differs between
    float32 and float64 sits at the threshold, so its mass is at most delta
    times the row or column mass.
  * Beyond the reference's reach, the stopping rule is checked against the
    all-particle residual of the returned potentials, evaluated densely on
    the GPU: at most tol + delta max(a, b) plus the float32 floor of the
    residual, 32 kappa max(a, b).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from oracle import fs2 as FS
from sk_inputs import eps32

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


def clustered(n, d, k, std, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    cen = rng.random((k, d))
    lab = rng.integers(0, k, n)
    p = (cen[lab] + std * rng.normal(size=(n, d))).astype(np.float32)
    w = rng.exponential(size=n) if skew == 0.0 else np.exp(skew * rng.normal(size=n))
    return p, (w / w.sum()).astype(np.float32)


@pytest.mark.parametrize("d", [1, 2, 3, 5])
def test_morton_order_matches_reference(d):
    x, a = clustered(6000, d, 12, 0.05, 1 + d)
    y, b = clustered(5000, d, 12, 0.05, 11 + d)
    x[100:140] = x[100]  # exact ties keep index order
    X, Y, A, B = dev(x, y, a, b)
    _, _, info = sk.fs2_solve(X, Y, A, B, eps=eps32(0.05), block=128, max_rounds=1, coarse_iters=1, max_iters=0,
                              n_sample=16, return_perm=True)
    lo, hi = np.minimum(x.min(0), y.min(0)), np.maximum(x.max(0), y.max(0))
    assert np.array_equal(host(info["perm_x"]).astype(np.int64), FS.morton_order(x, lo, hi))
    assert np.array_equal(host(info["perm_y"]).astype(np.int64), FS.morton_order(y, lo, hi))


FIXED_CASES = [
    # n, m, d, k clusters, std, eps, B, delta, rounds, coarse iters, fine iters, seed
    (1500, 1300, 2, 10, 0.03, 0.004, 64, 1e-6, 3, 10, 60, 21),
    (1200, 1400, 3, 8, 0.05, 0.01, 50, 1e-5, 2, 15, 40, 22),
    (700, 900, 2, 6, 0.04, 0.02, 512, 1e-6, 2, 10, 30, 23),  # one block per side
    (1000, 800, 1, 5, 0.02, 0.002, 32, 1e-4, 3, 10, 50, 24),
    # d = 4 ... 7: the screening's per-dimension block records (58-78% of the tiles kept)
    (900, 800, 4, 8, 0.02, 0.005, 32, 1e-5, 2, 10, 30, 25),
    (800, 700, 5, 8, 0.02, 0.005, 32, 1e-5, 2, 10, 30, 26),
    (700, 900, 6, 8, 0.02, 0.005, 32, 1e-5, 2, 10, 30, 27),
    (600, 700, 7, 8, 0.02, 0.005, 32, 1e-5, 2, 10, 30, 28),
]


@pytest.mark.parametrize("case", FIXED_CASES, ids=[f"{c[0]}x{c[1]}d{c[2]}B{c[6]}" for c in FIXED_CASES])
def test_fixed_counts_match_reference(case):
    n, m, d, k, std, eps, B, delta, rounds, ci, iters, seed = case
    x, a = clustered(n, d, k, std, seed)
    y, b = clustered(m, d, k, std, seed + 100, skew=1.5)
    eps = eps32(eps)
    kw = dict(B=B, tol=0.0, delta=delta, coarse_iters=ci, max_rounds=rounds, coarse_gain=-1e6, n_sample=64,
              max_iters=iters, check_every=10, screen_every=10)
    say("fs2 fixed", case)
    X, Y, A, Bt = dev(x, y, a, b)
    f_t, g_t, info = sk.fs2_solve(X, Y, A, Bt, eps=eps, block=B, tol=0.0, delta=delta, coarse_iters=ci,
                                  max_rounds=rounds, coarse_gain=-1e6, n_sample=64, max_iters=iters, check_every=10,
                                  screen_every=10)
    f, g = host(f_t), host(g_t)
    fo, go, io = FS.solve(x, y, a, b, eps, **kw)
    maxc = oracle.max_cost(x, y)
    err = max(np.abs(f - fo).max(), np.abs(g - go).max())
    say("rounds", info["rounds"], io["rounds"], "iters", info["fine_iters"], io["fine_iters"], "err/tol",
        err / (1e-4 * maxc), "kept", info["kept_fraction"], io["kept_fraction"][-1], "resid", info["residual"],
        io["residual"])
    assert info["rounds"] == rounds == io["rounds"] and info["fine_iters"] == iters == io["fine_iters"]
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    assert err <= 1e-4 * maxc
    assert abs(info["kept_fraction"] - io["kept_fraction"][-1]) <= 0.02


def _edge_weights(rng, n, zero_frac):
    v = rng.exponential(size=n)
    if zero_frac:
        v[rng.random(n) < zero_frac] = 0.0
    return (v / v.sum()).astype(np.float32)


EDGE_CASES = [
    # name, n, m, d, zero fractions (a, b), eps, B, coarse rounds
    ("one_source", 1, 7, 2, (0.0, 0.0), 0.05, 4, 1),
    ("one_target", 9, 1, 3, (0.0, 0.0), 0.05, 4, 1),
    ("d8", 300, 260, 8, (0.0, 0.0), 0.2, 32, 2),
    ("zero_weights", 400, 350, 2, (0.3, 0.2), 0.01, 32, 2),
    ("identical_points", 50, 40, 2, (0.0, 0.0), 0.05, 16, 1),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases_match_reference(case):
    """One point on a side, d = 8 (3 Morton bits per coordinate), zero weights (excluded from the
    block maxima of the screening), and a flat bounding box (all Morton codes 0)."""
    name, n, m, d, (za, zb), eps, B, rounds = case
    rng = np.random.default_rng(90 + len(name))
    x = rng.random((n, d)).astype(np.float32)
    y = rng.random((m, d)).astype(np.float32)
    if name == "identical_points":
        x[:] = 0.25
        y[:] = 0.25
    a, b = _edge_weights(rng, n, za), _edge_weights(rng, m, zb)
    eps = eps32(eps)
    # the residual is checked after the last iteration only: with one point on a side it can be
    # exactly 0 in float32 (and 1e-8 in float64), which would meet tol = 0 at an earlier check
    kw = dict(tol=0.0, delta=1e-6, coarse_iters=5, max_rounds=rounds, coarse_gain=-1e6, n_sample=16, max_iters=20,
              check_every=1000, screen_every=10)
    say("fs2 edge", case)
    fo, go, io = FS.solve(x, y, a, b, eps, B=B, **kw)
    X, Y, A, Bt = dev(x, y, a, b)
    f_t, g_t, info = sk.fs2_solve(X, Y, A, Bt, eps=eps, block=B, **kw)
    f, g = host(f_t), host(g_t)
    # the dense solve's bar, 1e-4 max C; with every cost 0 (identical points) the potentials are
    # of the size of eps times a log-sum of weights, so eps sets the scale there
    scale = max(oracle.max_cost(x, y), eps)
    err = max(np.abs(f - fo).max(), np.abs(g - go).max())
    say("err/tol", err / (1e-4 * scale), "kept", info["kept_fraction"], io["kept_fraction"][-1])
    assert info["rounds"] == rounds and info["fine_iters"] == 20
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    assert err <= 1e-4 * scale
    assert abs(info["kept_fraction"] - io["kept_fraction"][-1]) <= 0.02


ADAPTIVE_COARSE_CASES = [
    # eps, B, seed: the coarse stage runs 3 rounds (the check falls, then rises) / 2 rounds with
    # check values near 1e263 and 1e266, far beyond float32 (the decisions are taken on log2)
    (5e-4, 64, 41),
    (2e-4, 128, 44),
]


@pytest.mark.parametrize("eps,B,seed", ADAPTIVE_COARSE_CASES)
def test_coarse_decisions_match_reference(eps, B, seed):
    """The coarse stage's own stopping rule (coarse_gain 0.1, tol 0) takes the reference's
    decisions, also where the check value overflows float32, and the potentials then match."""
    x, a = clustered(1400, 2, 10, 0.03, seed)
    y, b = clustered(1200, 2, 10, 0.03, seed + 100, skew=1.5)
    eps = eps32(eps)
    kw = dict(tol=0.0, delta=1e-6, coarse_iters=10, max_rounds=6, coarse_gain=0.1, n_sample=64, max_iters=20,
              check_every=10, screen_every=10)
    say("fs2 coarse", (eps, B, seed))
    fo, go, io = FS.solve(x, y, a, b, eps, B=B, **kw)
    X, Y, A, Bt = dev(x, y, a, b)
    f_t, g_t, info = sk.fs2_solve(X, Y, A, Bt, eps=eps, block=B, **kw)
    f, g = host(f_t), host(g_t)
    err = max(np.abs(f - fo).max(), np.abs(g - go).max())
    maxc = oracle.max_cost(x, y)
    say("rounds", info["rounds"], io["rounds"], "checks", io["checks"], "gpu last", info["last_check"],
        "err/tol", err / (1e-4 * maxc))
    assert 1 < io["rounds"] < kw["max_rounds"]
    assert info["rounds"] == io["rounds"]
    if io["checks"][-1] > float(np.finfo(np.float32).max):
        assert info["last_check"] == np.inf
    else:
        assert abs(info["last_check"] - io["checks"][-1]) <= 0.05 * io["checks"][-1]
    assert err <= 1e-4 * maxc


def dense_residual(X, Y, A, B, f_t, g_t, eps):
    r = host(sk.marginal_residual(X, Y, A, B, f_t, g_t, eps=eps))
    return max(r[0], r[1])


@pytest.mark.parametrize("n,d,k,std,eps,B,seed", [(40000, 2, 64, 0.01, 1e-3, 256, 31),
                                                  (60000, 3, 128, 0.01, 2e-3, 512, 32)])
def test_reaches_target_residual(n, d, k, std, eps, B, seed):
    """Adaptive run (coarse rounds and stop rule on): the all-particle residual of the result,
    evaluated densely, is within tol + delta max(w) + the float32 floor, and its dual cost agrees to
    relative 1e-4 with that of a dense solve stopped by the same marginal tolerance."""
    x, a = clustered(n, d, k, std, seed)
    y, b = clustered(n, d, k, std, seed + 7)
    eps = eps32(eps)
    tol, delta = 1e-5 / n * 1000, 1e-6
    X, Y, A, B_ = dev(x, y, a, b)
    f_t, g_t, info = sk.fs2_solve(X, Y, A, B_, eps=eps, block=B, tol=tol, delta=delta, max_iters=20000)
    say("fs2", (n, d), info)
    assert info["converged"]
    wmax = float(max(a.max(), b.max()))
    f, g = host(f_t), host(g_t)
    maxc = float(d)  # the unit box
    kap = U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps
    r = dense_residual(X, Y, A, B_, f_t, g_t, eps)
    say("all-particle residual", r, "bound", tol + delta * wmax + 32 * kap * wmax)
    assert r <= tol + delta * wmax + 32 * kap * wmax
    assert info["kept_fraction"] < 0.5
    fd, gd, it, conv, viol = sk.solve_ex(X, Y, A, B_, eps=eps, stop_mode="marginal", stop_tol=tol, max_iter=20000,
                                         check_every=10)
    c_fs2 = float(host(sk.dual_cost(X, Y, A, B_, f_t, g_t, eps=eps))[0])
    c_dense = float(host(sk.dual_cost(X, Y, A, B_, fd, gd, eps=eps))[0])
    say("dense", it, "iterations; cost fs2", c_fs2, "dense", c_dense)
    assert conv and abs(c_fs2 - c_dense) <= 1e-4 * abs(c_dense)


def test_repeat_runs_are_bit_identical():
    """Fixed-order reductions, a stable radix sort and ordered tile lists: two solves give the same
    bits (potentials, counts, kept tiles, residual)."""
    x, a = clustered(20000, 3, 40, 0.01, 51)
    y, b = clustered(18000, 3, 40, 0.01, 52)
    X, Y, A, B = dev(x, y, a, b)
    runs = []
    for _ in range(2):
        f_t, g_t, info = sk.fs2_solve(X, Y, A, B, eps=eps32(2e-3), block=256, tol=1e-7, max_iters=300)
        runs.append((host(f_t), host(g_t), info))
    (f1, g1, i1), (f2, g2, i2) = runs
    assert np.array_equal(f1, f2) and np.array_equal(g1, g2)
    for k in ("rounds", "fine_iters", "kept", "converged", "residual"):
        assert i1[k] == i2[k] or (k == "residual" and np.isnan(i1[k]) and np.isnan(i2[k])), k


def test_workspace_query_at_large_block_counts():
    """The workspace size does not depend on the thresholds: it is returned for block counts whose
    every-pair-kept total would exceed the kept-tile lists (2^14 x 2^14 blocks and more)."""
    lib = sk.load_library()
    for n in (1 << 23, 1 << 24):
        nb = lib.sk_fs2_workspace_bytes(n, n, 3, 512, 1024)
        assert nb > 0
        # lists of 2^28 entries (two, 4 bytes each) plus O(n) arrays, not O(NB^2) ones
        assert nb < 4 * (1 << 30) + 400 * n
