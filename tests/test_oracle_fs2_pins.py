"""Pins for the two-stage block-sparse reference (oracle/fs2.py): textbook
Z-order codes, the screening bound checked by brute force against the dense
plan, the lift against the C oracle's c-transform, the sampled check against
the C oracle's marginals, the coarse stage's acceptance rule against check
values built by an independent route, reductions to dense Sinkhorn (delta = 0,
one point per block), far tiles omitted, and the all-particle residual at the
end; every
planted mistake in its source must trip at least one pin.

Source: "FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport", abstract.
"""
import importlib.util

import numpy as np
import pytest

import oracle
from oracle import fs2 as F0

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _clustered(n, d, k, std, seed, shift=0.0):
    rng = np.random.default_rng(seed)
    cen = rng.random((k, d))
    lab = rng.integers(0, k, n)
    p = (cen[lab] + std * rng.normal(size=(n, d)) + shift).astype(np.float32)
    w = rng.exponential(size=n)
    return p, w / w.sum()


def _plan(x, y, a, b, f, g, eps):
    C = ((x[:, None, :].astype(np.float64) - y[None, :, :]) ** 2).sum(-1)
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)


# --------------------------------------------------------------------------- pins
def pin_morton_textbook(F):
    """Z-order: interleaved bits, x first (d = 2: (1,0) -> 1, (0,1) -> 2, (3,3) -> 15, (4,0) -> 16; d = 3 alike)."""
    cases2 = {(0, 0): 0, (1, 0): 1, (0, 1): 2, (1, 1): 3, (2, 0): 4, (3, 0): 5, (2, 1): 6, (0, 2): 8, (3, 3): 15,
              (4, 0): 16, (5, 9): 0b10010011}
    q = np.array(list(cases2), dtype=np.float64)
    p = ((q + 0.5) / 1024.0).astype(np.float32)
    codes = F.morton_codes(p, np.zeros(2, np.float32), np.ones(2, np.float32))
    assert list(codes) == list(cases2.values())
    cases3 = {(1, 0, 0): 1, (0, 1, 0): 2, (0, 0, 1): 4, (1, 1, 1): 7, (2, 0, 0): 8, (0, 0, 2): 32}
    q = np.array(list(cases3), dtype=np.float64)
    p = ((q + 0.5) / 1024.0).astype(np.float32)
    codes = F.morton_codes(p, np.zeros(3, np.float32), np.ones(3, np.float32))
    assert list(codes) == list(cases3.values())
    # the order sorts by code and keeps equal codes in index order
    p = np.array([[0.9, 0.9], [0.1, 0.1], [0.1, 0.1], [0.6, 0.1]], np.float32)
    assert list(F.morton_order(p, np.zeros(2, np.float32), np.ones(2, np.float32))) == [1, 2, 3, 0]


def pin_screen_bound(F):
    """Brute force: the mass of omitted tiles is at most delta a_i in every row and delta b_j in every
    column -- also with very uneven block masses (a few heavy source points), where the row and the
    column conditions differ."""
    for skew, seed in ((0.0, 1), (4.0, 21)):
        x, a = _clustered(300, 2, 6, 0.03, seed)
        y, b = _clustered(260, 2, 6, 0.03, seed + 1)
        if skew:
            w = np.exp(skew * np.random.default_rng(seed + 2).normal(size=300))
            a = w / w.sum()
        lo, hi = np.minimum(x.min(0), y.min(0)), np.maximum(x.max(0), y.max(0))
        px, py = F.morton_order(x, lo, hi), F.morton_order(y, lo, hi)
        x, a, y, b = x[px], a[px], y[py], b[py]
        eps = 0.003
        f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 30)
        B = 20
        xb, yb = F.blocks(x, a, B), F.blocks(y, b, B)
        P = _plan(x, y, a, b, f, g, eps)
        for delta in (1e-2, 1e-3, 1e-6):
            keep = F.screen(f, g, a, b, B, xb, yb, eps, delta)
            om = ~F.tile_mask(keep, B, 300, 260)
            assert om.any() and keep.any()
            assert np.all((P * om).sum(1) <= delta * a + 1e-300)
            assert np.all((P * om).sum(0) <= delta * b + 1e-300)


def pin_screen_tile_bound_exact(F):
    """Blocks of identical points make the screening bound exact; then, over a sweep of delta, each
    omitted tile adds at most delta a_i / NBy to every row and delta b_j / NBx to every column, while
    uneven block masses make the row and column conditions differ."""
    rng = np.random.default_rng(31)
    B, nbx, nby = 10, 6, 5
    cx, cy = rng.random((nbx, 2)), rng.random((nby, 2))
    x = np.repeat(cx, B, axis=0).astype(np.float32)
    y = np.repeat(cy, B, axis=0).astype(np.float32)
    a = np.repeat(10.0 ** np.arange(nbx), B)
    b = np.repeat(10.0 ** (-np.arange(nby)), B)
    a, b = a / a.sum(), b / b.sum()
    lo, hi = np.minimum(x.min(0), y.min(0)), np.maximum(x.max(0), y.max(0))
    px, py = F.morton_order(x, lo, hi), F.morton_order(y, lo, hi)
    x, a, y, b = x[px], a[px], y[py], b[py]
    eps = 0.05
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 50)
    xb, yb = F.blocks(x, a, B), F.blocks(y, b, B)
    P = _plan(x, y, a, b, f, g, eps)
    T = P.reshape(nbx, B, nby, B)
    row_part = T.sum(axis=3)          # [I, i, J]: contribution of tile (I, J) to row i of block I
    col_part = T.sum(axis=1)          # [I, J, j]
    omitted_any = False
    for delta in np.logspace(-14, 0, 57):
        keep = F.screen(f, g, a, b, B, xb, yb, eps, float(delta))
        for I in range(nbx):
            for J in range(nby):
                if keep[I, J]:
                    continue
                omitted_any = True
                ai, bj = a[I * B:(I + 1) * B], b[J * B:(J + 1) * B]
                assert np.all(row_part[I, :, J] <= delta * ai / nby * (1 + 1e-9)), (delta, I, J)
                assert np.all(col_part[I, J, :] <= delta * bj / nbx * (1 + 1e-9)), (delta, I, J)
    assert omitted_any


def pin_far_tiles_omitted(F):
    """Two clusters far apart: at converged potentials every tile joining them is omitted."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=(40, 2)) * 0.01, rng.normal(size=(40, 2)) * 0.01 + 3.0]).astype(np.float32)
    y = np.concatenate([rng.normal(size=(40, 2)) * 0.01, rng.normal(size=(40, 2)) * 0.01 + 3.0]).astype(np.float32)
    a = np.full(80, 1 / 80)
    eps = 0.01
    f, g, _ = oracle.sinkhorn(x, y, a, a, eps, 200)
    xb, yb = F.blocks(x, a, 20), F.blocks(y, a, 20)
    keep = F.screen(f, g, a, a, 20, xb, yb, eps, 1e-6)
    assert not keep[:2, 2:].any() and not keep[2:, :2].any()
    assert keep[:2, :2].any() and keep[2:, 2:].any()


def pin_lift_and_check(F):
    """The lift is the C oracle's c-transform against the centroids; the check is the C oracle's row residual."""
    x, a = _clustered(200, 2, 4, 0.05, 4)
    y, b = _clustered(180, 2, 4, 0.05, 5)
    eps = 0.02
    B = 16
    mass, cen, _, _ = F.blocks(y, b, B)
    G = np.random.default_rng(6).normal(size=len(mass)) * 0.01
    lift = F.c_transform(x, cen, mass, G, eps)
    assert np.allclose(lift, oracle.half_step(x, cen, mass, G, eps), rtol=0, atol=1e-12)
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, 3)
    rows = F.sample_rows(200, 37)
    rs, _ = oracle.marginals(x, y, a, b, f, g, eps)
    assert F.row_check(x.astype(np.float64), y.astype(np.float64), a, b, f, g, eps, rows) == pytest.approx(
        np.abs(rs[rows] - a[rows]).max(), rel=1e-9)


def pin_delta_zero_is_dense(F):
    """delta = 0 keeps every tile: the fine stage is dense Sinkhorn and reaches the dense plan."""
    x, a = _clustered(150, 2, 3, 0.1, 7)
    y, b = _clustered(130, 2, 3, 0.1, 8)
    eps = 0.05
    f, g, info = F.solve(x, y, a, b, eps, B=16, tol=1e-12, delta=0.0, coarse_iters=5, max_rounds=2,
                         n_sample=32, max_iters=3000, check_every=20)
    assert all(k == 1.0 for k in info["kept_fraction"])
    fd, gd, _ = oracle.sinkhorn(x, y, a, b, eps, 3000)
    assert np.allclose(_plan(x, y, a, b, f, g, eps), _plan(x, y, a, b, fd, gd, eps), rtol=0, atol=1e-12)


def pin_single_point_blocks(F):
    """B = 1: the centroids are the points, the coarse stage is dense Sinkhorn and its lift is exact."""
    x, a = _clustered(60, 2, 3, 0.1, 9)
    y, b = _clustered(50, 2, 3, 0.1, 10)
    eps = 0.1
    f, g, info = F.solve(x, y, a, b, eps, B=1, tol=1e-11, delta=1e-8, coarse_iters=2000, max_rounds=1,
                         n_sample=60, max_iters=10, check_every=1)
    assert info["checks"][0] < 1e-11
    fd, gd, _ = oracle.sinkhorn(x, y, a, b, eps, 2000)
    assert np.allclose(_plan(x, y, a, b, f, g, eps), _plan(x, y, a, b, fd, gd, eps), rtol=0, atol=1e-11)


def pin_all_particle_residual(F):
    """At the end the all-particle residual (dense, C oracle) is within tol + delta max(a, b)."""
    x, a = _clustered(400, 2, 8, 0.02, 11)
    y, b = _clustered(350, 2, 8, 0.02, 12)
    eps, tol, delta = 0.004, 1e-5, 1e-4
    f, g, info = F.solve(x, y, a, b, eps, B=25, tol=tol, delta=delta, max_iters=3000)
    assert info["residual"] <= tol
    assert min(info["kept_fraction"]) < 1.0
    r = oracle.residual(x, y, a, b, f, g, eps)
    assert max(r[0], r[1]) <= tol + delta * max(a.max(), b.max()) * 1.0001


def _coarse_checks(F, x, y, a, b, eps, B, coarse_iters, rounds, n_sample):
    """Each round's check value built without the solver: blocks summed directly, the centroid solve by the C
    oracle continued from the previous round's G (g_init), both lifts by the C oracle's half-step, and the sampled
    row deviation from the C oracle's plan marginals at the lifted potentials."""
    lo, hi = np.minimum(x.min(0), y.min(0)), np.maximum(x.max(0), y.max(0))
    px, py = F.morton_order(x, lo, hi), F.morton_order(y, lo, hi)
    xs, ys = x[px].astype(np.float64), y[py].astype(np.float64)
    as_, bs = a[px], b[py]
    starts_x, starts_y = np.arange(0, len(xs), B), np.arange(0, len(ys), B)
    amass, bmass = np.add.reduceat(as_, starts_x), np.add.reduceat(bs, starts_y)
    xcen = np.add.reduceat(as_[:, None] * xs, starts_x) / amass[:, None]
    ycen = np.add.reduceat(bs[:, None] * ys, starts_y) / bmass[:, None]
    s = min(len(xs), n_sample)
    rows = np.array([k * (len(xs) // s) for k in range(s)])
    G = np.zeros(len(bmass))
    out = []
    for _ in range(rounds):
        Fc, G, _ = oracle.sinkhorn(xcen, ycen, amass, bmass, eps, coarse_iters, g_init=G)
        f = oracle.half_step(xs, ycen, bmass, G, eps)
        g = oracle.half_step(ys, xcen, amass, Fc, eps)
        rs, _ = oracle.marginals(xs, ys, as_, bs, f, g, eps)
        out.append(float(np.abs(rs[rows] - as_[rows]).max()))
    return out


def pin_coarse_acceptance_rule(F):
    """The coarse stage ends at the first round whose check value is <= tol, or fell by less than the fraction
    coarse_gain since the round before, or is the max_rounds-th (the abstract: a sampled marginal check accepts
    or rejects the lift, and a rejection continues on the centroids).  The check values come from an independent
    route; the four cases stop on the gain rule, on the tolerance, on the round cap, and on a rising check with
    coarse_gain = 0, and each case asserts which rule ended it."""
    x, a = _clustered(300, 2, 4, 0.1, 1)
    y, b = _clustered(260, 2, 4, 0.1, 2)
    eps, B, ci, ns = 0.05, 10, 1, 64
    ref = _coarse_checks(F, x, y, a, b, eps, B, ci, 6, ns)
    # the sequence these cases rely on: a large fall, a small fall, then a rise
    assert ref[1] < 0.6 * ref[0] and 0.8 * ref[1] < ref[2] < ref[1] and ref[3] > ref[2]
    for tol, gain, max_rounds, why in ((0.0, 0.3, 12, "gain"), (0.5 * (ref[0] + ref[1]), 0.3, 12, "tol"),
                                        (0.0, 0.3, 2, "cap"), (0.0, 0.0, 12, "gain")):
        rounds, rule = None, None
        for r in range(1, len(ref) + 1):
            if ref[r - 1] <= tol:
                rounds, rule = r, "tol"
            elif r >= max_rounds:
                rounds, rule = r, "cap"
            elif r >= 2 and ref[r - 1] > (1.0 - gain) * ref[r - 2]:
                rounds, rule = r, "gain"
            if rounds:
                break
        assert rule == why, (tol, gain, max_rounds, rule)
        _, _, info = F.solve(x, y, a, b, eps, B=B, tol=tol, delta=1e-6, coarse_iters=ci, max_rounds=max_rounds,
                             coarse_gain=gain, n_sample=ns, max_iters=1)
        assert info["rounds"] == rounds, (why, info["rounds"], rounds)
        assert np.allclose(info["checks"], ref[:rounds], rtol=1e-9, atol=0)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(F0)


MUTANTS = {
    "morton_coordinate_major": ("code |= ((q[:, t] >> k) & 1) << (k * d + t)", "code |= ((q[:, t] >> k) & 1) << (t * bits + k)"),
    "morton_unstable": ("return np.lexsort((np.arange(len(code)), code))", "return np.lexsort((-np.arange(len(code)), code))"),
    "screen_no_distance": ("E = (fmax[:, None] + gmax[None, :] - dmin2) / eps", "E = (fmax[:, None] + gmax[None, :]) / eps"),
    "screen_min_mass": ("lm = np.log(np.maximum(bmass[None, :] * nby, amass[:, None] * nbx))",
                        "lm = np.log(np.minimum(bmass[None, :] * nby, amass[:, None] * nbx))"),
    "screen_threshold": ("keep = score > math.log(delta) if delta > 0", "keep = score > math.log(delta) + 8.0 if delta > 0"),
    "check_sign": ("r = as_[rows] * np.expm1((f[rows] - t) / eps)", "r = as_[rows] * np.expm1((t - f[rows]) / eps)"),
    "lift_unweighted": ("f = c_transform(xs, ycen, bmass, G, eps)", "f = c_transform(xs, ycen, np.ones_like(bmass), G, eps)"),
    "fine_col_stale": ("g = masked_update(C.T, as_, f, eps, mask.T)", "g = masked_update(C.T, as_, f * 0.0, eps, mask.T)"),
    "gain_flipped": ("checks[-1] > (1.0 - coarse_gain) * checks[-2]", "checks[-1] < (1.0 - coarse_gain) * checks[-2]"),
    "gain_removed": ("if len(checks) >= 2 and checks[-1] > (1.0 - coarse_gain) * checks[-2]:", "if False:"),
    "coarse_restart": ("F, G = sinkhorn_dense(xcen, ycen, amass, bmass, eps, coarse_iters, G)",
                       "F, G = sinkhorn_dense(xcen, ycen, amass, bmass, eps, coarse_iters, G * 0.0)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(F0.__file__).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "fs2_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("fs2_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
