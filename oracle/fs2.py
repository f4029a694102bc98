"""Plain float64 reference of the two-stage block-sparse solver.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the GPU library never
imports or calls it.  Dense numpy arrays throughout (the n x m cost is formed
for the masked fine stage), so it is meant for a few thousand points.

Source: "FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport", Abstract.
The abstract outlines two stages.  First, Sinkhorn runs on the block centroids;
its potentials are extended to all points, and the centroid solve goes on for
as long as a marginal test on a sample of rows is not passed.  Second,
point-level iterations over Morton-ordered blocks correct what the centroids
got wrong, skipping the block pairs whose possible share of any row's or
column's mass, bounded through the block masses, is negligible.  The pages
give nothing beyond that; the reading written out here (each step a plain
definition) is:

  1. Morton order: the bounding box [lo, hi] of both clouds together; per
     coordinate q = min(2^bits - 1, floor((p - lo) * (2^bits / (hi - lo))))
     in float32 (0 when hi == lo), bits = 30 // d (at most 10); the code
     interleaves the bits, bit k of coordinate t at position k d + t; each
     cloud is sorted by (code, index).
  2. Blocks: runs of B consecutive sorted points.  Block mass = sum of
     weights; centroid = weighted mean (plain mean for a massless block); box =
     per-coordinate min and max of the block's points.
  3. Coarse stage: alternating Sinkhorn on the centroid measures from G = 0,
     in rounds of coarse_iters.  After each round the potentials are lifted to
     the points by one c-transform against the other side's centroids,
       f_i = -eps log sum_J B_J exp((G_J - |x_i - Ybar_J|^2)/eps)  (g alike),
     and the check value is the largest |(P 1)_i - a_i| over n_sample rows
     (every (n // n_sample)-th sorted row) at the lifted potentials, P over all
     points.  The lift is accepted -- the coarse stage ends -- when the check
     value is <= tol, or when it fell by less than the fraction coarse_gain
     since the previous round, or after max_rounds rounds; otherwise (the
     check rejects the lift) the coarse stage continues on the centroids.
  4. Screening: with f~_I = max of f over block I's points of positive weight,
     g~_J alike, and dmin_IJ the distance between the two boxes, tile (I, J) is
     kept iff
       (f~_I + g~_J - dmin_IJ^2)/eps + log max(B_J NBy, A_I NBx) > log delta,
     so an omitted tile adds at most delta a_i / NBy to row i and
     delta b_j / NBx to column j (NBx, NBy the block counts): all omitted tiles
     together add at most delta a_i (delta b_j).  Each row block and each
     column block also keeps its tile of largest bound, so no row is empty.
  5. Fine stage from the lifted potentials: alternating updates restricted to
     the kept tiles (the c-transform over kept keys only), screening again
     before every screen_every-th iteration; after every check_every-th
     iteration (and the last) the marginal residual of the kept-tile plan is
     checked and the stage stops once it is <= tol, or after max_iters.
The potentials are returned in the caller's point order.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def morton_bits(d: int) -> int:
    return max(1, min(10, 30 // d))


def morton_codes(p, lo, hi) -> np.ndarray:
    """Integer Morton codes of the float32 points p against the float32 box [lo, hi]."""
    p = np.asarray(p, dtype=np.float32)
    lo = np.asarray(lo, dtype=np.float32)
    hi = np.asarray(hi, dtype=np.float32)
    n, d = p.shape
    bits = morton_bits(d)
    top = (1 << bits) - 1
    span = hi - lo
    with np.errstate(divide="ignore"):
        scale = np.where(span > 0, np.float32(1 << bits) / np.where(span > 0, span, np.float32(1)), np.float32(0))
    scale = scale.astype(np.float32)
    q = np.floor((p - lo).astype(np.float32) * scale).astype(np.int64)
    q = np.clip(q, 0, top)
    code = np.zeros(n, dtype=np.int64)
    for k in range(bits):
        for t in range(d):
            code |= ((q[:, t] >> k) & 1) << (k * d + t)
    return code


def morton_order(p, lo, hi) -> np.ndarray:
    code = morton_codes(p, lo, hi)
    return np.lexsort((np.arange(len(code)), code))


def blocks(p, w, B: int):
    """Per block of B consecutive points: mass, centroid, box lo, box hi."""
    p, w = np.asarray(p, dtype=np.float64), np.asarray(w, dtype=np.float64)
    nb = (len(p) + B - 1) // B
    mass, cen = np.zeros(nb), np.zeros((nb, p.shape[1]))
    blo, bhi = np.zeros((nb, p.shape[1])), np.zeros((nb, p.shape[1]))
    for I in range(nb):
        sl = slice(I * B, min((I + 1) * B, len(p)))
        mass[I] = w[sl].sum()
        cen[I] = (w[sl, None] * p[sl]).sum(axis=0) / mass[I] if mass[I] > 0 else p[sl].mean(axis=0)
        blo[I], bhi[I] = p[sl].min(axis=0), p[sl].max(axis=0)
    return mass, cen, blo, bhi


def c_transform(q, k, wk, pot, eps):
    """-eps log sum_j wk_j exp((pot_j - |q_i - k_j|^2)/eps) for every query row."""
    C = ((np.asarray(q, np.float64)[:, None, :] - np.asarray(k, np.float64)[None, :, :]) ** 2).sum(-1)
    with np.errstate(divide="ignore"):
        lw = np.log(np.asarray(wk, np.float64))
    return -eps * logsumexp((np.asarray(pot)[None, :] - C) / eps + lw[None, :], axis=1)


def sinkhorn_dense(x, y, a, b, eps, n_iters, g0):
    """Alternating dense Sinkhorn from g0 (the centroid solve of the coarse stage)."""
    g = np.array(g0, dtype=np.float64)
    f = None
    for _ in range(n_iters):
        f = c_transform(x, y, b, g, eps)
        g = c_transform(y, x, a, f, eps)
    return f, g


def sample_rows(n: int, n_sample: int) -> np.ndarray:
    s = min(n, n_sample)
    return np.arange(s) * (n // s)


def row_check(xs, ys, as_, bs, f, g, eps, rows) -> float:
    """max |(P 1)_i - a_i| over the given rows, P over all points."""
    t = c_transform(xs[rows], ys, bs, g, eps)
    r = as_[rows] * np.expm1((f[rows] - t) / eps)
    return float(np.abs(r).max())


def screen(f, g, as_, bs, B, xb, yb, eps, delta):
    """Kept tiles (NBx x NBy bool) for potentials f, g on sorted points."""
    amass, _, xlo, xhi = xb
    bmass, _, ylo, yhi = yb
    nbx, nby = len(amass), len(bmass)
    fmax = np.full(nbx, -np.inf)
    gmax = np.full(nby, -np.inf)
    for I in range(nbx):
        sl = slice(I * B, min((I + 1) * B, len(f)))
        pos = as_[sl] > 0
        if pos.any():
            fmax[I] = f[sl][pos].max()
    for J in range(nby):
        sl = slice(J * B, min((J + 1) * B, len(g)))
        pos = bs[sl] > 0
        if pos.any():
            gmax[J] = g[sl][pos].max()
    gap = np.maximum(0.0, np.maximum(ylo[None, :, :] - xhi[:, None, :], xlo[:, None, :] - yhi[None, :, :]))
    dmin2 = (gap ** 2).sum(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        E = (fmax[:, None] + gmax[None, :] - dmin2) / eps
        lm = np.log(np.maximum(bmass[None, :] * nby, amass[:, None] * nbx))
        score = E + lm
    keep = score > math.log(delta) if delta > 0 else np.ones_like(score, dtype=bool)
    # every row block and every column block keeps its tile of largest bound
    keep[np.arange(nbx), np.argmax(score, axis=1)] = True
    keep[np.argmax(score, axis=0), np.arange(nby)] = True
    return keep


def masked_update(C, wk, pot, eps, mask):
    """c-transform over the rows of the cost C restricted to keys where mask[i, j] (a kept tile)."""
    with np.errstate(divide="ignore"):
        z = (pot[None, :] - C) / eps + np.log(wk)[None, :]
    z = np.where(mask, z, -np.inf)
    return -eps * logsumexp(z, axis=1)


def tile_mask(keep, B, n, m):
    return np.repeat(np.repeat(keep, B, axis=0)[:n], B, axis=1)[:, :m]


def sparse_residual(C, as_, bs, f, g, eps, mask):
    with np.errstate(over="ignore"):
        P = as_[:, None] * bs[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)
    P = np.where(mask, P, 0.0)
    return float(max(np.abs(P.sum(1) - as_).max(), np.abs(P.sum(0) - bs).max()))


def solve(x, y, a, b, eps, *, B=64, tol=1e-4, delta=1e-6, coarse_iters=20, max_rounds=10, coarse_gain=0.1,
          n_sample=256, max_iters=500, check_every=10, screen_every=10):
    """The two-stage solver.  Returns (f, g, info) with f, g in the caller's order."""
    x32, y32 = np.asarray(x, np.float32), np.asarray(y, np.float32)
    n, d = x32.shape
    m = y32.shape[0]
    lo = np.minimum(x32.min(axis=0), y32.min(axis=0))
    hi = np.maximum(x32.max(axis=0), y32.max(axis=0))
    px, py = morton_order(x32, lo, hi), morton_order(y32, lo, hi)
    xs, ys = x32[px].astype(np.float64), y32[py].astype(np.float64)
    as_, bs = np.asarray(a, np.float64)[px], np.asarray(b, np.float64)[py]
    xb, yb = blocks(xs, as_, B), blocks(ys, bs, B)
    amass, xcen = xb[0], xb[1]
    bmass, ycen = yb[0], yb[1]
    rows = sample_rows(n, n_sample)

    # coarse stage
    G = np.zeros(len(bmass))
    checks = []
    rounds = 0
    while True:
        F, G = sinkhorn_dense(xcen, ycen, amass, bmass, eps, coarse_iters, G)
        rounds += 1
        f = c_transform(xs, ycen, bmass, G, eps)
        g = c_transform(ys, xcen, amass, F, eps)
        checks.append(row_check(xs, ys, as_, bs, f, g, eps, rows))
        if checks[-1] <= tol or rounds >= max_rounds:
            break
        if len(checks) >= 2 and checks[-1] > (1.0 - coarse_gain) * checks[-2]:
            break

    # fine stage
    C = ((xs[:, None, :] - ys[None, :, :]) ** 2).sum(-1)
    keep = None
    resid = float("nan")
    it = 0
    kept_frac = []
    for it in range(1, max_iters + 1):
        if (it - 1) % screen_every == 0:
            keep = screen(f, g, as_, bs, B, xb, yb, eps, delta)
            kept_frac.append(float(keep.mean()))
            mask = tile_mask(keep, B, n, m)
        f = masked_update(C, bs, g, eps, mask)
        g = masked_update(C.T, as_, f, eps, mask.T)
        if it % check_every == 0 or it == max_iters:
            resid = sparse_residual(C, as_, bs, f, g, eps, mask)
            if resid <= tol:
                break
    fo, go = np.empty(n), np.empty(m)
    fo[px], go[py] = f, g
    info = dict(rounds=rounds, checks=checks, fine_iters=it, residual=resid, kept_fraction=kept_frac,
                perm_x=px, perm_y=py, keep=keep)
    return fo, go, info
