"""GPU parity of the streamed transport products and the Hessian-vector product
("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodology 3)
against the dense float64 oracle (oracle/transport.py), through the C ABI.

Tolerances (all at identical float32 inputs and potentials)
  * transport products: every plan entry carries the float32 error of its
    exponent, at most a few kappa relative, kappa = 2^-24 (max|f| + max|g| +
    max C) / eps; so |P v - (P v)*|_i <= 32 kappa (P |v|)_i, elementwise;
  * Hessian-vector product: relative 1e-4 of the magnitude of the terms it
    sums, S_i = 2 r_i |v_i| + (2/eps) sum_j P_ij (|phi_i| + |psi_j| + |Cdot_ij|)
    |y_j| (oracle values), once conjugate gradients has reduced its
    preconditioned residual below 1e-5; at sizes beyond the dense oracle the
    closed form for a common translation (H v)_i = 2 a_i t and the symmetry
    <u, H v> = <v, H u> are checked instead.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from oracle import transport as T
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


def kappa(f, g, maxc, eps):
    return U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps


def gpu_potentials(x, y, a, b, eps, iters):
    X, Y, A, B = dev(x, y, a, b)
    f, g, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=iters)
    return host(f).astype(np.float32), host(g).astype(np.float32)


TRANSPORT_CASES = [
    # n, m, d, eps, iters, k, transpose, seed, zero_frac
    (1, 5, 2, 0.2, 3, 1, False, 1, 0.0),
    (7, 1, 3, 0.2, 3, 2, True, 2, 0.0),
    (1100, 900, 2, 0.05, 10, 1, False, 3, 0.0),
    (1100, 900, 3, 0.1, 10, 4, True, 4, 0.1),
    (2600, 1900, 1, 0.1, 5, 3, False, 5, 0.0),
    (900, 1300, 5, 0.3, 5, 9, False, 6, 0.0),
    (1300, 700, 8, 0.5, 5, 11, True, 7, 0.05),
    (3000, 2500, 4, 0.2, 5, 7, False, 8, 0.0),
    # matrix cores (d > 8): a log-sum-exp pass, then weights <= 1 into a second MFMA
    (900, 700, 16, 0.3, 5, 1, False, 9, 0.0),
    (700, 900, 64, 0.5, 5, 70, True, 10, 0.05),
    (300, 500, 130, 0.5, 4, 5, False, 11, 0.0),
    (17, 5, 64, 0.2, 3, 3, True, 12, 0.0),
    (2600, 3100, 33, 0.3, 4, 16, False, 13, 0.0),
    (900, 800, 100, 0.5, 4, 40, False, 18, 0.0),  # a 64-column tile at P = 128
    (500, 600, 12, 0.3, 5, 20, True, 19, 0.05),   # two 16-column chunks at P = 16
    # one payload column on the vector ALUs inside the matrix-core kernel, split key range; its scores take
    # the fp16 split form (P = 32, 64, 128, 256 below)
    (1500, 2100, 64, 0.5, 5, 1, True, 14, 0.05),
    (2100, 1500, 130, 0.5, 4, 1, False, 15, 0.0),
    (1300, 1700, 20, 0.3, 5, 1, False, 16, 0.0),
    (1100, 900, 100, 0.5, 4, 1, True, 17, 0.0),
]


@pytest.mark.parametrize("case", TRANSPORT_CASES, ids=[f"{c[0]}x{c[1]}d{c[2]}k{c[5]}{'T' if c[6] else ''}"
                                                       for c in TRANSPORT_CASES])
def test_transport_matches_oracle(case):
    n, m, d, eps, iters, k, transpose, seed, zf = case
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.3, zero_frac=zf)
    eps = eps32(eps)
    f, g = gpu_potentials(x, y, a, b, eps, iters)
    rows_in = n if transpose else m
    v = np.random.default_rng(seed + 50).normal(size=(rows_in, k)).astype(np.float32)
    say("transport", case)
    X, Y, A, B, F, G, Vt = dev(x, y, a, b, f, g, v)
    got = host(sk.transport(X, Y, A, B, F, G, Vt, eps=eps, transpose=transpose))
    want = T.transport(x, y, a, b, f, g, eps, v, transpose=transpose)
    scale = T.transport(x, y, a, b, f, g, eps, np.abs(v), transpose=transpose)
    kap = kappa(f, g, oracle.max_cost(x, y), eps)
    err = np.abs(got - want)
    say("max err / bound", (err / (32 * kap * scale + 1e-30)).max(), "kappa", kap)
    assert np.all(err <= 32 * kap * scale + 1e-30)
    # vector form and the plan marginals
    if k == 1:
        one = np.ones(rows_in, dtype=np.float32)
        got1 = host(sk.transport(X, Y, A, B, F, G, dev(one)[0], eps=eps, transpose=transpose))
        rs, cs = oracle.marginals(x, y, a, b, f, g, eps)
        ref = cs if transpose else rs
        assert np.all(np.abs(got1 - ref) <= 32 * kap * ref + 1e-30)


# The matrix-core products split their payload into fp16 parts with a power of two per column: columns whose
# magnitudes lie 1e20 apart (and an all-zero one) must each keep the elementwise bound of their own column,
# which a single scale for all columns would lose to fp16 underflow. 40 columns: a 64-column tile with 24 padded.
COLUMN_SCALE_CASES = [(900, 700, 64, 0.5, 5, False, 21), (600, 800, 100, 0.4, 4, True, 22), (700, 500, 20, 0.3, 5, False, 23)]


@pytest.mark.parametrize("case", COLUMN_SCALE_CASES, ids=[f"{c[0]}x{c[1]}d{c[2]}{'T' if c[5] else ''}"
                                                          for c in COLUMN_SCALE_CASES])
def test_transport_payload_columns_far_apart(case):
    n, m, d, eps, iters, transpose, seed = case
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.3)
    eps = eps32(eps)
    f, g = gpu_potentials(x, y, a, b, eps, iters)
    rows_in = n if transpose else m
    k = 40 if d >= 64 else 16
    col_scale = np.array([10.0 ** (20 * ((c % 3) - 1)) for c in range(k)], dtype=np.float64)  # 1e-20, 1, 1e20
    v = np.random.default_rng(seed + 50).normal(size=(rows_in, k)) * col_scale
    v[:, 1] = 0.0
    v = v.astype(np.float32)
    say("transport columns far apart", case)
    X, Y, A, B, F, G, Vt = dev(x, y, a, b, f, g, v)
    got = host(sk.transport(X, Y, A, B, F, G, Vt, eps=eps, transpose=transpose))
    want = T.transport(x, y, a, b, f, g, eps, v, transpose=transpose)
    scale = T.transport(x, y, a, b, f, g, eps, np.abs(v), transpose=transpose)
    kap = kappa(f, g, oracle.max_cost(x, y), eps)
    err = np.abs(got - want)
    say("max err / bound", (err / (32 * kap * scale + 1e-300)).max(), "kappa", kap)
    assert np.all(got[:, 1] == 0.0)
    assert np.all(err <= 32 * kap * scale + 1e-300)


HVP_CASES = [
    # n, m, d, eps, solve iters, cg iters, seed
    (1, 6, 2, 0.3, 200, 20, 11),
    (300, 257, 2, 0.3, 300, 80, 12),
    (1100, 900, 3, 0.5, 300, 80, 13),
    (700, 600, 1, 0.2, 500, 150, 14),
    (500, 800, 8, 1.0, 200, 60, 15),
    (900, 700, 5, 0.5, 100, 80, 16),  # away from the optimum: the same formula at that plan
    # matrix cores (d > 8)
    (600, 500, 16, 0.5, 200, 80, 17),
    (500, 700, 64, 1.0, 200, 60, 18),
    (200, 300, 130, 1.0, 100, 60, 19),
    (1, 9, 64, 0.5, 50, 20, 20),
    (400, 500, 24, 0.5, 200, 60, 21),
    (300, 350, 100, 1.0, 100, 60, 22),
]


@pytest.mark.parametrize("case", HVP_CASES, ids=[f"{c[0]}x{c[1]}d{c[2]}" for c in HVP_CASES])
def test_hvp_matches_oracle(case):
    n, m, d, eps, iters, cg_iters, seed = case
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.3)
    eps = eps32(eps)
    f, g = gpu_potentials(x, y, a, b, eps, iters)
    v = np.random.default_rng(seed + 70).normal(size=(n, d)).astype(np.float32)
    say("hvp", case)
    X, Y, A, B, F, G, Vt = dev(x, y, a, b, f, g, v)
    out, res = sk.hvp(X, Y, A, B, F, G, Vt, eps=eps, cg_iters=cg_iters)
    got, cg_res = host(out), float(host(res)[0])
    want, parts = T.hvp(x, y, a, b, f, g, eps, v, return_parts=True)
    P = T.plan(x, y, a, b, f, g, eps)
    xd, yd = x.astype(np.float64), y.astype(np.float64)
    cdot = 2.0 * ((xd[:, None, :] - yd[None, :, :]) * v[:, None, :]).sum(axis=-1)
    terms = P * (np.abs(parts["phi"])[:, None] + np.abs(parts["psi"])[None, :] + np.abs(cdot))
    S = 2 * parts["r"][:, None] * np.abs(v) + (2.0 / eps) * (terms @ np.abs(yd))
    err = np.abs(got - want)
    say("cg residual", cg_res, "max err / (1e-4 S)", (err / (1e-4 * S + 1e-30)).max(), "|HV| max", np.abs(want).max())
    assert cg_res <= 1e-5
    assert np.all(err <= 1e-4 * S + 1e-30)


def test_hvp_translation_and_symmetry_at_size():
    """20k x 20k, d = 3, converged: (H v)_i = 2 a_i t for v_i = t, and <u, H v> = <v, H u>."""
    x, y, a, b = random_problem(20000, 20000, 3, 21, scale=0.5, shift=0.3)
    eps = eps32(0.2)
    X, Y, A, B = dev(x, y, a, b)
    F, G, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=300)
    r = host(sk.marginal_residual(X, Y, A, B, F, G, eps=eps))
    say("residual after 300 iterations", r[:2])
    t = np.array([0.5, -0.25, 0.125], dtype=np.float32)
    vt = np.tile(t, (20000, 1))
    out, res = sk.hvp(X, Y, A, B, F, G, dev(vt)[0], eps=eps, cg_iters=100)
    got = host(out)
    want = 2 * a[:, None].astype(np.float64) * t
    say("translation: max err", np.abs(got - want).max(), "scale", np.abs(want).max(), "cg", float(host(res)[0]))
    # observed 6e-6 relative (CG at its float32 floor)
    assert np.abs(got - want).max() <= 1e-4 * np.abs(want).max()
    rng = np.random.default_rng(22)
    u = rng.normal(size=(20000, 3)).astype(np.float32)
    v = rng.normal(size=(20000, 3)).astype(np.float32)
    Hv, _ = sk.hvp(X, Y, A, B, F, G, dev(v)[0], eps=eps, cg_iters=100)
    Hu, _ = sk.hvp(X, Y, A, B, F, G, dev(u)[0], eps=eps, cg_iters=100)
    lhs, rhs = float((u * host(Hv)).sum()), float((v * host(Hu)).sum())
    say("symmetry", lhs, rhs)
    # observed 1e-6 relative
    assert abs(lhs - rhs) <= 2e-5 * max(abs(lhs), abs(rhs))
