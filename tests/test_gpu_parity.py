"""GPU parity: the HIP library (through the C ABI, via the thin binding) against
the CPU float64 oracle on identical seeded float32 inputs.

Tolerances
  * potentials: max|f - f*|, max|g - g*| <= 1e-4 * max C  (end to end, same
    fixed iteration count from g = 0);
  * cost: relative error <= 1e-4;
  * single half-steps (sampled rows at full size): <= 1e-4 * max C / (2 K),
    so that, each half-step being 1-Lipschitz in the sup norm, K iterations of
    such steps stay within the end-to-end bound;
  * evaluations at identical inputs (gradient at the same g, residual at the
    same (f, g)) are bounded by the float32 precision of the exponent,
    kappa = 2^-24 (max|f| + max|g| + max C) / eps, which every float32 route
    to these quantities shares.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
from sk_inputs import WORKLOADS, eps32, make_inputs, random_problem

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


def gpu_solve(x, y, a, b, eps, iters, check_every=0):
    X, Y, A, B = dev(x, y, a, b)
    f, g, tr = sk.solve(X, Y, A, B, eps=eps, n_iters=iters, check_every=check_every)
    return host(f), host(g), host(tr)


def kappa(f, g, maxc, eps):
    return U32 * (np.abs(f).max() + np.abs(g).max() + maxc) / eps


SHAPES = [
    # n, m, d, eps, iters, seed, scale, zero_frac
    (1, 1, 1, 0.1, 3, 1, 1.0, 0.0),
    (1, 9, 2, 0.1, 4, 2, 1.0, 0.0),
    (9, 1, 3, 0.1, 4, 3, 1.0, 0.0),
    (257, 1023, 3, 0.05, 20, 4, 0.3, 0.0),
    (1025, 513, 2, 0.02, 30, 5, 1.0, 0.0),
    (2500, 3100, 1, 0.1, 10, 6, 1.0, 0.0),
    (2500, 3100, 2, 0.1, 10, 7, 1.0, 0.0),
    (2500, 3100, 3, 0.1, 10, 8, 1.0, 0.0),
    (3100, 2500, 4, 0.2, 10, 9, 1.0, 0.0),
    (2500, 3100, 5, 0.3, 10, 10, 1.0, 0.0),
    (2500, 3100, 6, 0.3, 10, 11, 1.0, 0.0),
    (2500, 3100, 7, 0.5, 10, 12, 1.0, 0.0),
    (2500, 3100, 8, 0.5, 10, 13, 1.0, 0.0),
    (3000, 2999, 3, 0.05, 15, 14, 0.5, 0.25),
    (4099, 130, 2, 0.01, 25, 15, 1.0, 0.0),
    # matrix-core path: d > 8, padded to 16, 32, 64, 128, 256
    (1500, 1700, 9, 0.2, 8, 16, 0.33, 0.0),
    (2000, 1100, 16, 0.3, 8, 17, 0.25, 0.1),
    (1200, 1300, 33, 0.3, 6, 18, 0.17, 0.0),
    (2100, 2300, 64, 0.5, 10, 19, 0.125, 0.0),
    (700, 900, 100, 0.5, 5, 20, 0.1, 0.0),
    (600, 700, 128, 0.5, 5, 21, 0.09, 0.0),
    (300, 500, 256, 0.5, 4, 22, 0.0625, 0.0),
    (17, 5, 64, 0.1, 3, 23, 0.125, 0.0),
    (1200, 1000, 40, 0.3, 6, 24, 0.15, 0.1),  # the fp16 split form with zero weights (keys of bias -inf)
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}z{s[7]}" for s in SHAPES])
def test_solve_matches_oracle(shape):
    n, m, d, eps, iters, seed, scale, zf = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=scale, shift=0.2, zero_frac=zf)
    eps = eps32(eps)
    say("solve", shape)
    f, g, _ = gpu_solve(x, y, a, b, eps, iters)
    fo, go, _ = oracle.sinkhorn(x, y, a, b, eps, iters)
    maxc = oracle.max_cost(x, y)
    tol = 1e-4 * maxc
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    say("err/tol f", np.max(np.abs(f - fo)) / tol, "g", np.max(np.abs(g - go)) / tol)
    assert np.max(np.abs(f - fo)) <= tol
    assert np.max(np.abs(g - go)) <= tol
    # cost: the library's float64 reduction at the GPU potentials vs the oracle's dual value
    F, G, A, B = dev(f.astype(np.float32), g.astype(np.float32), a, b)
    c_gpu = float(host(sk.cost(A, B, F, G, eps=eps))[0])
    c_or = oracle.dual_cost(x, y, a, b, fo, go, eps)
    assert abs(c_gpu - c_or) <= 1e-4 * abs(c_or) + 1e-12


# The matrix-core pass forms the cross term from a scaled two-part fp16 split of every coordinate (three
# products hh + hl + lh, fp32 accumulation; at P = 16 all four in two instructions): its error per term is a
# few float32 unit roundoffs. One iteration from g = 0 must then stay within a few float32 roundings of the
# exponent of the oracle's iterate: 4 kappa eps, kappa as above. (Emulated on the CPU for these inputs, the
# float32 rounding of q.y alone moves f by 0.04-0.14 kappa eps and the split, both clouds scaled by
# fl(sqrt(2 log2e / eps)), by 0.13-0.42 kappa eps, products summed exactly; keeping only the three largest
# products of a three-part bf16 split would move it by 2-21.)
SPLIT_SHAPES = [(1500, 1300, 16, 0.05, 81), (1500, 1300, 32, 0.05, 82), (1200, 1100, 64, 0.05, 83),
                (700, 900, 100, 0.05, 84), (600, 700, 128, 0.05, 85), (300, 500, 256, 0.05, 86),
                # ragged and tiny: partial 16-query blocks, a partial two-block step, one row or one key
                (33, 47, 64, 0.05, 87), (1, 7, 32, 0.05, 88), (9, 1, 100, 0.05, 89), (3, 5, 256, 0.05, 90)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}" for s in SPLIT_SHAPES])
def test_one_iteration_at_float32_precision(shape):
    n, m, d, eps, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.2)
    eps = eps32(eps)
    say("one iteration", shape)
    f, g, _ = gpu_solve(x, y, a, b, eps, 1)
    fo, go, _ = oracle.sinkhorn(x, y, a, b, eps, 1)
    maxc = oracle.max_cost(x, y)
    tol = 4 * eps * kappa(fo, go, maxc, eps)
    say("err/tol f", np.max(np.abs(f - fo)) / tol, "g", np.max(np.abs(g - go)) / tol)
    assert np.max(np.abs(f - fo)) <= tol
    assert np.max(np.abs(g - go)) <= tol


def test_gradient_flow_workload_end_to_end():
    """The 1000-point, eps = 0.01, 200-iteration problem in full, against a live oracle run."""
    w = WORKLOADS["gflow_d2"]
    x, y, a, b = make_inputs("gflow_d2")
    eps = eps32(w.eps)
    say("gflow_d2 full")
    X, Y, A, B = dev(x, y, a, b)
    f_t, g_t, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=w.n_iters)
    c_t = sk.cost(A, B, f_t, g_t, eps=eps)
    grad_t = sk.grad_x(X, Y, A, B, g_t, eps=eps)
    f, g, c, grad = host(f_t), host(g_t), float(host(c_t)[0]), host(grad_t)
    fo, go, _ = oracle.sinkhorn(x, y, a, b, eps, w.n_iters)
    maxc = oracle.max_cost(x, y)
    assert np.max(np.abs(f - fo)) <= 1e-4 * maxc
    assert np.max(np.abs(g - go)) <= 1e-4 * maxc
    c_or = oracle.dual_cost(x, y, a, b, fo, go, eps)
    assert abs(c - c_or) <= 1e-4 * abs(c_or)
    # gradient at the GPU's own g: evaluation parity
    gr_same = oracle.grad_x(x, y, a, b, g, eps)
    k = kappa(f, g, maxc, eps)
    tol_eval = 2 * a.max() * 16 * k * math.sqrt(maxc)
    assert np.max(np.abs(grad - gr_same)) <= tol_eval
    # end to end, with the bound implied by the potential error
    gr_or = oracle.grad_x(x, y, a, b, go, eps)
    dg = np.max(np.abs(g - go))
    tol_e2e = tol_eval + 2 * a.max() * 2 * math.sqrt(maxc) * math.expm1(2 * dg / eps)
    assert np.max(np.abs(grad - gr_or)) <= tol_e2e


# The split scales both clouds by fl(sqrt(2 log2e / eps)) and each by a power of two from its largest scaled
# |coordinate|, so the fp16 operands sit near the top of fp16's range at any data magnitude. These cases move
# that magnitude far from 1 on one side or both, mix dimensions 1e4 apart, put both clouds below the point
# where the power of two is capped (2^48), and collapse both clouds onto one point (largest |coordinate| 0);
# one iteration is held to the same 4 kappa eps.
def _scaled_problem(case):
    n, m, d = 700, 900, 64
    if case == "degenerate":
        x = np.full((5, d), 0.75, np.float32)
        return x, x[:3].copy(), np.full(5, 0.2, np.float32), np.full(3, 1.0 / 3.0, np.float32), 0.1
    x, y, a, b = random_problem(n, m, d, 91, scale=1.0 / math.sqrt(d), shift=0.2)
    if case == "tiny":
        return x * np.float32(1e-6), y * np.float32(1e-6), a, b, 5e-14
    if case == "huge":
        return x * np.float32(1e4), y * np.float32(1e4), a, b, 5e6
    if case == "unbalanced":
        return x * np.float32(1e-3), y * np.float32(1e3), a, b, 5e4
    if case == "vanishing":
        # scaled coordinates below 2^-38: the exponent of both clouds is capped, the score scale is 2^96
        return x * np.float32(1e-12), y * np.float32(1e-12), a, b, 1.0
    if case == "mixed_dims":
        x[:, : d // 2] *= np.float32(1e-4)
        y[:, : d // 2] *= np.float32(1e-4)
        return x, y, a, b, 0.02
    if case == "small_eps":
        return x, y, a, b, 2e-4
    raise ValueError(case)


@pytest.mark.parametrize("case", ["tiny", "huge", "unbalanced", "vanishing", "mixed_dims", "small_eps",
                                  "degenerate"])
def test_split_scales_at_extreme_magnitudes(case):
    x, y, a, b, eps = _scaled_problem(case)
    eps = eps32(eps)
    say("split scales", case)
    f, g, _ = gpu_solve(x, y, a, b, eps, 1)
    fo, go, _ = oracle.sinkhorn(x, y, a, b, eps, 1)
    maxc = oracle.max_cost(x, y)
    # kappa plus the float32 precision of the log-weights the biases carry (all that is left when the two
    # clouds are one point and f, g and the costs vanish)
    lw = max(np.abs(np.log2(a)).max(), np.abs(np.log2(b)).max())
    tol = 4 * eps * (kappa(fo, go, maxc, eps) + U32 * lw)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    say("err/tol f", np.max(np.abs(f - fo)) / tol, "g", np.max(np.abs(g - go)) / tol)
    assert np.max(np.abs(f - fo)) <= tol
    assert np.max(np.abs(g - go)) <= tol


GRAD_SHAPES = [(1, 5, 2, 0.1, 21), (700, 1300, 3, 0.05, 22), (2100, 2600, 2, 0.02, 23),
               (1500, 900, 5, 0.3, 24), (1200, 2000, 8, 0.5, 25),
               # matrix-core gradient (d > 8): lse pass + weighted key sums
               (900, 1100, 12, 0.3, 26), (1700, 1300, 64, 0.3, 27), (300, 700, 130, 0.5, 28), (5, 3, 64, 0.2, 29)]


@pytest.mark.parametrize("shape", GRAD_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}" for s in GRAD_SHAPES])
def test_grad_matches_oracle(shape):
    n, m, d, eps, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 if d <= 8 else 1.0 / math.sqrt(d), zero_frac=0.1)
    eps = eps32(eps)
    rng = np.random.default_rng(seed)
    g = (0.3 * rng.standard_normal(m)).astype(np.float32)
    say("grad", shape)
    X, Y, A, B, G = dev(x, y, a, b, g)
    grad = host(sk.grad_x(X, Y, A, B, G, eps=eps))
    want = oracle.grad_x(x, y, a, b, g, eps)
    maxc = oracle.max_cost(x, y)
    k = kappa(np.zeros(1), g, maxc, eps)
    assert np.all(grad[a == 0] == 0.0)
    say("grad err/tol", np.max(np.abs(grad - want)) / (2 * a.max() * 16 * k * math.sqrt(maxc)))
    assert np.max(np.abs(grad - want)) <= 2 * a.max() * 16 * k * math.sqrt(maxc)


RESID_SHAPES = [(600, 800, 2, 0.05, 7, 31), (2300, 1700, 3, 0.02, 12, 32), (1000, 1000, 6, 0.3, 3, 33),
                (1100, 900, 64, 0.02, 2, 34)]


@pytest.mark.parametrize("shape", RESID_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}" for s in RESID_SHAPES])
def test_marginal_residual_matches_oracle(shape):
    n, m, d, eps, iters, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), zero_frac=0.05)
    eps = eps32(eps)
    say("residual", shape)
    f, g, _ = gpu_solve(x, y, a, b, eps, iters)
    X, Y, A, B, F, G = dev(x, y, a, b, f.astype(np.float32), g.astype(np.float32))
    r = host(sk.marginal_residual(X, Y, A, B, F, G, eps=eps))
    ro = oracle.residual(x, y, a, b, f, g, eps)
    maxc = oracle.max_cost(x, y)
    k = kappa(f, g, maxc, eps)
    tol_inf = 32 * k * (max(a.max(), b.max()) + ro[:2].max())
    assert abs(r[0] - ro[0]) <= tol_inf
    assert abs(r[1] - ro[1]) <= tol_inf
    assert abs(r[2] - ro[2]) <= 32 * k * (a.sum() + ro[2])
    assert abs(r[3] - ro[3]) <= 32 * k * (b.sum() + ro[3])
    say("residual err/tol", abs(r[0] - ro[0]) / tol_inf, abs(r[1] - ro[1]) / tol_inf, "value/tol", ro[0] / tol_inf)
    assert ro[0] > 10 * tol_inf  # a residual well above the noise floor was compared


def test_residual_trace_matches_oracle_at_same_iterates():
    """The fused trace after iteration k equals the residual of the GPU's own
    (f_k, g_k) (deterministic prefixes) as the oracle evaluates it."""
    x, y, a, b = make_inputs("gauss_d2", n=2000, m=2000)
    eps = eps32(0.05)
    say("trace 2000x2000")
    _, _, tr = gpu_solve(x, y, a, b, eps, 30, check_every=10)
    assert tr.shape == (3,)
    maxc = oracle.max_cost(x, y)
    for idx, k in enumerate((10, 20, 30)):
        fk, gk, _ = gpu_solve(x, y, a, b, eps, k)
        ro = oracle.residual(x, y, a, b, fk, gk, eps)
        kap = kappa(fk, gk, maxc, eps)
        assert abs(tr[idx] - max(ro[0], ro[1])) <= 32 * kap * (a.max() + ro[0]), (k, tr[idx], ro)


# Sizes around one round of the one-workgroup reductions (1024 threads x 8 loads = 8192 elements) on each side.
REDUCTION_SHAPES = [(1, 7), (7, 8192), (1023, 8193), (8191, 300), (8192, 1), (8193, 9000), (16385, 64), (24577, 100)]


@pytest.mark.parametrize("n,m", REDUCTION_SHAPES)
def test_reductions_across_unroll_boundaries(n, m):
    """The cost equals its float64 sum at the GPU's own potentials, and the fused residual trace the oracle's
    residual at the same iterates, at sizes below, at and past whole rounds of the reductions' loads."""
    x, y, a, b = random_problem(n, m, 2, 97 + n % 13, zero_frac=0.05)
    eps = eps32(0.1)
    X, Y, A, B = dev(x, y, a, b)
    say("reductions", (n, m))
    f_t, g_t, tr_t = sk.solve(X, Y, A, B, eps=eps, n_iters=6, check_every=3)
    f, g, tr = host(f_t), host(g_t), host(tr_t)
    c = float(host(sk.cost(A, B, f_t, g_t, eps=eps))[0])
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    ka, kb = a != 0, b != 0  # zero weights add nothing (their potentials are not read)
    af, bg = np.dot(a64[ka], f[ka]), np.dot(b64[kb], g[kb])
    c_ref = float(af + bg - eps * b64.sum() * (1.0 - a64.sum()))
    scale = np.dot(a64[ka], np.abs(f[ka])) + np.dot(b64[kb], np.abs(g[kb])) + eps * b64.sum()
    say("cost err / scale", abs(c - c_ref) / scale)
    assert abs(c - c_ref) <= 1e-12 * scale
    ro = oracle.residual(x, y, a, b, f, g, eps)
    kap = kappa(f, g, oracle.max_cost(x, y), eps)
    assert tr.shape == (2,)
    assert abs(tr[-1] - max(ro[0], ro[1])) <= 32 * kap * (a.max() + ro[0]), (tr[-1], ro)


def test_deterministic_and_zero_iterations():
    x, y, a, b = random_problem(3000, 2000, 3, 41)
    say("determinism")
    f1, g1, t1 = gpu_solve(x, y, a, b, 0.05, 12, check_every=4)
    f2, g2, t2 = gpu_solve(x, y, a, b, 0.05, 12, check_every=4)
    assert np.array_equal(f1, f2) and np.array_equal(g1, g2) and np.array_equal(t1, t2)
    f0, g0, t0 = gpu_solve(x, y, a, b, 0.05, 0)
    assert np.all(f0 == 0) and np.all(g0 == 0) and t0.size == 0
    # check_every that does not divide n_iters: floor(n_iters / check_every) entries
    _, _, t3 = gpu_solve(x, y, a, b, 0.05, 13, check_every=4)
    assert t3.shape == (3,) and np.array_equal(t3, t1)


def test_check_inputs_rejects_bad_data():
    x, y, a, b = random_problem(100, 80, 2, 51)
    X, Y, A, B = dev(x, y, a, b)
    sk.check_inputs(X, Y, A, B)
    bad = A.clone()
    bad[3] = -1e-3
    with pytest.raises(ValueError, match="NEG_WEIGHT"):
        sk.check_inputs(X, Y, bad, B)
    with pytest.raises(ValueError, match="MASS_MISMATCH"):
        sk.check_inputs(X, Y, A * 1.01, B)
    with pytest.raises(ValueError, match="EMPTY"):
        sk.check_inputs(X, Y, A * 0, B * 0)
    xn = X.clone()
    xn[5, 1] = float("nan")
    with pytest.raises(ValueError, match="NONFINITE"):
        sk.check_inputs(xn, Y, A, B)
    with pytest.raises(ValueError, match="float32"):
        sk.solve(X.double(), Y.double(), eps=0.1, n_iters=2)
    # uniform default weights
    f, g, _ = sk.solve(X, Y, eps=0.1, n_iters=3)
    fo, go, _ = oracle.sinkhorn(x, y, np.full(100, 1 / 100), np.full(80, 1 / 80), eps32(0.1), 3)
    assert np.max(np.abs(host(f) - fo)) <= 1e-4 * oracle.max_cost(x, y)
