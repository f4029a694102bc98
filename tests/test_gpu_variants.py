"""GPU parity of the update variants, stop rules, general dual cost and debiased
divergence (SinkSLOT README: API Reference, Low-Level Solver API, opening
section) against the CPU float64 oracle, through the C ABI.

Tolerances
  * potentials after the same iterations: max|f - f*|, max|g - g*| <= 1e-4 max C
    (as for the fixed alternating solve);
  * a stop decision is an integer taken from a floating-point check value; the
    cases pick the tolerance between two consecutive oracle check values that
    are far apart compared with the error the GPU's value can carry (the
    bound below), so both sides must stop at the same iteration;
  * check values: the marginal residual of potentials that differ by dp from
    the oracle's differs by at most (max w + r) expm1(2 dp / eps) plus the
    float32 exponent error 32 kappa (max w + r), kappa = 2^-24 (max|f| + max|g|
    + max C) / eps; the potential change differs by at most 2 dp;
  * costs: relative 1e-4, as for the plain cost; the dual cost at the same
    float32 potentials: eps * mass * 32 kappa from the exponent of each plan
    entry (all sums are float64).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_solver_amd as sk
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


def gpu_ex(x, y, a, b, eps, **kw):
    X, Y, A, B = dev(x, y, a, b)
    f, g, it, conv, viol = sk.solve_ex(X, Y, A, B, eps=eps, **kw)
    return host(f), host(g), it, conv, viol


# ------------------------------------------------------------------ fixed stop
FIXED_EQ = [(1500, 1300, 3, 0.05, 12, 1), (300, 257, 2, 0.05, 9, 2), (900, 700, 64, 0.5, 6, 3)]


@pytest.mark.parametrize("shape", FIXED_EQ, ids=[f"{s[0]}x{s[1]}d{s[2]}" for s in FIXED_EQ])
def test_fixed_alternating_equals_plain_solve(shape):
    """stop_mode fixed with the alternating variant runs the same kernels as sk_solve: equal bit for bit."""
    n, m, d, eps, iters, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d))
    eps = eps32(eps)
    say("fixed alternating", shape)
    X, Y, A, B = dev(x, y, a, b)
    f0, g0, _ = sk.solve(X, Y, A, B, eps=eps, n_iters=iters)
    f1, g1, it, conv, viol = sk.solve_ex(X, Y, A, B, eps=eps, max_iter=iters)
    assert it == iters and conv is None and viol is None
    assert torch.equal(f0, f1) and torch.equal(g0, g1)


SYM_SHAPES = [
    # n, m, d, eps, iters, alpha, seed, zero_frac
    (1, 1, 2, 0.1, 5, 0.5, 11, 0.0),
    (1, 9, 3, 0.1, 6, 0.5, 12, 0.0),
    (300, 257, 2, 0.05, 15, 0.5, 13, 0.0),
    (2500, 3100, 3, 0.05, 20, 0.5, 14, 0.1),
    (3100, 2500, 5, 0.3, 12, 0.3, 15, 0.0),
    (2000, 1700, 2, 0.02, 25, 1.0, 16, 0.0),
    (1500, 1700, 16, 0.3, 10, 0.5, 17, 0.0),
    (1200, 1100, 64, 0.5, 10, 0.7, 18, 0.05),
    (300, 500, 130, 0.5, 6, 0.5, 19, 0.0),
]


@pytest.mark.parametrize("shape", SYM_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}a{s[5]}" for s in SYM_SHAPES])
def test_symmetric_fixed_matches_oracle(shape):
    n, m, d, eps, iters, alpha, seed, zf = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.2, zero_frac=zf)
    eps = eps32(eps)
    say("symmetric fixed", shape)
    f, g, it, conv, viol = gpu_ex(x, y, a, b, eps, variant="symmetric", alpha=alpha, max_iter=iters)
    fo, go, *_ = oracle.sinkhorn_ex(x, y, a, b, eps, variant="symmetric", alpha=alpha, max_iter=iters)
    tol = 1e-4 * oracle.max_cost(x, y)
    say("err/tol f", np.max(np.abs(f - fo)) / tol, "g", np.max(np.abs(g - go)) / tol)
    assert it == iters and conv is None and viol is None
    assert np.max(np.abs(f - fo)) <= tol and np.max(np.abs(g - go)) <= tol


def test_symmetric_problem_keeps_f_equal_g():
    """On (x, x, a, a) the two Jacobi passes are the same computation: f equals g bit for bit."""
    x, _, a, _ = random_problem(2100, 2100, 3, 21)
    f, g, *_ = gpu_ex(x, x, a, a, eps32(0.05), variant="symmetric", alpha=0.5, max_iter=9)
    assert np.array_equal(f, g)


# ------------------------------------------------------------------ stop rules
STOP_CASES = [
    # n, m, d, eps, variant, alpha, rule, check_every, seed
    (1800, 1500, 2, 0.1, "alternating", 1.0, "marginal", 5, 31),
    (1800, 1500, 3, 0.1, "symmetric", 0.5, "marginal", 12, 32),
    (1000, 1200, 64, 0.1, "alternating", 1.0, "marginal", 1, 33),
    (1000, 1200, 64, 0.5, "symmetric", 0.6, "marginal", 3, 34),
    (1800, 1500, 2, 0.1, "alternating", 1.0, "potential", 5, 35),
    (1800, 1500, 3, 0.1, "symmetric", 0.5, "potential", 4, 36),
    (1000, 1200, 64, 0.5, "symmetric", 0.6, "potential", 3, 37),
]


@pytest.mark.parametrize("case", STOP_CASES, ids=[f"{c[4][:3]}-{c[6][:3]}-d{c[2]}" for c in STOP_CASES])
def test_stop_rule_matches_oracle(case):
    """The tolerance is put between the first two consecutive oracle check values that are
    well apart (factor 1.4 for the residual, 20 % for the potential change) and, for the
    residual, far above the float32 floor 32 kappa max(w); both sides must stop at the same
    check, with the GPU's check value within the bound that its measured potential error
    implies, and that bound must keep the GPU's value on the same side."""
    n, m, d, eps, variant, alpha, rule, c, seed = case
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.3)
    eps = eps32(eps)
    maxc = oracle.max_cost(x, y)
    vals, prev, pick = [], (np.zeros(n), np.zeros(m)), None
    for k in range(c, 30 * c + 1, c):
        f, g, *_ = oracle.sinkhorn_ex(x, y, a, b, eps, variant=variant, alpha=alpha, max_iter=k)
        if rule == "marginal":
            r = oracle.residual(x, y, a, b, f, g, eps)
            vals.append(max(r[0], r[1]))
        else:
            vals.append(max(np.abs(f - prev[0]).max(), np.abs(g - prev[1]).max()))
        prev = (f, g)
        if len(vals) >= 2:
            hi, lo = vals[-2], vals[-1]
            floor = 32 * kappa(f, g, maxc, eps) * max(a.max(), b.max())
            apart = hi >= 1.4 * lo and lo >= 8 * floor if rule == "marginal" else hi - lo >= 0.2 * hi
            if apart and min(vals[:-1]) == hi:
                pick = (len(vals), math.sqrt(hi * lo) if rule == "marginal" else 0.5 * (hi + lo))
                break
    assert pick is not None, f"no well-separated checks among {vals}"
    n_checks, stol = pick
    say("stop", case, "check", n_checks, "tol", stol, "values", vals[-2:])
    fo, go, it_o, conv_o, viol_o = oracle.sinkhorn_ex(x, y, a, b, eps, variant=variant, alpha=alpha,
                                                      stop_mode=rule, stop_tol=stol, max_iter=30 * c,
                                                      check_every=c)
    assert it_o == n_checks * c and conv_o
    f, g, it, conv, viol = gpu_ex(x, y, a, b, eps, variant=variant, alpha=alpha, stop_mode=rule, stop_tol=stol,
                                  max_iter=30 * c, check_every=c)
    dp = max(np.abs(f - fo).max(), np.abs(g - go).max())
    if rule == "marginal":
        bound = (max(a.max(), b.max()) + viol_o) * (math.expm1(2 * dp / eps) + 32 * kappa(f, g, maxc, eps))
    else:
        bound = 2 * dp
    say("iters", it, it_o, "viol", viol, viol_o, "bound", bound, "dp/maxC", dp / maxc)
    assert it == it_o and conv is True
    assert dp <= 1e-4 * maxc
    assert abs(viol - viol_o) <= bound
    assert viol_o + bound < stol  # the GPU's value could not have landed on the other side


@pytest.mark.parametrize("size", [(1300, 1100), (2200, 2000)], ids=["deferred", "immediate"])
@pytest.mark.parametrize("variant", ["alternating", "symmetric"])
@pytest.mark.parametrize("rule", ["marginal", "potential"])
def test_stop_rule_cap_and_state(variant, rule, size):
    """An unreachable tolerance runs to the cap (not a multiple of the interval; the last
    iteration is checked too), and an early stop leaves exactly the state of a fixed run --
    both where checks are read one interval late (small problems) and where they are read at
    once (above 4.2e6 pairs per pass)."""
    x, y, a, b = random_problem(size[0], size[1], 3, 41, shift=0.3)
    eps = eps32(0.1)
    c, cap = 4, 10
    say("cap", variant, rule)
    f, g, it, conv, viol = gpu_ex(x, y, a, b, eps, variant=variant, stop_mode=rule, stop_tol=0.0, max_iter=cap,
                                  check_every=c)
    assert it == cap and conv is False and math.isfinite(viol) and viol > 0.0
    ff, gf, *_ = gpu_ex(x, y, a, b, eps, variant=variant, max_iter=cap)
    assert np.array_equal(f, ff) and np.array_equal(g, gf)
    # a huge tolerance stops at the first check, with the potentials of a fixed run of c iterations
    f1, g1, it1, conv1, _ = gpu_ex(x, y, a, b, eps, variant=variant, stop_mode=rule, stop_tol=1e30, max_iter=cap,
                                   check_every=c)
    fc, gc, *_ = gpu_ex(x, y, a, b, eps, variant=variant, max_iter=c)
    assert it1 == c and conv1 is True
    assert np.array_equal(f1, fc) and np.array_equal(g1, gc)
    # a tolerance met first at the second check (between its value and the first's): that check's state
    _, _, _, _, v1 = gpu_ex(x, y, a, b, eps, variant=variant, stop_mode=rule, stop_tol=0.0, max_iter=c,
                            check_every=c)
    _, _, _, _, v2 = gpu_ex(x, y, a, b, eps, variant=variant, stop_mode=rule, stop_tol=0.0, max_iter=2 * c,
                            check_every=c)
    if v2 < v1:
        tol2 = 0.5 * (v1 + v2)
        f2, g2, it2, conv2, vv = gpu_ex(x, y, a, b, eps, variant=variant, stop_mode=rule, stop_tol=tol2,
                                        max_iter=cap, check_every=c)
        f2c, g2c, *_ = gpu_ex(x, y, a, b, eps, variant=variant, max_iter=2 * c)
        assert it2 == 2 * c and conv2 is True and vv == v2
        assert np.array_equal(f2, f2c) and np.array_equal(g2, g2c)


def test_stop_rule_zero_iterations_and_capture_refusal():
    x, y, a, b = random_problem(200, 300, 2, 43)
    f, g, it, conv, viol = gpu_ex(x, y, a, b, eps32(0.1), stop_mode="marginal", max_iter=0)
    assert it == 0 and conv is False and math.isnan(viol)
    assert np.all(f == 0.0) and np.all(g == 0.0)
    X, Y, A, B = dev(x, y, a, b)
    ws = sk.workspace(200, 300, 2, X.device)
    F, G = torch.empty(200, device=DEV), torch.empty(300, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(ValueError, match="SK_ERR_CAPTURE"):
        with torch.cuda.graph(graph):
            sk.solve_ex(X, Y, A, B, eps=eps32(0.1), stop_mode="potential", max_iter=5, ws=ws, f=F, g=G, check=False)


# ------------------------------------------------------------------ dual cost, divergence
DUAL_SHAPES = [(1700, 1300, 2, 0.05, 51), (900, 1100, 5, 0.2, 52), (800, 1000, 64, 0.5, 53), (1, 7, 3, 0.1, 54)]


@pytest.mark.parametrize("shape", DUAL_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}" for s in DUAL_SHAPES])
def test_dual_cost_matches_oracle(shape):
    """General dual objective at non-converged symmetric-variant potentials (plan mass != sum b)."""
    n, m, d, eps, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.2, zero_frac=0.05)
    eps = eps32(eps)
    say("dual cost", shape)
    f, g, *_ = gpu_ex(x, y, a, b, eps, variant="symmetric", alpha=0.5, max_iter=3)
    X, Y, A, B, F, G = dev(x, y, a, b, f.astype(np.float32), g.astype(np.float32))
    c = float(host(sk.dual_cost(X, Y, A, B, F, G, eps=eps))[0])
    want = oracle.dual_cost(x, y, a, b, f, g, eps)
    rs, _ = oracle.marginals(x, y, a, b, f, g, eps)
    mass = rs.sum()
    k = kappa(f, g, oracle.max_cost(x, y), eps)
    say("dual err", abs(c - want), "bound", eps * mass * 32 * k, "mass-1", mass - 1.0)
    assert abs(c - want) <= eps * mass * 32 * k + 1e-12


DIV_SHAPES = [
    # n, m, d, eps, iters, variant, seed
    (1500, 1100, 2, 0.05, 30, "alternating", 61),
    (900, 1300, 3, 0.1, 20, "symmetric", 62),
    (700, 600, 64, 0.5, 10, "alternating", 63),
    (1, 5, 3, 0.2, 5, "alternating", 64),
]


@pytest.mark.parametrize("shape", DIV_SHAPES, ids=[f"{s[0]}x{s[1]}d{s[2]}{s[5][:3]}" for s in DIV_SHAPES])
def test_divergence_matches_oracle(shape):
    n, m, d, eps, iters, variant, seed = shape
    x, y, a, b = random_problem(n, m, d, seed, scale=1.0 / math.sqrt(d), shift=0.3)
    eps = eps32(eps)
    say("divergence", shape)
    X, Y, A, B = dev(x, y, a, b)
    out = host(sk.divergence(X, Y, A, B, eps=eps, n_iters=iters, variant=variant))
    S, terms = oracle.divergence(x, y, a, b, eps, iters, variant=variant)
    for got, want in zip(out[1:], terms):
        assert abs(got - want) <= 1e-4 * abs(want) + 1e-9, (got, want)
    scale = abs(terms[0]) + 0.5 * abs(terms[1]) + 0.5 * abs(terms[2])
    say("S", out[0], S, "err/scale", abs(out[0] - S) / scale)
    assert abs(out[0] - S) <= 1e-4 * scale
    assert out[0] == out[1] - 0.5 * out[2] - 0.5 * out[3]


def test_divergence_of_a_translate():
    """S(x, x + t) = |t|^2 at convergence (unit mass): the translated cost differs by a
    separable term whose integral is |t|^2; the self-terms are translation invariant."""
    x, _, a, _ = random_problem(2000, 2000, 3, 71, scale=0.5)
    t = np.array([0.25, -0.125, 0.0625], dtype=np.float32)  # exact in float32 next to these coordinates
    y = (x + t).astype(np.float32)
    eps = eps32(0.5)
    X, Y, A = dev(x, y, a)
    out = host(sk.divergence(X, Y, A, A, eps=eps, n_iters=200))
    shift = float(t.astype(np.float64) @ t.astype(np.float64))
    scale = abs(out[1]) + 0.5 * abs(out[2]) + 0.5 * abs(out[3])
    say("translate S", out[0], "|t|^2", shift, "err/scale", abs(out[0] - shift) / scale)
    assert abs(out[0] - shift) <= 1e-4 * scale


# ------------------------------------------------------------------ a NaN state is never converged
@pytest.mark.parametrize("rule", ["marginal", "potential"])
def test_nan_state_is_not_reported_converged(rule):
    """At an eps near the smallest the library accepts (1e-37: 2 log2(e)/eps is still finite in float32) and
    clouds spread over tens of units, the pre-scaled scores overflow to inf - inf = NaN, so the potentials
    become NaN.  Every check value taken from that state must then be NaN, and a NaN check never meets the
    tolerance: converged is False, final_viol NaN, the cap is run.  The same state gives a NaN residual trace
    and a NaN standalone residual."""
    x, y, a, b = random_problem(600, 500, 3, seed=41, scale=10.0)
    X, Y, A, B = dev(x, y, a, b)
    eps = 1e-37
    say("nan state", rule)
    f, g, it, conv, viol = sk.solve_ex(X, Y, A, B, eps=eps, stop_mode=rule, stop_tol=1e30, max_iter=6,
                                       check_every=2)
    fh, gh = host(f), host(g)
    assert np.isnan(fh).any() or np.isnan(gh).any()
    assert conv is False and math.isnan(viol) and it == 6
    _, _, tr = sk.solve(X, Y, A, B, eps=eps, n_iters=4, check_every=2)
    assert np.isnan(host(tr)).all()
    r = host(sk.marginal_residual(X, Y, A, B, f, g, eps=eps))
    assert np.isnan(r[0]) or np.isnan(r[1])


# ------------------------------------------------------------------ the process-wide pools under concurrent calls
def test_concurrent_calls_from_two_threads():
    """The library keeps two process-wide pools: pinned host slots for stop-rule check values and the events of
    the pass timing.  Calls from two host threads at once, each on its own stream, with stop rules (both the
    deferred and the immediate check path) and timing on, must return exactly what the same calls return one
    after the other."""
    import threading

    # two stop at their first check, two run to the cap
    cases = [(1300, 1100, 3, 61, "marginal", 1e30), (2200, 2000, 2, 62, "potential", 1e-9),
             (900, 700, 64, 63, "marginal", 0.0), (1500, 1600, 3, 64, "potential", 1e30)]
    probs = []
    for n, m, d, seed, rule, tol in cases:
        x, y, a, b = random_problem(n, m, d, seed, shift=0.3)
        probs.append((dev(x, y, a, b), rule, tol, eps32(0.1 if d < 64 else 0.5)))

    def run(k, out):
        (X, Y, A, B), rule, tol, eps = probs[k]
        f, g, it, conv, viol = sk.solve_ex(X, Y, A, B, eps=eps, stop_mode=rule, stop_tol=tol, max_iter=60,
                                           check_every=5)
        torch.cuda.current_stream().synchronize()
        out[k] = (f.cpu().numpy(), g.cpu().numpy(), it, conv, viol)

    seq = {}
    for k in range(len(cases)):
        run(k, seq)
    torch.cuda.synchronize()
    sk.timing_enable(True, 1)
    par, errs = {}, []

    def worker(ks):
        try:
            with torch.cuda.stream(torch.cuda.Stream()):
                for k in ks:
                    run(k, par)
        except Exception as e:  # surfaced below
            errs.append(e)

    threads = [threading.Thread(target=worker, args=([0, 2],)), threading.Thread(target=worker, args=([1, 3],))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    _, launches, _ = sk.timing_read()
    sk.timing_enable(False)
    assert not errs and all(not t.is_alive() for t in threads)
    assert launches > 0
    for k in range(len(cases)):
        fs, gs, its, cs, vs = seq[k]
        fp, gp, itp, cp, vp = par[k]
        say("concurrent", cases[k], its, itp)
        assert its == itp and cs == cp and vs == vp
        assert its == (5 if cases[k][5] > 1.0 else 60)
        assert np.array_equal(fs, fp) and np.array_equal(gs, gp)
