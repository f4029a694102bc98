"""Pins for the dense transport-product and Hessian-vector-product oracle
(oracle/transport.py): each function is checked against something other than
itself -- the C oracle's marginals and gradient, finite differences of the
converged gradient, symmetry of a Hessian, and closed forms -- and every
planted mistake in its source must trip at least one pin.

Source: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
Methodology 3 (transport products; Hessian-vector products built from them).
"""
import importlib.util

import numpy as np
import pytest

import oracle
from oracle import transport as T0

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _problem(n, m, d, seed, shift=0.5):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(n, d))
    y = rng.normal(size=(m, d)) * 0.8 + shift
    a, b = rng.exponential(size=n), rng.exponential(size=m)
    return x, y, a / a.sum(), b / b.sum()


def _converged(x, y, a, b, eps, iters=20000):
    f, g, _ = oracle.sinkhorn(x, y, a, b, eps, iters)
    assert oracle.residual(x, y, a, b, f, g, eps)[0] < 1e-13
    return f, g


def _grad(x, y, a, b, eps, iters=20000):
    _, g = _converged(x, y, a, b, eps, iters)
    return oracle.grad_x(x, y, a, b, g, eps)


# --------------------------------------------------------------------------- pins
def pin_transport_marginals(T):
    """P 1 and P^T 1 equal the C oracle's plan marginals (at arbitrary potentials)."""
    x, y, a, b = _problem(9, 7, 3, 1)
    rng = np.random.default_rng(2)
    f, g = rng.normal(size=9) * 0.3, rng.normal(size=7) * 0.3
    rs, cs = oracle.marginals(x, y, a, b, f, g, 0.4)
    assert np.allclose(T.transport(x, y, a, b, f, g, 0.4, np.ones(7)), rs, rtol=1e-13, atol=0)
    assert np.allclose(T.transport(x, y, a, b, f, g, 0.4, np.ones(9), transpose=True), cs, rtol=1e-13, atol=0)


def pin_transport_barycentre(T):
    """With f the c-transform of g the rows of P sum to a, and P Y is the barycentric numerator:
    the C oracle's gradient equals 2 (a x - P Y)."""
    x, y, a, b = _problem(8, 11, 2, 3)
    eps = 0.3
    g = np.random.default_rng(4).normal(size=11) * 0.2
    f = oracle.half_step(x, y, b, g, eps)
    PY = T.transport(x, y, a, b, f, g, eps, y)
    assert np.allclose(2 * (a[:, None] * x - PY), oracle.grad_x(x, y, a, b, g, eps), rtol=0, atol=1e-13)


def pin_transport_bruteforce(T):
    """Tiny case by explicit loops over i, j."""
    x, y, a, b = _problem(3, 2, 2, 5)
    f, g = np.array([0.1, -0.2, 0.05]), np.array([0.3, -0.1])
    V = np.array([[1.0, 2.0], [-0.5, 0.25]])
    U = np.array([[0.5], [1.5], [-1.0]])
    eps = 0.7
    want = np.zeros((3, 2))
    want_t = np.zeros((2, 1))
    for i in range(3):
        for j in range(2):
            c = sum((x[i, t] - y[j, t]) ** 2 for t in range(2))
            p = a[i] * b[j] * np.exp((f[i] + g[j] - c) / eps)
            want[i] += p * V[j]
            want_t[j] += p * U[i]
    assert np.allclose(T.transport(x, y, a, b, f, g, eps, V), want, rtol=1e-14, atol=0)
    assert np.allclose(T.transport(x, y, a, b, f, g, eps, U, transpose=True), want_t, rtol=1e-14, atol=0)


def pin_hvp_finite_difference(T):
    """H V equals the central difference of the converged gradient along V."""
    for (n, m, d, eps, seed) in [(7, 6, 2, 0.5, 11), (6, 9, 3, 0.8, 12), (10, 4, 1, 0.3, 13)]:
        x, y, a, b = _problem(n, m, d, seed)
        V = np.random.default_rng(seed + 100).normal(size=(n, d))
        f, g = _converged(x, y, a, b, eps)
        HV = T.hvp(x, y, a, b, f, g, eps, V)
        h = 1e-5
        fd = (_grad(x + h * V, y, a, b, eps) - _grad(x - h * V, y, a, b, eps)) / (2 * h)
        assert np.allclose(HV, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max())), (n, m, d)


def pin_hvp_symmetric(T):
    """<U, H V> = <V, H U> at the optimum (a Hessian is symmetric)."""
    x, y, a, b = _problem(8, 7, 2, 21)
    eps = 0.4
    f, g = _converged(x, y, a, b, eps)
    rng = np.random.default_rng(22)
    U, V = rng.normal(size=(8, 2)), rng.normal(size=(8, 2))
    lhs = (U * T.hvp(x, y, a, b, f, g, eps, V)).sum()
    rhs = (V * T.hvp(x, y, a, b, f, g, eps, U)).sum()
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


def pin_hvp_translation(T):
    """Moving every x_i by the same t adds a separable term to C, so F(x + s t) =
    F(x) + 2 s <sum a x - sum b y, t> + s^2 |t|^2 and (H V)_i = 2 a_i t for V_i = t."""
    x, y, a, b = _problem(9, 8, 3, 31)
    eps = 0.5
    f, g = _converged(x, y, a, b, eps)
    t = np.array([0.3, -1.2, 0.7])
    V = np.tile(t, (9, 1))
    assert np.allclose(T.hvp(x, y, a, b, f, g, eps, V), 2 * a[:, None] * t, rtol=0, atol=1e-12)


def pin_hvp_single_target(T):
    """One target point: F(x) = sum_i a_i |x_i - y|^2, so H V = 2 a V."""
    x, _, a, _ = _problem(6, 1, 2, 41)
    y = np.array([[0.2, -0.4]])
    f, g = _converged(x, y, a, np.ones(1), 0.3, iters=50)
    V = np.random.default_rng(42).normal(size=(6, 2))
    assert np.allclose(T.hvp(x, y, a, np.ones(1), f, g, 0.3, V), 2 * a[:, None] * V, rtol=0, atol=1e-12)


def pin_hvp_gauge(T):
    """The result does not depend on the gauge (f + c, g - c), also away from the optimum."""
    x, y, a, b = _problem(7, 8, 2, 51)
    f, g, _ = oracle.sinkhorn(x, y, a, b, 0.3, 5)
    V = np.random.default_rng(52).normal(size=(7, 2))
    h0 = T.hvp(x, y, a, b, f, g, 0.3, V)
    h1 = T.hvp(x, y, a, b, f + 0.37, g - 0.37, 0.3, V)
    assert np.allclose(h0, h1, rtol=0, atol=1e-11 * np.abs(h0).max())


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(T0)


MUTANTS = {
    "plan_cost_sign": ("(f[:, None] + g[None, :] - sq_cost(x, y)) / eps", "(f[:, None] + g[None, :] + sq_cost(x, y)) / eps"),
    "transpose_ignored": ("return (P.T if transpose else P) @ _f64(V)", "return P @ _f64(V)"),
    "hvp_no_row_term": ("HV = 2.0 * r[:, None] * V - (2.0 / eps) * (W @ y)", "HV = -(2.0 / eps) * (W @ y)"),
    "hvp_eps_factor": ("HV = 2.0 * r[:, None] * V - (2.0 / eps) * (W @ y)", "HV = 2.0 * r[:, None] * V - (1.0 / eps) * (W @ y)"),
    "hvp_cdot_sign": ("(x[:, None, :] - y[None, :, :]) * V[:, None, :]", "(y[None, :, :] - x[:, None, :]) * V[:, None, :]"),
    "hvp_no_phi": ("W = P * (phi[:, None] + psi[None, :] - Cdot)", "W = P * (psi[None, :] - Cdot)"),
    "hvp_no_psi": ("W = P * (phi[:, None] + psi[None, :] - Cdot)", "W = P * (phi[:, None] - Cdot)"),
    "hvp_no_cdot": ("W = P * (phi[:, None] + psi[None, :] - Cdot)", "W = P * (phi[:, None] + psi[None, :])"),
    "hvp_rhs_rows_only": ("rhs = np.concatenate([(P * Cdot).sum(axis=1), (P * Cdot).sum(axis=0)])",
                          "rhs = np.concatenate([(P * Cdot).sum(axis=1), 0.0 * (P * Cdot).sum(axis=0)])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(T0.__file__).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "transport_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("transport_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, np.linalg.LinAlgError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
