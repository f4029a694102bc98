"""Dense float64 reference for transport products and the Hessian-vector product.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the GPU library never
imports or calls it.  Everything is the definition written out with dense
numpy arrays -- the n x m plan is formed explicitly -- so it is meant for
small problems.

Source: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
Methodology 3 (transport-matrix application; a Hessian-vector product built
from transport-vector and transport-matrix products).  The pages give no
formula; the reading written out here is:

  * plan at potentials (f, g): P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps),
    C_ij = |x_i - y_j|^2;
  * transport products P V (V: m x k) and P^T U (U: n x k);
  * the Hessian of the entropic OT cost F(x) = OT_eps(x, y) with respect to
    the source points, applied to V (n x d), by implicit differentiation at
    the plan: with r = P 1, c = P^T 1 and Cdot_ij = 2 <x_i - y_j, V_i> (the
    derivative of C_ij along V), the potential derivatives (phi, psi) solve
        r_i phi_i + sum_j P_ij psi_j = sum_j P_ij Cdot_ij      (rows)
        sum_i P_ij phi_i + c_j psi_j = sum_i P_ij Cdot_ij      (columns)
    (the plan's marginals stay fixed; the system is singular along the gauge
    (phi + t, psi - t) and consistent), and
        (H V)_i = 2 r_i V_i - (2 / eps) sum_j P_ij (phi_i + psi_j - Cdot_ij) y_j,
    the derivative of the gradient G_i = 2 sum_j P_ij (x_i - y_j).  At the
    optimal (f, g) this is the exact Hessian; elsewhere it is the same formula
    at the given plan.  The linear system is solved with numpy's
    least-squares routine (minimum-norm solution); the result does not depend
    on the gauge.
"""
from __future__ import annotations

import numpy as np


def _f64(v):
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64))


def sq_cost(x, y):
    x, y = _f64(x), _f64(y)
    diff = x[:, None, :] - y[None, :, :]
    return (diff * diff).sum(axis=-1)


def plan(x, y, a, b, f, g, eps: float) -> np.ndarray:
    """P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) as a dense n x m array."""
    a, b, f, g = _f64(a), _f64(b), _f64(f), _f64(g)
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - sq_cost(x, y)) / eps)


def transport(x, y, a, b, f, g, eps: float, V, transpose: bool = False) -> np.ndarray:
    """P V (V: m x k, or a length-m vector) or, with transpose, P^T V (V: n x k)."""
    P = plan(x, y, a, b, f, g, eps)
    return (P.T if transpose else P) @ _f64(V)


def hvp(x, y, a, b, f, g, eps: float, V, return_parts: bool = False):
    """(H V) of the entropic OT cost in x at the plan of (f, g); V is n x d."""
    x, y, V = _f64(x), _f64(y), _f64(V)
    n, m = x.shape[0], y.shape[0]
    P = plan(x, y, a, b, f, g, eps)
    r, c = P.sum(axis=1), P.sum(axis=0)
    Cdot = 2.0 * ((x[:, None, :] - y[None, :, :]) * V[:, None, :]).sum(axis=-1)
    rhs = np.concatenate([(P * Cdot).sum(axis=1), (P * Cdot).sum(axis=0)])
    K = np.block([[np.diag(r), P], [P.T, np.diag(c)]])
    sol = np.linalg.lstsq(K, rhs, rcond=None)[0]
    phi, psi = sol[:n], sol[n:]
    W = P * (phi[:, None] + psi[None, :] - Cdot)
    HV = 2.0 * r[:, None] * V - (2.0 / eps) * (W @ y)
    if return_parts:
        return HV, dict(phi=phi, psi=psi, r=r, c=c, rhs=rhs, K=K)
    return HV
