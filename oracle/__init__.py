"""CPU float64 oracle for dense log-domain Sinkhorn (squared-Euclidean cost).

TEST INFRASTRUCTURE ONLY.  The solver library never imports, links or calls
anything here; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  The arithmetic lives in ``sk_oracle.c`` (plain C, float64, difference
form of the cost, natural exp/log); this module compiles it with gcc on first
use and marshals numpy arrays.

Every function promotes its float32 inputs exactly to float64 and solves the
same problem the GPU solves: eps is taken as given (callers pass the float32
value of eps as a Python float).

Passages followed (page title and section):
  * "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodology 1
    (the log-domain update and its transpose), Methodology 2 (exact running
    max/sum-exp LSE), Methodology 3 (gradient as a barycentric projection).
  * SinkSLOT README, Tensor Contract (cost |x-y|^2, weights as given, zeros
    legal) and API Reference (alternating and symmetric variants, the fixed,
    marginal and potential stop modes, the infinity-norm marginal residual),
    Low-Level Solver API (iters_run, converged, final_viol), Basic Usage (the
    loss returns the primal value of the achieved plan), and the opening
    section (entropic OT is not zero at (x, x): the debiased divergence), Gradient Flow (descent on the
    analytic gradient).
Pins: every function here is checked in tests/test_oracle_pins.py against
closed forms, a textbook matrix-scaling route, library routines and brute
force; none is pinned only against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sk_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library (gcc, -O2, OpenMP)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building if missing or stale) the oracle library and declare signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or _LIB_PATH
        if path is None and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(p)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_half_step.argtypes = [_dp, i64, _dp, i64, i32, _dp, _dp, dbl, _i64p, i64, _dp]
        lib.oracle_half_step.restype = None
        lib.oracle_marginals.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, _dp, _dp, _dp, _dp]
        lib.oracle_marginals.restype = None
        lib.oracle_residual.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, _dp, _dp, _dp]
        lib.oracle_residual.restype = None
        lib.oracle_sinkhorn.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, i32, i32, _dp, _dp, _dp, _dp]
        lib.oracle_sinkhorn.restype = None
        lib.oracle_sinkhorn_ex.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, i32, dbl, i32, dbl, i32, i32, _dp,
                                           _dp, ctypes.POINTER(i32), ctypes.POINTER(i32), _dp]
        lib.oracle_sinkhorn_ex.restype = None
        lib.oracle_divergence.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, i32, dbl, i32, _dp]
        lib.oracle_divergence.restype = None
        lib.oracle_gradient_flow.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, i32, i32, dbl, _dp, _dp, _dp,
                                             _dp]
        lib.oracle_gradient_flow.restype = None
        lib.oracle_grad_x.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, _dp, _i64p, i64, _dp]
        lib.oracle_grad_x.restype = None
        lib.oracle_dual_cost.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, _dp, _dp]
        lib.oracle_dual_cost.restype = dbl
        lib.oracle_primal.argtypes = [_dp, _dp, _dp, _dp, i64, i64, i32, dbl, _dp, _dp, _dp]
        lib.oracle_primal.restype = None
        lib.oracle_max_cost.argtypes = [_dp, _dp, i64, i64, i32]
        lib.oracle_max_cost.restype = dbl
        if path is None:
            _lib = lib
        return lib


def _f64(v) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64))


def _ptr(v: np.ndarray):
    return v.ctypes.data_as(_dp)


def _cloud(v) -> np.ndarray:
    v = _f64(v)
    if v.ndim != 2:
        raise ValueError("point cloud must be 2-D (points, d)")
    if v.shape[1] > 256:
        raise ValueError("oracle supports d <= 256")
    return v


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def half_step(qry, key, w_key, pot_key, eps: float, idx=None, lib=None) -> np.ndarray:
    """c-transform: out_i = -eps log sum_j w_j exp((pot_j - |q_i - k_j|^2)/eps).

    Row half-step: half_step(x, y, b, g, eps) -> f.  Column: half_step(y, x, a, f, eps) -> g.
    ``idx`` restricts the output to those query rows (in that order).
    """
    lib = lib or load()
    q, k = _cloud(qry), _cloud(key)
    w, p = _f64(w_key), _f64(pot_key)
    assert q.shape[1] == k.shape[1] and w.shape == (k.shape[0],) and p.shape == (k.shape[0],)
    if idx is None:
        out = np.empty(q.shape[0])
        lib.oracle_half_step(_ptr(q), q.shape[0], _ptr(k), k.shape[0], q.shape[1], _ptr(w), _ptr(p),
                             float(eps), None, q.shape[0], _ptr(out))
    else:
        ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
        assert ix.size == 0 or (ix.min() >= 0 and ix.max() < q.shape[0])
        out = np.empty(ix.size)
        lib.oracle_half_step(_ptr(q), q.shape[0], _ptr(k), k.shape[0], q.shape[1], _ptr(w), _ptr(p),
                             float(eps), ix.ctypes.data_as(_i64p), ix.size, _ptr(out))
    return out


def sinkhorn(x, y, a, b, eps: float, n_iters: int, check_every: int = 0, g_init=None, lib=None):
    """Fixed-count alternating Sinkhorn from g = g_init (default 0), f first.

    Returns (f, g, resid_trace); resid_trace[k] is the residual after iteration
    (k+1)*check_every (empty when check_every == 0).
    """
    lib = lib or load()
    x, y, a, b = _cloud(x), _cloud(y), _f64(a), _f64(b)
    n, d = x.shape
    m = y.shape[0]
    f, g = np.empty(n), np.empty(m)
    nt = n_iters // check_every if check_every > 0 else 0
    trace = np.zeros(max(nt, 1))
    gi = None if g_init is None else _f64(g_init)
    lib.oracle_sinkhorn(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), int(check_every),
                        None if gi is None else _ptr(gi), _ptr(f), _ptr(g), _ptr(trace))
    return f, g, trace[:nt]


VARIANTS = {"alternating": 0, "symmetric": 1}
STOP_MODES = {"fixed": 0, "marginal": 1, "potential": 2}


def sinkhorn_ex(x, y, a, b, eps: float, *, variant: str = "alternating", alpha: float = 0.5,
                stop_mode: str = "fixed", stop_tol: float = 1e-6, max_iter: int = 200, check_every: int = 5, lib=None):
    """Sinkhorn with update variant and stop rule.  Returns (f, g, iters_run, converged, final_viol);
    converged is None and final_viol NaN under stop_mode="fixed"."""
    lib = lib or load()
    x, y, a, b = _cloud(x), _cloud(y), _f64(a), _f64(b)
    n, d = x.shape
    m = y.shape[0]
    f, g = np.empty(n), np.empty(m)
    it, conv, viol = ctypes.c_int(), ctypes.c_int(), ctypes.c_double()
    lib.oracle_sinkhorn_ex(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), VARIANTS[variant], float(alpha),
                           STOP_MODES[stop_mode], float(stop_tol), int(max_iter), int(check_every), _ptr(f), _ptr(g),
                           ctypes.byref(it), ctypes.byref(conv), ctypes.byref(viol))
    return f, g, it.value, (None if conv.value < 0 else bool(conv.value)), viol.value


def divergence(x, y, a, b, eps: float, n_iters: int, variant: str = "alternating", alpha: float = 0.5, lib=None):
    """Debiased entropic divergence OT(x,y) - OT(x,x)/2 - OT(y,y)/2, each term the dual objective after
    n_iters iterations of the given variant (fixed stop).  Returns (S, (OT_xy, OT_xx, OT_yy))."""
    lib = lib or load()
    x, y, a, b = _cloud(x), _cloud(y), _f64(a), _f64(b)
    out = np.empty(4)
    lib.oracle_divergence(_ptr(x), _ptr(y), _ptr(a), _ptr(b), x.shape[0], y.shape[0], x.shape[1], float(eps),
                          VARIANTS[variant], float(alpha), int(n_iters), _ptr(out))
    return float(out[0]), tuple(float(v) for v in out[1:])


def marginals(x, y, a, b, f, g, eps: float, lib=None):
    """(P1, P^T 1) of P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps)."""
    lib = lib or load()
    x, y, a, b, f, g = _cloud(x), _cloud(y), _f64(a), _f64(b), _f64(f), _f64(g)
    rs, cs = np.empty(x.shape[0]), np.empty(y.shape[0])
    lib.oracle_marginals(_ptr(x), _ptr(y), _ptr(a), _ptr(b), x.shape[0], y.shape[0], x.shape[1], float(eps),
                         _ptr(f), _ptr(g), _ptr(rs), _ptr(cs))
    return rs, cs


def residual(x, y, a, b, f, g, eps: float, lib=None) -> np.ndarray:
    """[linf_row, linf_col, l1_row, l1_col] of (P1 - a, P^T 1 - b)."""
    lib = lib or load()
    x, y, a, b, f, g = _cloud(x), _cloud(y), _f64(a), _f64(b), _f64(f), _f64(g)
    out = np.empty(4)
    lib.oracle_residual(_ptr(x), _ptr(y), _ptr(a), _ptr(b), x.shape[0], y.shape[0], x.shape[1], float(eps),
                        _ptr(f), _ptr(g), _ptr(out))
    return out


def grad_x(x, y, a, b, g, eps: float, idx=None, lib=None) -> np.ndarray:
    """grad_i = 2 a_i (x_i - sum_j w_ij y_j), w_i. = softmax_j((g_j - C_ij)/eps + log b_j)."""
    lib = lib or load()
    x, y, a, b, g = _cloud(x), _cloud(y), _f64(a), _f64(b), _f64(g)
    n, d = x.shape
    if idx is None:
        out = np.empty((n, d))
        lib.oracle_grad_x(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, y.shape[0], d, float(eps), _ptr(g),
                          None, n, _ptr(out))
    else:
        ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
        assert ix.size == 0 or (ix.min() >= 0 and ix.max() < n)
        out = np.empty((ix.size, d))
        lib.oracle_grad_x(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, y.shape[0], d, float(eps), _ptr(g),
                          ix.ctypes.data_as(_i64p), ix.size, _ptr(out))
    return out


def gradient_flow(x, y, a, b, eps: float, n_iters: int, n_steps: int, lr: float, lib=None):
    """n_steps of x <- x - lr * grad_x, each at a fresh n_iters-iteration solve.

    Returns (x_final, cost_trace, f, g, grad) with f, g, grad of the last step."""
    lib = lib or load()
    x = _cloud(x).copy()
    y, a, b = _cloud(y), _f64(a), _f64(b)
    n, d = x.shape
    m = y.shape[0]
    f, g, grad = np.empty(n), np.empty(m), np.empty((n, d))
    trace = np.empty(max(n_steps, 1))
    lib.oracle_gradient_flow(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), int(n_steps),
                             float(lr), _ptr(trace), _ptr(f), _ptr(g), _ptr(grad))
    return x, trace[:n_steps], f, g, grad


def dual_cost(x, y, a, b, f, g, eps: float, lib=None) -> float:
    """D(f,g) = <a,f> + <b,g> - eps (sum_ij P_ij - sum(a) sum(b))."""
    lib = lib or load()
    x, y, a, b, f, g = _cloud(x), _cloud(y), _f64(a), _f64(b), _f64(f), _f64(g)
    return float(lib.oracle_dual_cost(_ptr(x), _ptr(y), _ptr(a), _ptr(b), x.shape[0], y.shape[0], x.shape[1],
                                      float(eps), _ptr(f), _ptr(g)))


def primal(x, y, a, b, f, g, eps: float, lib=None):
    """(<P,C> + eps KL(P | a x b), <P,C>) of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps), with the
    generalised KL(P | Q) = sum P log(P/Q) - P + Q."""
    lib = lib or load()
    x, y, a, b, f, g = _cloud(x), _cloud(y), _f64(a), _f64(b), _f64(f), _f64(g)
    out = np.empty(2)
    lib.oracle_primal(_ptr(x), _ptr(y), _ptr(a), _ptr(b), x.shape[0], y.shape[0], x.shape[1], float(eps),
                      _ptr(f), _ptr(g), _ptr(out))
    return float(out[0]), float(out[1])


def max_cost(x, y, lib=None) -> float:
    """max_ij |x_i - y_j|^2 by exhaustive scan."""
    lib = lib or load()
    x, y = _cloud(x), _cloud(y)
    return float(lib.oracle_max_cost(_ptr(x), _ptr(y), x.shape[0], y.shape[0], x.shape[1]))


def max_cost_hull(x, y) -> float:
    """max_ij |x_i - y_j|^2 for large low-dimensional clouds.

    |x - y|^2 is convex in y, so for every x its maximum over the cloud y is
    attained at a vertex of y's convex hull; scanning x against those vertices
    is exact.  Requires d >= 2 (scipy's Qhull).
    """
    from scipy.spatial import ConvexHull

    xv, yv = _f64(x), _f64(y)
    verts = yv[ConvexHull(yv).vertices]
    return max_cost(xv, verts)
