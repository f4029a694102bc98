"""Streaming log-domain Sinkhorn on AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/sk.h`` (libsk.so): argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  There is no
CPU fallback: if libsk.so is missing or cannot be loaded, every call raises.

Tensor contract (SinkSLOT README, Tensor Contract): x (n, d) and y (m, d)
float32 point clouds, optional nonnegative weights a (n,), b (m,) -- uniform
if omitted, used exactly as given, sum(a) must equal sum(b) (ValueError
otherwise), zeros legal -- all on the same CUDA/HIP device.  float64 inputs
raise ValueError: the kernels are float32-only.  The cost is
C_ij = |x_i - y_j|^2 with no 1/2 factor; eps is measured against it.
Potentials are returned in cost units (f, g), not divided by eps.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libsk.so")

SK_OK = 0
_STATUS_NAMES = {
    0: "SK_OK", 1: "SK_ERR_NULL", 2: "SK_ERR_SHAPE", 3: "SK_ERR_UNSUPPORTED_D", 4: "SK_ERR_EPS",
    5: "SK_ERR_ITERS", 6: "SK_ERR_CHECK_EVERY", 7: "SK_ERR_NEG_WEIGHT", 8: "SK_ERR_MASS_MISMATCH",
    9: "SK_ERR_EMPTY_MEASURE", 10: "SK_ERR_NONFINITE", 11: "SK_ERR_WORKSPACE", 12: "SK_ERR_HIP",
    13: "SK_ERR_VARIANT", 14: "SK_ERR_STOP", 15: "SK_ERR_CAPTURE", 16: "SK_ERR_LR", 17: "SK_ERR_SCRATCH",
}
_VALUE_ERRORS = {1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 13, 14, 15, 16, 17}
NOALLOC_SCRATCH_BYTES = 64 << 20  # SK_NOALLOC_SCRATCH_BYTES of include/sk.h

# SinkSLOT README, API Reference: variant and stop_mode names
VARIANTS = {"alternating": 0, "symmetric": 1}
STOP_MODES = {"fixed": 0, "marginal": 1, "potential": 2}

# C ABI: (name, restype, argtypes)
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "sk_abi_version": (ctypes.c_int, []),
    "sk_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sk_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "sk_check_inputs": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _vp]),
    "sk_solve": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _vp, _vp, _i32, _vp, _vp, _sz,
                                _vp]),
    "sk_solve_warm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _vp, _vp, _vp, _i32, _vp,
                                     _vp, _sz, _vp]),
    "sk_solve_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _vp, _vp, _i32, _vp,
                                        _vp]),
    "sk_primal_cost": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sk_cost": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _vp]),
    "sk_marginal_residual": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _vp, _vp, _sz,
                                            _vp]),
    "sk_grad_x": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sk_solve_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _f32, _i32, _f32, _i32, _i32,
                                   _vp, _vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_f32), _vp,
                                   _sz, _vp]),
    "sk_dual_cost": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sk_divergence_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "sk_divergence": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _f32, _i32, _vp, _vp, _sz,
                                     _vp]),
    "sk_gradient_flow": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _i32, _f32, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]),
    "sk_transport_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "sk_transport": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _i32, _vp, _i32, _vp, _vp,
                                    _sz, _vp]),
    "sk_hvp": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz,
                              _vp]),
    "sk_fs2_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "sk_fs2_solve": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _i32, _f32, _f32, _i32, _i32, _f32,
                                    _i32, _i32, _i32, _i32, _vp, _vp, ctypes.POINTER(_i32), ctypes.POINTER(_f32), _vp,
                                    _vp, _vp, _sz, _vp]),
    "sk_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "sk_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_double)]),
}

_lock = threading.Lock()
_lib = None


class SinkhornError(RuntimeError):
    """A HIP failure inside the library."""


def load_library(path: str | None = None):
    """Load libsk.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"libsk.so not found at {p}; build it with "
                               "`python -m streaming_sinkhorn_solver_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def status_string(code: int) -> str:
    return load_library().sk_status_string(int(code)).decode()


def _raise(code: int, where: str):
    if code == SK_OK:
        return
    msg = f"{where}: {_STATUS_NAMES.get(code, code)} ({status_string(code)})"
    if code in _VALUE_ERRORS:
        raise ValueError(msg)
    raise SinkhornError(msg)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _buf(t, shape, dtype, device, name: str) -> torch.Tensor:
    """A caller-supplied output (checked: dtype, device, shape, contiguous) or a new one."""
    shape = tuple(int(k) for k in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor on {device}")
    if tuple(t.shape) != shape or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of shape {shape} (got {tuple(t.shape)})")
    return t


def _in(t, shape, device, name: str) -> torch.Tensor:
    """A float32 input of the given shape on the device, made contiguous."""
    shape = tuple(int(k) for k in shape)
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device:
        raise ValueError(f"{name} must be a float32 tensor on {device}")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape} (got {tuple(t.shape)})")
    return t.contiguous()


def _at_least(t, count: int, dtype, device, name: str) -> torch.Tensor:
    """A caller-supplied contiguous buffer of at least count elements (dtype, device checked)."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on {device}")
    if t.numel() < count:
        raise ValueError(f"{name} must hold at least {count} values")
    return t


def _ws(ws, device, make) -> torch.Tensor:
    """A caller-supplied workspace (a contiguous uint8 tensor on the device; the library checks its
    size and alignment) or a new one from make()."""
    if ws is None:
        return make()
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous uint8 tensor on {device}")
    return ws


def _as_problem(x, y, a, b):
    if not isinstance(x, torch.Tensor) or not isinstance(y, torch.Tensor):
        raise TypeError("x and y must be torch tensors")
    if x.dtype != torch.float32 or y.dtype != torch.float32:
        raise ValueError("the kernels are float32-only (got %s, %s)" % (x.dtype, y.dtype))
    if x.dim() != 2 or y.dim() != 2 or x.shape[1] != y.shape[1]:
        raise ValueError("x must be (n, d) and y (m, d) with the same d")
    if x.device.type != "cuda" or y.device != x.device:
        raise ValueError("x and y must be on the same GPU device")
    n, d = x.shape
    m = y.shape[0]
    if a is None:
        a = torch.full((n,), 1.0 / n, dtype=torch.float32, device=x.device)
    if b is None:
        b = torch.full((m,), 1.0 / m, dtype=torch.float32, device=x.device)
    for name, w, k in (("a", a, n), ("b", b, m)):
        if w.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 (got {w.dtype})")
        if w.shape != (k,) or w.device != x.device:
            raise ValueError(f"{name} must have shape ({k},) on {x.device}")
    return x.contiguous(), y.contiguous(), a.contiguous(), b.contiguous(), n, m, d


def workspace_bytes(n: int, m: int, d: int) -> int:
    return int(load_library().sk_workspace_bytes(n, m, d))


def workspace(n: int, m: int, d: int, device) -> torch.Tensor:
    """A workspace tensor for problems of this size (uint8, 256-byte aligned by torch's allocator)."""
    nb = workspace_bytes(n, m, d)
    if nb == 0:
        raise ValueError(f"invalid problem size n={n} m={m} d={d}")
    ws = torch.empty(nb, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("allocator returned a workspace that is not 256-byte aligned")
    return ws


def check_inputs(x, y, a=None, b=None, ws: torch.Tensor | None = None) -> None:
    """Validate the data (finite, nonnegative weights, equal nonzero masses); raises ValueError."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    _raise(lib.sk_check_inputs(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, _ptr(ws), ws.numel(),
                               _stream(x.device)), "sk_check_inputs")


def solve(x, y, a=None, b=None, *, eps: float, n_iters: int, check_every: int = 0,
          ws: torch.Tensor | None = None, f: torch.Tensor | None = None, g: torch.Tensor | None = None,
          trace: torch.Tensor | None = None, check: bool = True):
    """Fixed-count alternating log-domain Sinkhorn from g = 0.

    Returns (f, g, resid_trace); resid_trace holds n_iters // check_every
    marginal residuals (empty when check_every == 0).  Outputs are enqueued on
    the current stream.
    """
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    if check:
        check_inputs(x, y, a, b, ws)
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    nt = n_iters // check_every if check_every > 0 else 0
    if trace is None:
        trace = torch.empty(max(nt, 0), dtype=torch.float32, device=x.device)
    else:
        trace = _at_least(trace, nt, torch.float32, x.device, "trace")
    _raise(lib.sk_solve(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), _ptr(f), _ptr(g),
                        int(check_every), _ptr(trace) if nt > 0 else None, _ptr(ws), ws.numel(),
                        _stream(x.device)), "sk_solve")
    return f, g, trace


def solve_warm(x, y, a=None, b=None, *, eps: float, n_iters: int, g_init: torch.Tensor, check_every: int = 0,
               ws: torch.Tensor | None = None, f: torch.Tensor | None = None, g: torch.Tensor | None = None,
               trace: torch.Tensor | None = None, check: bool = True):
    """The fixed-count solve of ``solve`` started from g = g_init (m,) instead of 0; g_init may be g itself
    (continued in place).  Returns (f, g, resid_trace)."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    if check:
        check_inputs(x, y, a, b, ws)
    g_init = _in(g_init, (m,), x.device, "g_init")
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    nt = n_iters // check_every if check_every > 0 else 0
    if trace is None:
        trace = torch.empty(max(nt, 0), dtype=torch.float32, device=x.device)
    else:
        trace = _at_least(trace, nt, torch.float32, x.device, "trace")
    _raise(lib.sk_solve_warm(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), _ptr(g_init),
                             _ptr(f), _ptr(g), int(check_every), _ptr(trace) if nt > 0 else None, _ptr(ws),
                             ws.numel(), _stream(x.device)), "sk_solve_warm")
    return f, g, trace


def primal_cost(x, y, a, b, f, g, *, eps: float, ws: torch.Tensor | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """[<P,C> + eps KL(P | a x b), <P,C>] of the plan at (f, g), as a 2-element float64 tensor."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: transport_workspace(n, m, d, x.device))
    f, g = _potentials(f, g, n, m, x.device)
    out = _buf(out, (2,), torch.float64, x.device, "out")
    _raise(lib.sk_primal_cost(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(f), _ptr(g), _ptr(out),
                              _ptr(ws), ws.numel(), _stream(x.device)), "sk_primal_cost")
    return out


def solve_noalloc(x, y, a=None, b=None, *, eps: float, n_iters: int, f: torch.Tensor, g: torch.Tensor,
                  check_every: int = 0, trace: torch.Tensor | None = None):
    """sk_solve_noalloc: the fixed-count solve of ``solve`` in the library's static device scratch, with
    caller-supplied outputs (f (n,), g (m,) and, when check_every > 0, trace of n_iters // check_every
    floats).  Nothing is allocated, so the data checks of ``check_inputs`` (which need a workspace) are not
    run here; call it beforehand if the data may be invalid.  Problems whose workspace would exceed
    NOALLOC_SCRATCH_BYTES raise ValueError.  Calls whose work overlaps on one GPU race (one scratch per GPU).
    """
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    nt = n_iters // check_every if check_every > 0 else 0
    if nt > 0:
        trace = _at_least(trace, nt, torch.float32, x.device, "trace")
    _raise(lib.sk_solve_noalloc(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), _ptr(f),
                                _ptr(g), int(check_every), _ptr(trace) if nt > 0 else None, _stream(x.device)),
           "sk_solve_noalloc")
    return f, g, trace


def solve_ex(x, y, a=None, b=None, *, eps: float, variant: str = "alternating", alpha: float = 0.5,
             stop_mode: str = "fixed", stop_tol: float = 1e-6, max_iter: int = 200, check_every: int = 5,
             ws: torch.Tensor | None = None, f: torch.Tensor | None = None, g: torch.Tensor | None = None,
             check: bool = True):
    """Sinkhorn with update variant ("alternating" | "symmetric" with blend alpha) and stop rule
    ("fixed" | "marginal" | "potential"; max_iter is the iteration count or cap).

    Returns (f, g, iters_run, converged, final_viol); converged and final_viol
    are None under stop_mode="fixed" (then nothing synchronises and the
    outputs are enqueued on the current stream).
    """
    lib = load_library()
    if variant not in VARIANTS or stop_mode not in STOP_MODES:
        raise ValueError(f"variant must be one of {list(VARIANTS)}, stop_mode one of {list(STOP_MODES)}")
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    if check:
        check_inputs(x, y, a, b, ws)
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    it, conv, viol = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    _raise(lib.sk_solve_ex(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), VARIANTS[variant],
                           float(alpha), STOP_MODES[stop_mode], float(stop_tol), int(max_iter), int(check_every),
                           _ptr(f), _ptr(g), ctypes.byref(it), ctypes.byref(conv), ctypes.byref(viol), _ptr(ws),
                           ws.numel(), _stream(x.device)), "sk_solve_ex")
    if stop_mode == "fixed":
        return f, g, it.value, None, None
    return f, g, it.value, bool(conv.value), viol.value


def dual_cost(x, y, a, b, f, g, *, eps: float, ws: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """<a,f> + <b,g> - eps (sum_ij P_ij - sum(a) sum(b)) at any potentials (1-element float64 tensor)."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    f, g = _potentials(f, g, n, m, x.device)
    out = _buf(out, (1,), torch.float64, x.device, "out")
    _raise(lib.sk_dual_cost(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(f), _ptr(g), _ptr(out),
                            _ptr(ws), ws.numel(), _stream(x.device)), "sk_dual_cost")
    return out


def divergence_workspace(n: int, m: int, d: int, device) -> torch.Tensor:
    nb = int(load_library().sk_divergence_workspace_bytes(n, m, d))
    if nb == 0:
        raise ValueError(f"invalid problem size n={n} m={m} d={d}")
    ws = torch.empty(nb, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("allocator returned a workspace that is not 256-byte aligned")
    return ws


def divergence(x, y, a=None, b=None, *, eps: float, n_iters: int, variant: str = "alternating",
               alpha: float = 0.5, ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
               check: bool = True) -> torch.Tensor:
    """Debiased divergence OT(x,y) - OT(x,x)/2 - OT(y,y)/2 after n_iters iterations per term.

    Returns a 4-element float64 device tensor [S, OT(x,y), OT(x,x), OT(y,y)].
    """
    lib = load_library()
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {list(VARIANTS)}")
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    if check:
        check_inputs(x, y, a, b)
    ws = _ws(ws, x.device, lambda: divergence_workspace(n, m, d, x.device))
    out = _buf(out, (4,), torch.float64, x.device, "out")
    _raise(lib.sk_divergence(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), VARIANTS[variant],
                             float(alpha), int(n_iters), _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)),
           "sk_divergence")
    return out


def gradient_flow(x, y, a=None, b=None, *, eps: float, n_iters: int, n_steps: int, lr: float,
                  ws: torch.Tensor | None = None, f: torch.Tensor | None = None, g: torch.Tensor | None = None,
                  grad: torch.Tensor | None = None, cost_trace: torch.Tensor | None = None, check: bool = True):
    """n_steps of x <- x - lr * grad_x, each at a fresh n_iters-iteration solve; x is updated in place.

    Returns (x, f, g, grad, cost_trace): f, g, grad of the last step, cost_trace (float64, n_steps) of
    every step."""
    lib = load_library()
    x_in = x
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    if x.data_ptr() != x_in.data_ptr():
        raise ValueError("x is updated in place and must be contiguous")
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    if check:
        check_inputs(x, y, a, b, ws)
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    grad = _buf(grad, (n, d), torch.float32, x.device, "grad")
    if cost_trace is None:
        cost_trace = torch.empty(max(n_steps, 1), dtype=torch.float64, device=x.device)
    else:
        cost_trace = _at_least(cost_trace, n_steps, torch.float64, x.device, "cost_trace")
    _raise(lib.sk_gradient_flow(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(n_iters), int(n_steps),
                                float(lr), _ptr(f), _ptr(g), _ptr(grad), _ptr(cost_trace), _ptr(ws), ws.numel(),
                                _stream(x.device)), "sk_gradient_flow")
    return x, f, g, grad, cost_trace[:n_steps]


def transport_workspace(n: int, m: int, d: int, device) -> torch.Tensor:
    nb = int(load_library().sk_transport_workspace_bytes(n, m, d))
    if nb == 0:
        raise ValueError(f"invalid problem size n={n} m={m} d={d}")
    ws = torch.empty(nb, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("allocator returned a workspace that is not 256-byte aligned")
    return ws


def _potentials(f, g, n, m, device):
    return _in(f, (n,), device, "f"), _in(g, (m,), device, "g")


def transport(x, y, a, b, f, g, v, *, eps: float, transpose: bool = False, ws: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """P v (v: (m,) or (m, k)) or, with transpose, P^T v (v: (n,) or (n, k)), with
    P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps)."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    f, g = _potentials(f, g, n, m, x.device)
    rows_in, rows_out = (n, m) if transpose else (m, n)
    vec = v.dim() == 1
    v2 = v.reshape(-1, 1) if vec else v
    if v2.dim() != 2 or v2.shape[0] != rows_in:
        raise ValueError(f"v must have {rows_in} rows")
    k = v2.shape[1]
    v2 = _in(v2, (rows_in, k), x.device, "v")
    ws = _ws(ws, x.device, lambda: transport_workspace(n, m, d, x.device))
    out = _buf(out, (rows_out, k), torch.float32, x.device, "out")
    _raise(lib.sk_transport(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(f), _ptr(g),
                            1 if transpose else 0, _ptr(v2), k, _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)),
           "sk_transport")
    return out.reshape(-1) if vec else out


def hvp(x, y, a, b, f, g, v, *, eps: float, cg_iters: int = 50, ws: torch.Tensor | None = None,
        out: torch.Tensor | None = None, cg_resid: torch.Tensor | None = None):
    """Hessian-vector product of OT_eps(x, y) in x at the plan of (f, g); v and the result are (n, d).

    Returns (H v, cg_resid) with cg_resid a 1-element device tensor."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    f, g = _potentials(f, g, n, m, x.device)
    v = _in(v, (n, d), x.device, "v")
    ws = _ws(ws, x.device, lambda: transport_workspace(n, m, d, x.device))
    out = _buf(out, (n, d), torch.float32, x.device, "out")
    cg_resid = _buf(cg_resid, (1,), torch.float32, x.device, "cg_resid")
    _raise(lib.sk_hvp(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(f), _ptr(g), _ptr(v),
                      int(cg_iters), _ptr(out), _ptr(cg_resid), _ptr(ws), ws.numel(), _stream(x.device)), "sk_hvp")
    return out, cg_resid


def fs2_solve(x, y, a=None, b=None, *, eps: float, block: int = 512, tol: float = 1e-4, delta: float = 1e-6,
              coarse_iters: int = 20, max_rounds: int = 10, coarse_gain: float = 0.1, n_sample: int = 1024,
              max_iters: int = 1000, check_every: int = 10, screen_every: int = 10, ws: torch.Tensor | None = None,
              f: torch.Tensor | None = None, g: torch.Tensor | None = None, return_perm: bool = False,
              check: bool = True):
    """Two-stage block-sparse solver (d <= 8).  Returns (f, g, info); info holds rounds, fine_iters,
    kept (block pairs at the last screening), kept_fraction, converged, residual, last_check and,
    with return_perm, the Morton orders perm_x, perm_y (device int32)."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    if check:
        check_inputs(x, y, a, b)
    def make_ws():
        nb = int(lib.sk_fs2_workspace_bytes(n, m, d, int(block), int(n_sample)))
        if nb == 0:
            raise ValueError(f"invalid arguments for the block-sparse solver (n={n} m={m} d={d} block={block})")
        return torch.empty(nb, dtype=torch.uint8, device=x.device)

    ws = _ws(ws, x.device, make_ws)
    f = _buf(f, (n,), torch.float32, x.device, "f")
    g = _buf(g, (m,), torch.float32, x.device, "g")
    px = torch.empty(n, dtype=torch.int32, device=x.device) if return_perm else None
    py = torch.empty(m, dtype=torch.int32, device=x.device) if return_perm else None
    ii = (ctypes.c_int32 * 4)()
    ff = (ctypes.c_float * 2)()
    _raise(lib.sk_fs2_solve(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(block), float(tol),
                            float(delta), int(coarse_iters), int(max_rounds), float(coarse_gain), int(n_sample),
                            int(max_iters), int(check_every), int(screen_every), _ptr(f), _ptr(g), ii, ff, _ptr(px),
                            _ptr(py), _ptr(ws), ws.numel(), _stream(x.device)), "sk_fs2_solve")
    nbx, nby = (n + block - 1) // block, (m + block - 1) // block
    info = dict(rounds=ii[0], fine_iters=ii[1], kept=ii[2], kept_fraction=ii[2] / (nbx * nby), converged=bool(ii[3]),
                residual=ff[0], last_check=ff[1])
    if return_perm:
        info["perm_x"], info["perm_y"] = px, py
    return f, g, info


def cost(a, b, f, g, *, eps: float, out: torch.Tensor | None = None) -> torch.Tensor:
    """<a,f> + <b,g> - eps sum(b)(1 - sum(a)) in float64 (a 1-element device tensor)."""
    lib = load_library()
    if not isinstance(a, torch.Tensor) or a.device.type != "cuda":
        raise ValueError("a must be a float32 GPU tensor")
    n, m = a.numel(), b.numel()
    a, b = _in(a, (n,), a.device, "a"), _in(b, (m,), a.device, "b")
    f, g = _in(f, (n,), a.device, "f"), _in(g, (m,), a.device, "g")
    out = _buf(out, (1,), torch.float64, a.device, "out")
    _raise(lib.sk_cost(_ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m, float(eps), _ptr(out), _stream(a.device)),
           "sk_cost")
    return out


def marginal_residual(x, y, a, b, f, g, *, eps: float, ws: torch.Tensor | None = None) -> torch.Tensor:
    """[max|P1-a|, max|P^T1-b|, sum|P1-a|, sum|P^T1-b|] at (f, g), as a 4-element float32 tensor."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    out = torch.empty(4, dtype=torch.float32, device=x.device)
    f, g = _potentials(f, g, n, m, x.device)
    _raise(lib.sk_marginal_residual(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(f), _ptr(g),
                                    _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)), "sk_marginal_residual")
    return out


def grad_x(x, y, a, b, g, *, eps: float, ws: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """grad_i = 2 a_i (x_i - sum_j w_ij y_j), w_i. = softmax_j((g_j - C_ij)/eps + log b_j)."""
    lib = load_library()
    x, y, a, b, n, m, d = _as_problem(x, y, a, b)
    ws = _ws(ws, x.device, lambda: workspace(n, m, d, x.device))
    g = _in(g, (m,), x.device, "g")
    out = _buf(out, (n, d), torch.float32, x.device, "out")
    _raise(lib.sk_grad_x(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), _ptr(g), _ptr(out), _ptr(ws),
                         ws.numel(), _stream(x.device)), "sk_grad_x")
    return out


def timing_enable(enable: bool = True, stride: int = 1) -> None:
    """Start (reset) or stop event timing of the streamed-pass kernels; every
    stride-th pass launch is timed."""
    if stride < 1:
        raise ValueError("stride must be >= 1")
    _raise(load_library().sk_timing_enable(int(stride) if enable else 0), "sk_timing_enable")


def timing_read() -> tuple[float, int, float]:
    """(total kernel ms, launches, pairs evaluated) since timing_enable(True)."""
    ms, n, pairs = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double()
    _raise(load_library().sk_timing_read(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(pairs)), "sk_timing_read")
    return ms.value, n.value, pairs.value


__all__ = ["timing_enable", "timing_read", "solve", "solve_ex", "gradient_flow", "transport", "hvp", "fs2_solve",
           "transport_workspace", "cost", "dual_cost", "divergence",
           "divergence_workspace", "marginal_residual", "grad_x", "check_inputs", "workspace", "workspace_bytes",
           "load_library", "status_string", "SinkhornError", "LIB_PATH", "SIGNATURES", "VARIANTS", "STOP_MODES",
           "solve_noalloc", "NOALLOC_SCRATCH_BYTES", "solve_warm", "primal_cost"]
