"""CPU-side checks of the C ABI boundary: the library loads, exports every entry
point the header declares, sizes its workspace linearly in n + m, and rejects
bad arguments with the documented status codes before enqueuing any GPU work
(so these run without a GPU).  No compute entry point is executed here."""
import ctypes
import os
import re

import pytest
import torch

import streaming_sinkhorn_solver_amd as sk
from streaming_sinkhorn_solver_amd import build as skbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sk.h")

SK_OK, SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_UNSUPPORTED_D, SK_ERR_EPS = 0, 1, 2, 3, 4
SK_ERR_ITERS, SK_ERR_CHECK_EVERY, SK_ERR_WORKSPACE = 5, 6, 11
SK_ERR_VARIANT, SK_ERR_STOP, SK_ERR_CAPTURE = 13, 14, 15
SK_ERR_SCRATCH = 17


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sk.LIB_PATH):
        skbuild.build()
    return sk.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = header_functions()
    for must in ("sk_solve", "sk_cost", "sk_marginal_residual", "sk_grad_x", "sk_workspace_bytes",
                 "sk_check_inputs", "sk_status_string", "sk_abi_version", "sk_solve_ex", "sk_dual_cost",
                 "sk_divergence", "sk_divergence_workspace_bytes", "sk_gradient_flow", "sk_transport",
                 "sk_transport_workspace_bytes", "sk_hvp", "sk_fs2_solve", "sk_fs2_workspace_bytes"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing
    # the binding declares a signature for each of them
    assert sorted(sk.SIGNATURES) == names


def test_status_strings(lib):
    for code in range(0, 18):
        s = lib.sk_status_string(code)
        assert s and len(s) > 1 and s != b"unknown status"
    assert lib.sk_status_string(999) == b"unknown status"
    assert lib.sk_abi_version() == 2


def test_workspace_is_linear(lib):
    for d in (1, 2, 3, 8):
        w1 = lib.sk_workspace_bytes(10000, 12000, d)
        w2 = lib.sk_workspace_bytes(20000, 24000, d)
        w4 = lib.sk_workspace_bytes(40000, 48000, d)
        assert 0 < w1 < w2 < w4
        assert w4 - w2 <= 2.2 * (w2 - w1) + 65536  # grows no faster than linearly
        # far below an n x m float array
        assert w4 < 40000 * 48000 * 4 / 20
    assert lib.sk_workspace_bytes(1 << 20, 1 << 20, 3) < 200 << 20


def test_workspace_rejects_bad_sizes(lib):
    for n, m, d in [(0, 5, 2), (5, 0, 2), (5, 5, 0), (5, 5, 257), (-1, 5, 2), (1 << 31, 5, 2)]:
        assert lib.sk_workspace_bytes(n, m, d) == 0


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation returns first


def _solve(lib, *, x=FAKE, n=10, m=12, d=2, eps=0.1, iters=5, check_every=0, trace=None, ws=FAKE,
           ws_bytes=None):
    wb = lib.sk_workspace_bytes(max(n, 1), max(m, 1), max(min(d, 256), 1)) if ws_bytes is None else ws_bytes
    return lib.sk_solve(x, FAKE, FAKE, FAKE, n, m, d, eps, iters, FAKE, FAKE, check_every, trace, ws, wb, None)


def test_solve_argument_errors(lib):
    assert _solve(lib, x=None) == SK_ERR_NULL
    assert _solve(lib, n=0) == SK_ERR_SHAPE
    assert _solve(lib, m=-3) == SK_ERR_SHAPE
    assert _solve(lib, d=0) == SK_ERR_SHAPE
    assert _solve(lib, d=300) == SK_ERR_UNSUPPORTED_D
    assert _solve(lib, eps=0.0) == SK_ERR_EPS
    assert _solve(lib, eps=-1.0) == SK_ERR_EPS
    assert _solve(lib, eps=float("nan")) == SK_ERR_EPS
    assert _solve(lib, eps=float("inf")) == SK_ERR_EPS
    assert _solve(lib, eps=1e-39) == SK_ERR_EPS  # 2 log2e / eps overflows fp32
    assert _solve(lib, iters=-1) == SK_ERR_ITERS
    assert _solve(lib, check_every=-1) == SK_ERR_CHECK_EVERY
    assert _solve(lib, check_every=2, trace=None) == SK_ERR_CHECK_EVERY
    assert _solve(lib, ws=None) == SK_ERR_WORKSPACE
    assert _solve(lib, ws=ctypes.c_void_p(0x100010)) == SK_ERR_WORKSPACE  # not 256-byte aligned
    assert _solve(lib, ws_bytes=1000) == SK_ERR_WORKSPACE


def test_noalloc_argument_errors(lib):
    # the same checks as sk_solve, then the scratch limit, all before any GPU work
    def call(x=FAKE, n=10, m=12, d=2, eps=0.1, iters=5, check_every=0, trace=None):
        return lib.sk_solve_noalloc(x, FAKE, FAKE, FAKE, n, m, d, eps, iters, FAKE, FAKE, check_every, trace, None)

    assert call(x=None) == SK_ERR_NULL
    assert call(n=0) == SK_ERR_SHAPE
    assert call(d=300) == SK_ERR_UNSUPPORTED_D
    assert call(eps=0.0) == SK_ERR_EPS
    assert call(iters=-1) == SK_ERR_ITERS
    assert call(check_every=2) == SK_ERR_CHECK_EVERY
    limit = sk.NOALLOC_SCRATCH_BYTES
    assert limit == 64 << 20
    # 2^20 x 2^20 at d = 3 needs about 100 MiB; 16384^2 at d = 64 and 50,000^2 at d = 3 fit
    assert lib.sk_workspace_bytes(1 << 20, 1 << 20, 3) > limit
    assert call(n=1 << 20, m=1 << 20, d=3) == SK_ERR_SCRATCH
    assert lib.sk_workspace_bytes(16384, 16384, 64) <= limit and lib.sk_workspace_bytes(50000, 50000, 3) <= limit


def test_warm_and_primal_argument_errors(lib):
    wb = lib.sk_workspace_bytes(10, 12, 2)
    tb = lib.sk_transport_workspace_bytes(10, 12, 2)

    def warm(g_init=FAKE, n=10, iters=5, check_every=0, ws=FAKE, nbytes=wb):
        return lib.sk_solve_warm(FAKE, FAKE, FAKE, FAKE, n, 12, 2, 0.1, iters, g_init, FAKE, FAKE, check_every,
                                 None, ws, nbytes, None)

    assert warm(g_init=None) == SK_ERR_NULL
    assert warm(n=0) == SK_ERR_SHAPE
    assert warm(iters=-1) == SK_ERR_ITERS
    assert warm(check_every=1) == SK_ERR_CHECK_EVERY
    assert warm(ws=None) == SK_ERR_WORKSPACE
    assert warm(nbytes=wb - 1) == SK_ERR_WORKSPACE

    def primal(out=FAKE, eps=0.1, nbytes=tb):
        return lib.sk_primal_cost(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, eps, FAKE, FAKE, out, FAKE, nbytes, None)

    assert primal(out=None) == SK_ERR_NULL
    assert primal(eps=0.0) == SK_ERR_EPS
    assert primal(nbytes=wb) == SK_ERR_WORKSPACE  # needs the transport workspace


def test_other_entry_points_argument_errors(lib):
    wb = lib.sk_workspace_bytes(10, 12, 2)
    assert lib.sk_cost(None, FAKE, FAKE, FAKE, 10, 12, 0.1, FAKE, None) == SK_ERR_NULL
    assert lib.sk_cost(FAKE, FAKE, FAKE, FAKE, 0, 12, 0.1, FAKE, None) == SK_ERR_SHAPE
    assert lib.sk_cost(FAKE, FAKE, FAKE, FAKE, 10, 12, 0.0, FAKE, None) == SK_ERR_EPS
    assert lib.sk_marginal_residual(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, 0.1, FAKE, None, FAKE, FAKE, wb,
                                    None) == SK_ERR_NULL
    assert lib.sk_marginal_residual(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, 0.1, FAKE, FAKE, FAKE, FAKE, 10,
                                    None) == SK_ERR_WORKSPACE
    assert lib.sk_grad_x(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, float("nan"), FAKE, FAKE, FAKE, wb,
                         None) == SK_ERR_EPS
    assert lib.sk_grad_x(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, 0.1, None, FAKE, FAKE, wb, None) == SK_ERR_NULL
    assert lib.sk_check_inputs(FAKE, FAKE, None, FAKE, 10, 12, 2, FAKE, wb, None) == SK_ERR_NULL
    assert lib.sk_check_inputs(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, None, wb, None) == SK_ERR_WORKSPACE


def _solve_ex(lib, *, x=FAKE, n=10, m=12, d=2, eps=0.1, variant=0, alpha=0.5, stop=0, tol=1e-6, max_iter=20,
              check_every=5, iters=None, ws=FAKE, ws_bytes=None):
    wb = lib.sk_workspace_bytes(max(n, 1), max(m, 1), max(min(d, 256), 1)) if ws_bytes is None else ws_bytes
    it, conv, viol = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    return lib.sk_solve_ex(x, FAKE, FAKE, FAKE, n, m, d, eps, variant, alpha, stop, tol, max_iter, check_every,
                           FAKE, FAKE, ctypes.byref(it) if iters is None else iters, ctypes.byref(conv),
                           ctypes.byref(viol), ws, wb, None)


def test_solve_ex_argument_errors(lib):
    assert _solve_ex(lib, x=None) == SK_ERR_NULL
    assert _solve_ex(lib, iters=ctypes.POINTER(ctypes.c_int32)()) == SK_ERR_NULL
    assert _solve_ex(lib, n=0) == SK_ERR_SHAPE
    assert _solve_ex(lib, d=257) == SK_ERR_UNSUPPORTED_D
    assert _solve_ex(lib, eps=0.0) == SK_ERR_EPS
    assert _solve_ex(lib, variant=2) == SK_ERR_VARIANT
    assert _solve_ex(lib, variant=-1) == SK_ERR_VARIANT
    assert _solve_ex(lib, variant=1, alpha=0.0) == SK_ERR_VARIANT
    assert _solve_ex(lib, variant=1, alpha=1.5) == SK_ERR_VARIANT
    assert _solve_ex(lib, variant=1, alpha=float("nan")) == SK_ERR_VARIANT
    assert _solve_ex(lib, max_iter=-1) == SK_ERR_ITERS
    assert _solve_ex(lib, stop=3) == SK_ERR_STOP
    assert _solve_ex(lib, stop=1, tol=-1e-3) == SK_ERR_STOP
    assert _solve_ex(lib, stop=2, tol=float("nan")) == SK_ERR_STOP
    assert _solve_ex(lib, stop=1, tol=float("inf")) == SK_ERR_STOP
    assert _solve_ex(lib, stop=1, check_every=0) == SK_ERR_STOP
    assert _solve_ex(lib, ws=None) == SK_ERR_WORKSPACE
    assert _solve_ex(lib, ws_bytes=lib.sk_workspace_bytes(10, 12, 2) - 1) == SK_ERR_WORKSPACE


def test_dual_cost_and_divergence_argument_errors(lib):
    wb = lib.sk_workspace_bytes(10, 12, 2)
    assert lib.sk_dual_cost(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, 0.1, FAKE, FAKE, None, FAKE, wb, None) == SK_ERR_NULL
    assert lib.sk_dual_cost(FAKE, FAKE, FAKE, FAKE, 10, 12, 0, 0.1, FAKE, FAKE, FAKE, FAKE, wb, None) == SK_ERR_SHAPE
    assert lib.sk_dual_cost(FAKE, FAKE, FAKE, FAKE, 10, 12, 2, 0.1, FAKE, FAKE, FAKE, FAKE, 8, None) == SK_ERR_WORKSPACE
    db = lib.sk_divergence_workspace_bytes(10, 12, 2)
    # holds the largest of the three problems (x,y), (x,x), (y,y) plus a potential pair
    assert db >= max(lib.sk_workspace_bytes(10, 12, 2), lib.sk_workspace_bytes(12, 12, 2)) + 2 * 12 * 4
    assert lib.sk_divergence_workspace_bytes(0, 12, 2) == 0
    assert lib.sk_divergence_workspace_bytes(10, 12, 300) == 0
    div = lambda **k: lib.sk_divergence(k.get("x", FAKE), FAKE, FAKE, FAKE, 10, 12, 2, k.get("eps", 0.1),
                                        k.get("variant", 0), k.get("alpha", 0.5), k.get("iters", 10),
                                        k.get("out", FAKE), k.get("ws", FAKE), k.get("wb", db), None)
    assert div(x=None) == SK_ERR_NULL
    assert div(out=None) == SK_ERR_NULL
    assert div(eps=-1.0) == SK_ERR_EPS
    assert div(variant=5) == SK_ERR_VARIANT
    assert div(variant=1, alpha=2.0) == SK_ERR_VARIANT
    assert div(iters=-2) == SK_ERR_ITERS
    assert div(wb=db - 1) == SK_ERR_WORKSPACE
    assert div(ws=ctypes.c_void_p(0x100040)) == SK_ERR_WORKSPACE


def test_gradient_flow_argument_errors(lib):
    wb = lib.sk_workspace_bytes(10, 12, 2)
    flow = lambda **k: lib.sk_gradient_flow(k.get("x", FAKE), FAKE, FAKE, FAKE, 10, 12, k.get("d", 2),
                                            k.get("eps", 0.1), k.get("iters", 5), k.get("steps", 3), k.get("lr", 0.1),
                                            FAKE, FAKE, k.get("grad", FAKE), None, k.get("ws", FAKE), k.get("wb", wb),
                                            None)
    assert flow(x=None) == SK_ERR_NULL
    assert flow(grad=None) == SK_ERR_NULL
    assert flow(d=0) == SK_ERR_SHAPE
    assert flow(eps=0.0) == SK_ERR_EPS
    assert flow(iters=-1) == SK_ERR_ITERS
    assert flow(steps=-1) == SK_ERR_ITERS
    assert flow(lr=float("nan")) == 16
    assert flow(lr=float("inf")) == 16
    assert flow(wb=wb - 256) == SK_ERR_WORKSPACE


def test_transport_and_hvp_argument_errors(lib):
    tb = lib.sk_transport_workspace_bytes(10, 12, 2)
    assert tb > lib.sk_workspace_bytes(10, 12, 2)
    assert lib.sk_transport_workspace_bytes(10, 12, 64) > lib.sk_workspace_bytes(10, 12, 64)
    assert lib.sk_transport_workspace_bytes(10, 12, 257) == 0
    assert lib.sk_transport_workspace_bytes(0, 12, 2) == 0
    w1 = lib.sk_transport_workspace_bytes(10000, 12000, 3)
    w2 = lib.sk_transport_workspace_bytes(20000, 24000, 3)
    w4 = lib.sk_transport_workspace_bytes(40000, 48000, 3)
    assert w4 - w2 <= 2.2 * (w2 - w1) + 65536 and w4 < 40000 * 48000 * 4 / 20
    tr = lambda **k: lib.sk_transport(k.get("x", FAKE), FAKE, FAKE, FAKE, 10, 12, k.get("d", 2), k.get("eps", 0.1),
                                      FAKE, k.get("g", FAKE), k.get("t", 0), FAKE, k.get("k", 3), FAKE,
                                      k.get("ws", FAKE), k.get("wb", tb), None)
    assert tr(x=None) == SK_ERR_NULL
    assert tr(g=None) == SK_ERR_NULL
    assert tr(d=257) == SK_ERR_UNSUPPORTED_D
    assert tr(d=0) == SK_ERR_SHAPE
    assert tr(eps=-1.0) == SK_ERR_EPS
    assert tr(k=0) == SK_ERR_SHAPE
    assert tr(t=2) == SK_ERR_SHAPE
    assert tr(wb=tb - 1) == SK_ERR_WORKSPACE
    assert tr(ws=ctypes.c_void_p(0x100080)) == SK_ERR_WORKSPACE
    hv = lambda **k: lib.sk_hvp(k.get("x", FAKE), FAKE, FAKE, FAKE, 10, 12, k.get("d", 2), 0.1, FAKE, FAKE,
                                k.get("v", FAKE), k.get("it", 10), k.get("out", FAKE), None, FAKE, k.get("wb", tb), None)
    assert hv(v=None) == SK_ERR_NULL
    assert hv(out=None) == SK_ERR_NULL
    assert hv(d=300) == SK_ERR_UNSUPPORTED_D
    assert hv(it=-1) == SK_ERR_ITERS
    assert hv(wb=100) == SK_ERR_WORKSPACE


def test_fs2_argument_errors(lib):
    # the workspace size needs the radix sort's scratch size, queried from the device: only shape errors here
    assert lib.sk_fs2_workspace_bytes(1000, 1000, 9, 256, 64) == 0
    assert lib.sk_fs2_workspace_bytes(1000, 1000, 2, 0, 64) == 0
    assert lib.sk_fs2_workspace_bytes(1000, 1000, 2, 513, 64) == 0
    ii, ff = (ctypes.c_int32 * 4)(), (ctypes.c_float * 2)()
    fs = lambda **k: lib.sk_fs2_solve(k.get("x", FAKE), FAKE, FAKE, FAKE, k.get("n", 1000), k.get("m", 900),
                                      k.get("d", 2), k.get("eps", 0.01),
                                      k.get("B", 64), k.get("tol", 1e-5), k.get("delta", 1e-6), k.get("ci", 10),
                                      k.get("mr", 5), k.get("gain", 0.1), k.get("ns", 64), k.get("mi", 100),
                                      k.get("ce", 10), k.get("se", 10), FAKE, FAKE, ii, ff, None, None, FAKE, 1 << 30,
                                      None)
    assert fs(x=None) == SK_ERR_NULL
    assert fs(d=9) == SK_ERR_UNSUPPORTED_D
    assert fs(eps=0.0) == SK_ERR_EPS
    assert fs(B=0) == SK_ERR_SHAPE and fs(B=600) == SK_ERR_SHAPE
    assert fs(tol=-1.0) == SK_ERR_STOP and fs(delta=float("nan")) == SK_ERR_STOP and fs(gain=float("inf")) == SK_ERR_STOP
    assert fs(ci=0) == SK_ERR_ITERS and fs(mr=0) == SK_ERR_ITERS and fs(ns=0) == SK_ERR_ITERS
    assert fs(mi=-1) == SK_ERR_ITERS and fs(ce=0) == SK_ERR_ITERS and fs(se=0) == SK_ERR_ITERS
    # block-pair limits: at most 2^36 pairs scored; with delta = 0 (every pair kept) at most 2^28
    assert fs(n=(1 << 22) + 16, m=1 << 22, B=16) == SK_ERR_SHAPE  # (2^18 + 1) 2^18 pairs
    assert fs(n=(1 << 18) + 16, m=1 << 18, B=16, delta=0.0) == SK_ERR_SHAPE  # (2^14 + 1) 2^14 pairs, all kept


def test_python_contract_errors_before_gpu():
    x = torch.zeros(4, 2, dtype=torch.float64)
    y = torch.zeros(5, 2, dtype=torch.float64)
    with pytest.raises(ValueError, match="float32"):
        sk.solve(x, y, eps=0.1, n_iters=3)
    with pytest.raises(ValueError):
        sk.solve(torch.zeros(4, 2), torch.zeros(5, 3), eps=0.1, n_iters=3)
    with pytest.raises(ValueError, match="GPU"):
        sk.grad_x(torch.zeros(4, 2), torch.zeros(5, 2), None, None, torch.zeros(5), eps=0.1)
    with pytest.raises(ValueError, match="variant"):
        sk.solve_ex(torch.zeros(4, 2), torch.zeros(5, 2), eps=0.1, variant="jacobi")
    with pytest.raises(ValueError, match="stop_mode"):
        sk.solve_ex(torch.zeros(4, 2), torch.zeros(5, 2), eps=0.1, stop_mode="residual")
    with pytest.raises(ValueError, match="GPU"):
        sk.divergence(torch.zeros(4, 2), torch.zeros(5, 2), eps=0.1, n_iters=3)


def test_no_oracle_on_product_path():
    """The product package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "streaming_sinkhorn_solver_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "liboracle" not in text and "sk_oracle" not in text, fn


def test_binding_checks_caller_buffers():
    """Caller-supplied outputs, workspaces and inputs are checked for dtype, device, shape and
    layout before their pointers reach the library (a wrong one would be written or read out of
    bounds, or be a host address on the GPU)."""
    dev = torch.device("cpu")  # the checks are device-generic; "cpu" stands in for the GPU here
    assert sk._buf(None, (3, 2), torch.float32, dev, "out").shape == (3, 2)
    good = torch.empty(3, 2)
    assert sk._buf(good, (3, 2), torch.float32, dev, "out") is good
    with pytest.raises(ValueError, match="shape"):
        sk._buf(torch.empty(2, 2), (3, 2), torch.float32, dev, "out")
    with pytest.raises(ValueError, match="contiguous"):
        sk._buf(torch.empty(2, 3).t(), (3, 2), torch.float32, dev, "out")
    with pytest.raises(ValueError, match="float32"):
        sk._buf(torch.empty(3, 2, dtype=torch.float64), (3, 2), torch.float32, dev, "out")
    with pytest.raises(ValueError, match="on meta"):
        sk._buf(good, (3, 2), torch.float32, torch.device("meta"), "out")
    # inputs: float32, device, exact shape; made contiguous
    v = torch.empty(2, 3).t()
    assert sk._in(v, (3, 2), dev, "v").is_contiguous()
    with pytest.raises(ValueError, match="shape"):
        sk._in(torch.empty(4), (3,), dev, "f")
    with pytest.raises(ValueError, match="float32 tensor on meta"):
        sk._in(torch.empty(3), (3,), torch.device("meta"), "f")
    # at-least buffers (traces)
    assert sk._at_least(torch.empty(5), 4, torch.float32, dev, "trace").numel() == 5
    with pytest.raises(ValueError, match="at least 6"):
        sk._at_least(torch.empty(5), 6, torch.float32, dev, "trace")
    # workspaces: contiguous uint8 on the device (size and alignment are the library's checks)
    ws = torch.empty(64, dtype=torch.uint8)
    assert sk._ws(ws, dev, None) is ws
    with pytest.raises(ValueError, match="uint8"):
        sk._ws(torch.empty(16), dev, None)
    assert sk._ws(None, dev, lambda: ws) is ws
