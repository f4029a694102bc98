"""sk_solve_noalloc (the solve in the library's static device scratch, for
callers that cannot allocate) against sk_solve with a caller-owned workspace:
the same kernels on the same inputs, so the outputs must agree bit for bit.
Two calls in a row on one GPU, the second smaller than the first, so the
second runs in a scratch that still holds the first call's contents."""
import sys

import numpy as np
import pytest
import torch

import streaming_sinkhorn_solver_amd as sk
from sk_inputs import eps32, make_inputs, random_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def _pair(x, y, a, b, eps, n_iters, check_every):
    X, Y, A, B = (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (x, y, a, b))
    n, m = x.shape[0], y.shape[0]
    nt = n_iters // check_every if check_every else 0
    f0, g0, t0 = sk.solve(X, Y, A, B, eps=eps, n_iters=n_iters, check_every=check_every)
    f1 = torch.full((n,), float("nan"), device=DEV)
    g1 = torch.full((m,), float("nan"), device=DEV)
    t1 = torch.full((max(nt, 1),), float("nan"), device=DEV)
    sk.solve_noalloc(X, Y, A, B, eps=eps, n_iters=n_iters, f=f1, g=g1, check_every=check_every, trace=t1)
    torch.cuda.synchronize()
    assert torch.equal(f0, f1) and torch.equal(g0, g1)
    if nt:
        assert torch.equal(t0[:nt], t1[:nt])
    assert torch.isfinite(f1).all() and torch.isfinite(g1).all()


@pytest.mark.parametrize("first,second", [
    (("gmm8_d3_sq", None, None, 10, 10), ("random", 1000, 777, 12, 3)),
    (("gauss_d64", 4096, 4096, 6, 0), ("random64", 300, 513, 5, 5)),
])
def test_noalloc_matches_workspace_solve_twice(first, second):
    for case in (first, second):
        name, n, m, iters, ce = case
        say("noalloc", case)
        if name.startswith("random"):
            d = 64 if name == "random64" else 3
            x, y, a, b = random_problem(n, m, d, seed=n + m)
            eps = eps32(0.1)
        else:
            x, y, a, b = make_inputs(name, n=n, m=m)
            from sk_inputs import WORKLOADS
            eps = eps32(WORKLOADS[name].eps)
        _pair(x, y, a, b, eps, iters, ce)


def test_noalloc_rejects_oversize_before_launch():
    # 2^20 x 2^20 at d = 3 needs about 100 MiB of workspace: beyond the 64 MiB scratch
    lib = sk.load_library()
    assert lib.sk_workspace_bytes(1 << 20, 1 << 20, 3) > sk.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1 << 20, 3), device=DEV)
    a = torch.full((1 << 20,), 1.0 / (1 << 20), device=DEV)
    f = torch.empty(1 << 20, device=DEV)
    with pytest.raises(ValueError, match="SK_ERR_SCRATCH"):
        sk.solve_noalloc(x, x, a, a, eps=0.1, n_iters=1, f=f, g=f.clone())
