"""ra_ring_bwd_noalloc on the GPU, through the C-ABI: the backward walk that
keeps its row terms in the library's static device scratch matches
ra_ring_bwd (caller workspace) on the same inputs, to the parity bar, on two
calls in a row with the second on a smaller input (the scratch keeps the
first call's contents)."""

import ctypes
import math

import numpy as np
import pytest
import torch

import long_context_exact_step_amd as ra
import oracle
from parity import TOL_GRAD, assert_close, dev, f64, ring_tensors

pytestmark = pytest.mark.gpu


def run_both(wid, B, H, Hk, P, C, d, rank):
    print(f"noalloc vs workspace backward: B={B} H={H} H_kv={Hk} P={P} C={C} d={d} rank={rank}", flush=True)
    scale = 1 / math.sqrt(d)
    q, k, v, do = ring_tensors(wid, B, H, P, C, d, with_do=True, ranks=[rank], H_kv=Hk)
    qd, dod = q[rank].to(dev()), do[rank].to(dev())
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, True, scale, ring_mode="resident")
    out = {}
    for name in ("workspace", "noalloc"):
        dq = torch.full((B, H, C, d), float("nan"), device=dev())
        dk = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
        dv = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
        if name == "workspace":
            ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, True, scale)
        else:
            ra.ring_bwd_noalloc(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, True, scale)
        torch.cuda.synchronize()
        out[name] = (dq.cpu(), [t.cpu() for t in dk], [t.cpu() for t in dv])
    # The oracle on these inputs, too, so both sit inside the parity bar.
    kf, vf = f64(torch.cat(k, 2)), f64(torch.cat(v, 2))
    rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, True,
                                      q_pos=rank * C + np.arange(C))
    return out, (rq, rk, rv)


@pytest.mark.parametrize("first,second", [
    ((700, 1, 4, 4, 4, 300, 128, 3), (701, 1, 2, 2, 4, 100, 64, 2)),
    ((702, 2, 4, 2, 3, 256, 128, 2), (703, 1, 2, 1, 3, 129, 128, 1)),
])
def test_noalloc_matches_workspace_twice(first, second):
    for wid, B, H, Hk, P, C, d, rank in (first, second):
        out, (rq, rk, rv) = run_both(wid, B, H, Hk, P, C, d, rank)
        (wq, wk, wv), (nq, nk, nv) = out["workspace"], out["noalloc"]
        # Against the existing entry point: the same kernels on the same
        # row terms, so the same values up to summation order.
        assert_close(f64(nq), f64(wq), TOL_GRAD, "dq noalloc vs workspace")
        for j in range(P):
            assert_close(f64(nk[j]), f64(wk[j]), TOL_GRAD, f"dk[{j}] noalloc vs workspace")
            assert_close(f64(nv[j]), f64(wv[j]), TOL_GRAD, f"dv[{j}] noalloc vs workspace")
        # And both against the oracle.
        assert_close(f64(nq), rq, TOL_GRAD, "dq noalloc vs oracle")
        for j in range(rank + 1):
            sl = slice(j * C, (j + 1) * C)
            assert_close(f64(nk[j]), rk[:, :, sl], TOL_GRAD, f"dk[{j}] noalloc vs oracle")
            assert_close(f64(nv[j]), rv[:, :, sl], TOL_GRAD, f"dv[{j}] noalloc vs oracle")
        print(f"  max|dq noalloc - workspace|={np.abs(f64(nq) - f64(wq)).max():.2e}", flush=True)


def test_noalloc_rejects_too_many_rows():
    B, H, P, d = 1, 32, 2, 128
    C = ra.NOALLOC_MAX_ROWS // H + 1
    t = torch.empty(1, device=dev())
    # Validation happens before any device access: shapes only, via the C-ABI.
    arr = lambda: (ctypes.c_void_p * P)(*([t.data_ptr()] * P))
    L = ra.lib()
    p = ctypes.c_void_p(t.data_ptr())
    st = L.ra_ring_bwd_noalloc(p, arr(), arr(), P, p, p, p, p, arr(), arr(), 1, 1, 0.1, B, H, H, C, d, None)
    assert st == 6  # RA_ERR_WORKSPACE
