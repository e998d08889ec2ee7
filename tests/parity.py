"""Shared helpers of the GPU parity tests: seeded inputs, the oracle on the
CPU, and the tolerance checks (max-abs 2e-2 on O, 1e-3 on lse, 3e-2 on
gradients, plus a relative Frobenius guard of 1e-2 so that a near-zero output
cannot pass on max-abs alone)."""

import os

import numpy as np
import torch

from long_context_exact_step_amd import inputs

TOL_O = 2e-2
TOL_LSE = 1e-3
TOL_GRAD = 3e-2
TOL_REL = 1e-2


def f64(t):
    """bf16/fp32 tensor -> float64 numpy (exact)."""
    return t.detach().float().cpu().double().numpy()


def gen(wid, kind, j, B, H, C, d):
    return inputs.chunk(wid, kind, j, B, H, C, d)


def ring_tensors(wid, B, H, P, C, d, with_do=False, ranks=None, H_kv=None):
    """CPU bf16 chunks: q_chunks[r], k_chunks[j], v_chunks[j] (and dO).  The
    key/value chunks carry H_kv heads (default H)."""
    ranks = range(P) if ranks is None else ranks
    Hk = H if H_kv is None else H_kv
    q = {r: gen(wid, inputs.Q, r, B, H, C, d) for r in ranks}
    k = [gen(wid, inputs.K, j, B, Hk, C, d) for j in range(P)]
    v = [gen(wid, inputs.V, j, B, Hk, C, d) for j in range(P)]
    do = {r: gen(wid, inputs.DO, r, B, H, C, d) for r in ranks} if with_do else None
    return q, k, v, do


def assert_close(got, ref, atol, name, rel=TOL_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= atol, f"{name}: max abs err {err:.3e} > {atol:.1e}"
    nr = np.linalg.norm(ref)
    if nr > 0 and rel is not None:
        r = np.linalg.norm(got - ref) / nr
        assert r <= rel, f"{name}: relative Frobenius err {r:.3e} > {rel:.1e}"
    return err


def workers():
    """CPU workers for oracle fan-out (the box gives one GPU 16 CPUs)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def dev():
    return torch.device("cuda", 0)
