"""Pins of the all-gather sequence-parallel share in the fp64 oracle.

* Library routine, forward: the share equals torch's fp64 attention over the
  whole sequence, restricted to the rank's query rows.
* Library routine, backward: the share's dq, dk, dv equal torch autograd of
  that attention with the upstream gradient set only on the rank's rows.
* Invariant across methods: the share equals the ring walk for the same rank.
* Planted mistakes (chunks gathered in the wrong order, local instead of
  global query positions, only the own chunk gathered, the key gradient's
  sign flipped) each fail a pin.
"""

import numpy as np
import pytest
import torch

from oracle import ring_fwd_chunked
from oracle.allgather import allgather_kv, allgather_positions, allgather_share_bwd, allgather_share_fwd

TIGHT = 1e-12
GRAD_TOL = 1e-10


def chunks(P, B, H, C, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, C, d)) for _ in range(P)]


def pin_library_fwd(fwd):
    P, B, H, Hk, C, d = 4, 1, 4, 2, 5, 8
    q, k, v = chunks(P, B, H, C, d, 11), chunks(P, B, Hk, C, d, 12), chunks(P, B, Hk, C, d, 13)
    qf = torch.from_numpy(np.concatenate(q, axis=2))
    # The library's grouped form: each key/value head repeated over its group.
    kf = torch.from_numpy(np.repeat(np.concatenate(k, axis=2), H // Hk, axis=1))
    vf = torch.from_numpy(np.repeat(np.concatenate(v, axis=2), H // Hk, axis=1))
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=causal, scale=0.3).numpy()
        for r in range(P):
            o, lse = fwd(q[r], k, v, r, causal, 0.3)
            want = ref[:, :, r * C:(r + 1) * C]
            if o.shape != want.shape or not np.allclose(o, want, atol=TIGHT, rtol=0):
                return f"fwd causal={causal} rank={r}"
            if not np.all(np.isfinite(lse)):
                return f"lse causal={causal} rank={r}"
    return None


def pin_library_bwd(bwd):
    P, B, H, Hk, C, d = 3, 1, 2, 1, 4, 6
    q, k, v = chunks(P, B, H, C, d, 21), chunks(P, B, Hk, C, d, 22), chunks(P, B, Hk, C, d, 23)
    do = chunks(P, B, H, C, d, 24)
    for causal in (False, True):
        for r in range(P):
            qf = torch.from_numpy(np.concatenate(q, axis=2)).requires_grad_(True)
            kf = torch.from_numpy(np.concatenate(k, axis=2)).requires_grad_(True)
            vf = torch.from_numpy(np.concatenate(v, axis=2)).requires_grad_(True)
            o = torch.nn.functional.scaled_dot_product_attention(
                qf, kf.repeat_interleave(H // Hk, dim=1), vf.repeat_interleave(H // Hk, dim=1),
                is_causal=causal, scale=0.35)
            g = torch.zeros_like(o)
            g[:, :, r * C:(r + 1) * C] = torch.from_numpy(do[r])
            (o * g).sum().backward()
            dq, dk, dv = bwd(q[r], k, v, do[r], r, causal, 0.35)
            checks = ((dq, qf.grad[:, :, r * C:(r + 1) * C]), (dk, kf.grad), (dv, vf.grad))
            for name, (got, want) in zip(("dq", "dk", "dv"), checks):
                want = want.numpy()
                if got.shape != want.shape or not np.allclose(got, want, atol=GRAD_TOL, rtol=0):
                    return f"{name} causal={causal} rank={r}"
    return None


def pin_ring_equivalence(fwd):
    P, B, H, C, d = 4, 2, 2, 3, 4
    q, k, v = chunks(P, B, H, C, d, 31), chunks(P, B, H, C, d, 32), chunks(P, B, H, C, d, 33)
    for causal in (False, True):
        for r in range(P):
            o, lse = fwd(q[r], k, v, r, causal, 0.5)
            ro, rl = ring_fwd_chunked(q[r], k, v, r, causal, 0.5)
            if not (np.allclose(o, ro, atol=TIGHT, rtol=0) and np.allclose(lse, rl, atol=TIGHT, rtol=0)):
                return f"ring causal={causal} rank={r}"
    return None


def test_share_equals_library_attention():
    assert pin_library_fwd(allgather_share_fwd) is None


def test_share_backward_equals_autograd():
    assert pin_library_bwd(allgather_share_bwd) is None


def test_share_equals_ring_walk():
    assert pin_ring_equivalence(allgather_share_fwd) is None


def test_gather_and_positions():
    k = chunks(3, 1, 2, 4, 5, 41)
    g = allgather_kv(k)
    assert g.shape == (1, 2, 12, 5)
    assert np.array_equal(g[:, :, 4:8], k[1])
    assert np.array_equal(allgather_positions(2, 4), np.array([8, 9, 10, 11]))


def test_future_keys_get_no_gradient():
    P, C = 3, 4
    q, k, v, do = (chunks(P, 1, 2, C, 4, s) for s in (51, 52, 53, 54))
    _, dk, dv = allgather_share_bwd(q[1], k, v, do[1], 1, True, 0.5)
    assert np.all(dk[:, :, 2 * C:] == 0) and np.all(dv[:, :, 2 * C:] == 0)
    assert np.any(dk[:, :, :2 * C] != 0)


def _mutants():
    from oracle.attention import attention_bwd, attention_fwd

    def reversed_gather_fwd(q, k, v, rank, causal, scale):
        return attention_fwd(q, allgather_kv(k[::-1]), allgather_kv(v[::-1]), scale, causal,
                             q_pos=allgather_positions(rank, q.shape[2]))

    def local_positions_fwd(q, k, v, rank, causal, scale):
        return attention_fwd(q, allgather_kv(k), allgather_kv(v), scale, causal)

    def own_chunk_fwd(q, k, v, rank, causal, scale):
        return attention_fwd(q, k[rank], v[rank], scale, causal)

    def local_positions_bwd(q, k, v, do, rank, causal, scale):
        return attention_bwd(q, allgather_kv(k), allgather_kv(v), do, scale, causal)

    def flipped_dk_bwd(q, k, v, do, rank, causal, scale):
        dq, dk, dv = allgather_share_bwd(q, k, v, do, rank, causal, scale)
        return dq, -dk, dv

    return [reversed_gather_fwd, local_positions_fwd, own_chunk_fwd], [local_positions_bwd, flipped_dk_bwd]


def _run(pin, *args):
    try:
        return pin(*args)
    except Exception as e:  # noqa: BLE001 -- any exception is a failed pin
        return f"raised {type(e).__name__}"


@pytest.mark.parametrize("i", range(3))
def test_forward_mutants_fail_a_pin(i):
    fwd = _mutants()[0][i]
    fails = [_run(pin_library_fwd, fwd), _run(pin_ring_equivalence, fwd)]
    assert any(f is not None for f in fails), f"mutant {fwd.__name__} passed every pin"


@pytest.mark.parametrize("i", range(2))
def test_backward_mutants_fail_a_pin(i):
    bwd = _mutants()[1][i]
    assert _run(pin_library_bwd, bwd) is not None, f"mutant {bwd.__name__} passed the autograd pin"
