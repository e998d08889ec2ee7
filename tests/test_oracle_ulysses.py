"""Pins of the Ulysses (head-partitioned) share in the fp64 oracle.

* Library routine: a rank's share equals torch's fp64 attention over the
  whole sequence, restricted to that rank's heads.
* Invariant across the two methods: the ranks' shares, regrouped by sequence
  (step 4), equal the ring walk's output for every query chunk.
* Planted mistakes (interleaved head assignment, queries not regrouped,
  chunks restored in the wrong order) each fail a pin.
"""


import numpy as np
import pytest
import torch

from oracle import ring_fwd_chunked
from oracle.ulysses import ulysses_gather, ulysses_heads, ulysses_scatter, ulysses_share

TIGHT = 1e-12


def chunks(P, B, H, C, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, C, d)) for _ in range(P)]


def pin_library(share):
    P, B, H, C, d = 4, 1, 8, 6, 8
    q, k, v = chunks(P, B, H, C, d, 1), chunks(P, B, H, C, d, 2), chunks(P, B, H, C, d, 3)
    full = [torch.from_numpy(np.concatenate(x, axis=2)) for x in (q, k, v)]
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(*full, is_causal=causal, scale=0.4).numpy()
        for r in range(P):
            o, _ = share(q, k, v, r, causal, 0.4)
            want = ref[:, ulysses_heads(r, P, H)]
            if o.shape != want.shape or not np.allclose(o, want, atol=TIGHT, rtol=0):
                return f"library causal={causal} rank={r}"
    return None


def pin_ring_equivalence(share, scatter):
    P, B, H, C, d = 3, 1, 6, 5, 4
    q, k, v = chunks(P, B, H, C, d, 4), chunks(P, B, H, C, d, 5), chunks(P, B, H, C, d, 6)
    for causal in (False, True):
        shares = [share(q, k, v, r, causal, 0.5)[0] for r in range(P)]
        back = scatter(shares, C)
        for j in range(P):
            ring_o, _ = ring_fwd_chunked(q[j], k, v, j, causal, 0.5)
            if back[j].shape != ring_o.shape or not np.allclose(back[j], ring_o, atol=TIGHT, rtol=0):
                return f"ring equivalence causal={causal} chunk={j}"
    return None


def test_share_equals_library_attention():
    assert pin_library(ulysses_share) is None


def test_shares_regrouped_equal_ring_walk():
    assert pin_ring_equivalence(ulysses_share, ulysses_scatter) is None


def test_gather_layout():
    P, B, H, C, d = 2, 2, 4, 3, 5
    q = chunks(P, B, H, C, d, 7)
    g = ulysses_gather(q, 1)
    assert g.shape == (B, 2, P * C, d)
    assert np.array_equal(g[:, :, C:2 * C], q[1][:, 2:4])


def test_uneven_heads_rejected():
    with pytest.raises(ValueError):
        ulysses_heads(0, 3, 8)


def _mutants():
    from oracle.attention import attention_fwd

    def interleaved_heads(q, k, v, rank, causal, scale):
        P = len(q)
        heads = np.arange(rank, q[0].shape[1], P)
        g = lambda cs: np.concatenate([c[:, heads] for c in cs], axis=2)
        return attention_fwd(g(q), g(k), g(v), scale, causal)

    def local_queries_only(q, k, v, rank, causal, scale):
        P, C = len(q), q[0].shape[2]
        heads = ulysses_heads(rank, P, q[0].shape[1])
        g = lambda cs: np.concatenate([c[:, heads] for c in cs], axis=2)
        return attention_fwd(q[rank][:, heads], g(k), g(v), scale, causal, q_pos=rank * C + np.arange(C))

    def reversed_scatter(o_shares, C):
        return ulysses_scatter(o_shares, C)[::-1]

    return [(interleaved_heads, ulysses_scatter), (local_queries_only, ulysses_scatter),
            (ulysses_share, reversed_scatter)]


def _run(pin, *args):
    try:
        return pin(*args)
    except Exception as e:  # noqa: BLE001 -- any exception is a failed pin
        return f"raised {type(e).__name__}"


def test_mutants_fail_a_pin():
    for share, scatter in _mutants():
        fails = [_run(pin_library, share), _run(pin_ring_equivalence, share, scatter)]
        assert any(f is not None for f in fails), f"mutant {share.__name__}/{scatter.__name__} passed every pin"
