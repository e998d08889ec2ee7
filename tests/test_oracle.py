"""Pins of the fp64 CPU oracle against things other than itself.

Each pin is one of: a library routine the special case reduces to (torch's
scaled_dot_product_attention and autograd, in fp64 on the CPU), brute force in
pure Python on tiny inputs, a closed form, an invariant of the method, or a
number the pages print.  ``test_mutants_fail_a_pin`` plants plausible mistakes
in copies of the oracle and checks that each one fails at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (attention_bwd, attention_bwd_key_rows, attention_fwd,
                    kv_bytes_per_step, lse_merge, ring_fwd_chunked,
                    ring_schedule, step_partial, visible_pairs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def ring_inputs(B, H, P, C, d, seed=0):
    q_all = rnd(B, H, P * C, d, seed=seed)
    k = rnd(B, H, P * C, d, seed=seed + 1)
    v = rnd(B, H, P * C, d, seed=seed + 2)
    return q_all, k, v


def torch_sdpa(q, k, v, scale, mask=None, is_causal=False):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, is_causal=is_causal, scale=scale).numpy()


# ---------------------------------------------------------------------------
# Pin checkers, written so the mutation test can run them on altered oracles.
# Each returns None on success or a string naming the failure.
# ---------------------------------------------------------------------------

def pin_sdpa(fwd):
    """P = 1 (one chunk holds the whole sequence): ordinary attention."""
    q, k, v = rnd(1, 2, 37, 16, seed=1), rnd(1, 2, 37, 16, seed=2), rnd(1, 2, 37, 16, seed=3)
    scale = 1 / math.sqrt(16)
    for causal in (False, True):
        o, _ = fwd(q, k, v, scale, causal)
        ref = torch_sdpa(q, k, v, scale, is_causal=causal)
        if not np.allclose(o, ref, atol=TIGHT, rtol=0):
            return f"sdpa causal={causal} err={np.abs(o - ref).max()}"
    # A rank's share: query rows at global positions 2C..3C-1 of a P=4 ring.
    C = 9
    qa, k, v = ring_inputs(1, 2, 4, C, 8, seed=4)
    pos = 2 * C + np.arange(C)
    q = qa[:, :, 2 * C:3 * C]
    mask = (np.arange(4 * C)[None, :] <= pos[:, None])
    o, _ = fwd(q, k, v, 0.3, True, q_pos=pos)
    ref = torch_sdpa(q, k, v, 0.3, mask=mask)
    if not np.allclose(o, ref, atol=TIGHT, rtol=0):
        return f"sdpa shifted err={np.abs(o - ref).max()}"
    return None


def pin_sdpa_gqa(fwd):
    """Grouped-query attention (fewer key/value heads than query heads): the
    library's fp64 attention with enable_gqa, which repeats each key/value
    head over a contiguous group of query heads."""
    for H, Hk in ((6, 2), (6, 3), (4, 1)):
        q, k, v = rnd(1, H, 23, 8, seed=70 + H), rnd(1, Hk, 23, 8, seed=71 + Hk), rnd(1, Hk, 23, 8, seed=72)
        for causal in (False, True):
            o, _ = fwd(q, k, v, 0.35, causal)
            tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, is_causal=causal, scale=0.35, enable_gqa=True).numpy()
            if not np.allclose(o, ref, atol=TIGHT, rtol=0):
                return f"sdpa gqa H={H} Hk={Hk} causal={causal} err={np.abs(o - ref).max()}"
    return None


def brute(q, k, v, scale, causal, q_pos):
    """Attention straight from its definition, scalar by scalar."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    o = [[[[0.0] * d for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                keys = [t for t in range(Sk) if (not causal) or t <= q_pos[i]]
                sc = {t: scale * math.fsum(float(q[b, h, i, c]) * float(k[b, h, t, c]) for c in range(d))
                      for t in keys}
                z = math.fsum(math.exp(x) for x in sc.values())
                lse[b][h][i] = math.log(z)
                for c in range(d):
                    o[b][h][i][c] = math.fsum(math.exp(sc[t]) / z * float(v[b, h, t, c]) for t in keys)
    return np.array(o), np.array(lse)


def pin_bruteforce(fwd):
    for causal in (False, True):
        q, k, v = rnd(1, 2, 4, 3, seed=5), rnd(1, 2, 9, 3, seed=6), rnd(1, 2, 9, 3, seed=7)
        pos = np.array([2, 4, 5, 8])
        o, lse = fwd(q, k, v, 0.7, causal, q_pos=pos)
        ob, lb = brute(q, k, v, 0.7, causal, pos)
        if not (np.allclose(o, ob, atol=TIGHT, rtol=0) and np.allclose(lse, lb, atol=TIGHT, rtol=0)):
            return f"brute causal={causal} errO={np.abs(o - ob).max()} errL={np.abs(lse - lb).max()}"
    return None


def pin_q_zero(fwd):
    """Q = 0: every visible score is 0, so lse_p = ln(#visible) and O_p is the
    mean of the visible values (the prefix mean under causal masking)."""
    P, C, d = 4, 6, 5
    _, k, v = ring_inputs(1, 2, P, C, d, seed=8)
    for rank in range(P):
        pos = rank * C + np.arange(C)
        q = np.zeros((1, 2, C, d))
        o, lse = fwd(q, k, v, 0.5, True, q_pos=pos)
        pref = np.cumsum(v, axis=2)[:, :, pos] / (pos + 1)[None, None, :, None]
        if not (np.allclose(lse, np.log(pos + 1.0)[None, None], atol=TIGHT, rtol=0)
                and np.allclose(o, pref, atol=TIGHT, rtol=0)):
            return f"q=0 causal rank={rank}"
        o, lse = fwd(q, k, v, 0.5, False, q_pos=pos)
        if not (np.allclose(lse, math.log(P * C), atol=TIGHT, rtol=0)
                and np.allclose(o, v.mean(axis=2, keepdims=True), atol=TIGHT, rtol=0)):
            return f"q=0 non-causal rank={rank}"
    return None


def pin_dominant_key(fwd):
    """Q = alpha * K_t with K_t much longer than other keys: softmax puts all
    mass on key t, so O -> V_t and lse -> scale * alpha * |K_t|^2."""
    d, Sk, t = 16, 20, 7
    k = rnd(1, 1, Sk, d, seed=9)
    v = rnd(1, 1, Sk, d, seed=10)
    k[0, 0, t] *= 3.0
    alpha, scale = 40.0, 0.25
    q = alpha * k[:, :, t:t + 1].copy()
    o, lse = fwd(q, k, v, scale, False)
    st = scale * alpha * float(k[0, 0, t] @ k[0, 0, t])
    if not (np.allclose(o[0, 0, 0], v[0, 0, t], atol=1e-12, rtol=0) and abs(lse[0, 0, 0] - st) < 1e-12):
        return "dominant key"
    return None


def pin_v_constant(fwd):
    q, k = rnd(1, 2, 11, 8, seed=11), rnd(1, 2, 11, 8, seed=12)
    c = rnd(8, seed=13)
    v = np.broadcast_to(c, (1, 2, 11, 8)).copy()
    for causal in (False, True):
        o, _ = fwd(q, k, v, 0.35, causal)
        if not np.allclose(o, np.broadcast_to(c, o.shape), atol=TIGHT, rtol=0):
            return f"v const causal={causal}"
    return None


def pin_chunk_merge(fwd, merge):
    """Chunked with merge equals unchunked, for arbitrary splits of the keys."""
    rng = np.random.default_rng(14)
    Sk, d = 40, 6
    q, k, v = rnd(1, 2, 10, d, seed=15), rnd(1, 2, Sk, d, seed=16), rnd(1, 2, Sk, d, seed=17)
    pos = np.arange(20, 30)
    for causal in (False, True):
        ref_o, ref_l = fwd(q, k, v, 0.4, causal, q_pos=pos)
        for P in (1, 2, 3, 4, 8):
            cuts = np.sort(rng.choice(np.arange(1, Sk), size=P - 1, replace=False))
            bounds = [0, *cuts.tolist(), Sk]
            o = lse = None
            for a, b in zip(bounds[:-1], bounds[1:]):
                op, lp = fwd(q, k[:, :, a:b], v[:, :, a:b], 0.4, causal, q_pos=pos, k_pos=np.arange(a, b))
                o, lse = (op, lp) if o is None else merge(o, lse, op, lp)
            if not (np.allclose(o, ref_o, atol=TIGHT, rtol=0) and np.allclose(lse, ref_l, atol=TIGHT, rtol=0)):
                return f"chunk merge P={P} causal={causal}"
    return None


def pin_merge_order(fwd, merge):
    """The merge is commutative and associative: any order gives the same."""
    rng = np.random.default_rng(18)
    q = rnd(1, 1, 5, 4, seed=19)
    parts = []
    for i in range(5):
        k, v = rnd(1, 1, 7, 4, seed=20 + i), rnd(1, 1, 7, 4, seed=30 + i)
        parts.append(fwd(q, 3.0 * k, v, 0.5, False))
    ref = None
    for trial in range(12):
        order = rng.permutation(len(parts)).tolist()
        items = [parts[i] for i in order]
        while len(items) > 1:  # random binary-tree order
            i = int(rng.integers(0, len(items) - 1))
            a, b = items[i], items[i + 1]
            items[i:i + 2] = [merge(a[0], a[1], b[0], b[1])]
        if ref is None:
            ref = items[0]
        elif not (np.allclose(items[0][0], ref[0], atol=TIGHT, rtol=0)
                  and np.allclose(items[0][1], ref[1], atol=TIGHT, rtol=0)):
            return "merge order"
    return None


def autograd_ref(q, k, v, do, scale, q_pos):
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    mask = torch.from_numpy(np.arange(k.shape[2])[None, :] <= q_pos[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    (o * torch.from_numpy(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_bwd_autograd(bwd):
    P, C, d = 4, 7, 8
    qa, k, v = ring_inputs(1, 2, P, C, d, seed=40)
    do = rnd(1, 2, C, d, seed=41)
    for rank in (0, 2, 3):
        pos = rank * C + np.arange(C)
        q = qa[:, :, rank * C:(rank + 1) * C]
        dq, dk, dv = bwd(q, k, v, do, 0.3, True, q_pos=pos)
        rq, rk, rv = autograd_ref(q, k, v, do, 0.3, pos)
        for a, b in ((dq, rq), (dk, rk), (dv, rv)):
            if not np.allclose(a, b, atol=1e-11, rtol=0):
                return f"autograd rank={rank} err={np.abs(a - b).max()}"
    return None


def pin_bwd_autograd_gqa(bwd):
    """Grouped-query backward: autograd through the library's fp64 attention
    with enable_gqa; a key/value head's gradient sums over its query heads."""
    P, C, d, H, Hk = 3, 6, 8, 6, 2
    qa = rnd(1, H, P * C, d, seed=80)
    k, v = rnd(1, Hk, P * C, d, seed=81), rnd(1, Hk, P * C, d, seed=82)
    do = rnd(1, H, C, d, seed=83)
    for rank in (0, 2):
        pos = rank * C + np.arange(C)
        q = qa[:, :, rank * C:(rank + 1) * C]
        dq, dk, dv = bwd(q, k, v, do, 0.3, True, q_pos=pos)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        mask = torch.from_numpy(np.arange(P * C)[None, :] <= pos[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3,
                                                             enable_gqa=True)
        (o * torch.from_numpy(do)).sum().backward()
        for a, b in ((dq, tq.grad.numpy()), (dk, tk.grad.numpy()), (dv, tv.grad.numpy())):
            if a.shape != b.shape or not np.allclose(a, b, atol=1e-11, rtol=0):
                return f"autograd gqa rank={rank}"
    return None


def pin_bwd_fd(bwd):
    """Central finite differences of L = sum(dO * O) in fp64, tiny sizes."""
    P, C, d, h = 2, 3, 4, 1e-6
    qa, k, v = ring_inputs(1, 1, P, C, d, seed=50)
    do = rnd(1, 1, C, d, seed=51)
    for causal, rank in ((True, 1), (False, 0)):
        pos = rank * C + np.arange(C)
        q = qa[:, :, rank * C:(rank + 1) * C].copy()

        def loss(qq, kk, vv):
            o, _ = attention_fwd(qq, kk, vv, 0.5, causal, q_pos=pos)
            return float((o * do).sum())

        grads = bwd(q, k, v, do, 0.5, causal, q_pos=pos)
        for which, (x, g) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            rel = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
            if rel > 1e-6:
                return f"finite differences causal={causal} arg={which} rel={rel}"
    return None


def pin_bwd_sums(bwd):
    """Summed over every key: sum_k dS_qk = 0 so sum_k dK_k = 0, and
    sum_k P_qk = 1 so sum_k dV_k = sum_q dO_q."""
    P, C, d = 3, 8, 6
    qa, k, v = ring_inputs(1, 2, P, C, d, seed=60)
    for rank in range(P):
        pos = rank * C + np.arange(C)
        q = qa[:, :, rank * C:(rank + 1) * C]
        do = rnd(1, 2, C, d, seed=61 + rank)
        _, dk, dv = bwd(q, k, v, do, 0.4, True, q_pos=pos)
        if not (np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
                and np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)):
            return f"gradient sums rank={rank}"
    return None


# ---------------------------------------------------------------------------
# The oracle as it stands, against every pin.
# ---------------------------------------------------------------------------

def test_fwd_equals_library_sdpa():
    assert pin_sdpa(attention_fwd) is None


def test_fwd_gqa_equals_library_sdpa():
    assert pin_sdpa_gqa(attention_fwd) is None


def test_bwd_gqa_equals_library_autograd():
    assert pin_bwd_autograd_gqa(attention_bwd) is None


def test_bwd_gqa_key_rows_match_full():
    H, Hk, C, d = 4, 2, 20, 8
    q, k, v = rnd(1, H, C, d, seed=90), rnd(1, Hk, C, d, seed=91), rnd(1, Hk, C, d, seed=92)
    do = rnd(1, H, C, d, seed=93)
    _, dk, dv = attention_bwd(q, k, v, do, 0.4, True)
    rows = np.array([0, 7, 19])
    dkr, dvr = attention_bwd_key_rows(q, k, v, do, 0.4, True, rows)
    assert np.allclose(dkr, dk[:, :, rows], atol=1e-12) and np.allclose(dvr, dv[:, :, rows], atol=1e-12)


def test_gqa_rejects_uneven_groups():
    with pytest.raises(ValueError):
        attention_fwd(rnd(1, 5, 4, 8), rnd(1, 2, 4, 8), rnd(1, 2, 4, 8), 0.5, False)


def test_fwd_bruteforce_tiny():
    assert pin_bruteforce(attention_fwd) is None


def test_fwd_q_zero_closed_form():
    assert pin_q_zero(attention_fwd) is None


def test_fwd_dominant_key_limit():
    assert pin_dominant_key(attention_fwd) is None


def test_fwd_v_constant():
    assert pin_v_constant(attention_fwd) is None


def test_softmax_rows_sum_to_one():
    q, k, v = rnd(1, 3, 13, 8, seed=70), rnd(1, 3, 13, 8, seed=71), rnd(1, 3, 13, 8, seed=72)
    for causal in (False, True):
        o, lse = attention_fwd(q, k, v, 0.6, causal)
        s = 0.6 * np.einsum("bhqd,bhkd->bhqk", q, k)
        if causal:
            s = np.where(np.tril(np.ones((13, 13), bool)), s, -np.inf)
        p = np.exp(s - lse[..., None])
        assert np.allclose(p.sum(-1), 1.0, atol=TIGHT)
        assert np.allclose(p @ v, o, atol=TIGHT)


def test_chunked_merge_equals_unchunked():
    assert pin_chunk_merge(attention_fwd, lse_merge) is None


def test_merge_order_independent():
    assert pin_merge_order(attention_fwd, lse_merge) is None


def test_merge_with_empty_partial():
    o = rnd(1, 1, 4, 3, seed=80)
    lse = rnd(1, 1, 4, seed=81)
    zero, ninf = np.zeros_like(o), np.full_like(lse, -np.inf)
    for a, b in (((o, lse), (zero, ninf)), ((zero, ninf), (o, lse))):
        mo, ml = lse_merge(a[0], a[1], b[0], b[1])
        assert np.array_equal(ml, lse) and np.allclose(mo, o, atol=0, rtol=0)
    mo, ml = lse_merge(zero, ninf, zero, ninf)
    assert np.all(np.isneginf(ml)) and np.all(mo == 0) and not np.isnan(mo).any()


@pytest.mark.parametrize("P,C", [(1, 5), (2, 1), (2, 6), (4, 5), (4, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_ring_walk_equals_unchunked_every_rank(P, C, causal):
    qa, k, v = ring_inputs(1, 2, P, C, 8, seed=90 + P + C)
    kc = [k[:, :, j * C:(j + 1) * C] for j in range(P)]
    vc = [v[:, :, j * C:(j + 1) * C] for j in range(P)]
    for rank in range(P):
        q = qa[:, :, rank * C:(rank + 1) * C]
        o, lse = ring_fwd_chunked(q, kc, vc, rank, causal, 0.35)
        ro, rl = attention_fwd(q, k, v, 0.35, causal, q_pos=rank * C + np.arange(C))
        assert np.allclose(o, ro, atol=TIGHT) and np.allclose(lse, rl, atol=TIGHT)


def test_step_partial_diag_is_causal_sdpa():
    q, k, v = rnd(1, 2, 12, 8, seed=100), rnd(1, 2, 12, 8, seed=101), rnd(1, 2, 12, 8, seed=102)
    o, _ = step_partial(q, k, v, 0.3, diagonal=True)
    assert np.allclose(o, torch_sdpa(q, k, v, 0.3, is_causal=True), atol=TIGHT)
    o, _ = step_partial(q, k, v, 0.3, diagonal=False)
    assert np.allclose(o, torch_sdpa(q, k, v, 0.3), atol=TIGHT)


def test_bwd_equals_library_autograd():
    assert pin_bwd_autograd(attention_bwd) is None


def test_bwd_finite_differences():
    assert pin_bwd_fd(attention_bwd) is None


def test_bwd_gradient_sums():
    assert pin_bwd_sums(attention_bwd) is None


def test_bwd_key_rows_match_full():
    P, C, d = 3, 10, 8
    qa, k, v = ring_inputs(1, 2, P, C, d, seed=110)
    q = qa[:, :, 2 * C:]
    do = rnd(1, 2, C, d, seed=111)
    pos = 2 * C + np.arange(C)
    _, dk, dv = attention_bwd(q, k, v, do, 0.4, True, q_pos=pos)
    rows = np.array([0, 3, 11, 19, 20, 29])
    dkr, dvr = attention_bwd_key_rows(q, k, v, do, 0.4, True, rows, q_pos=pos)
    assert np.allclose(dkr, dk[:, :, rows], atol=1e-12)
    assert np.allclose(dvr, dv[:, :, rows], atol=1e-12)


def test_ring_accumulation_over_ranks_equals_full_gradient():
    """dK_j, dV_j accumulated over every rank's walk equal the gradient of the
    full-sequence loss."""
    P, C, d = 3, 5, 4
    qa, k, v = ring_inputs(1, 1, P, C, d, seed=120)
    do_all = rnd(1, 1, P * C, d, seed=121)
    dk_acc, dv_acc = np.zeros_like(k), np.zeros_like(v)
    for rank in range(P):
        sl = slice(rank * C, (rank + 1) * C)
        _, dk, dv = attention_bwd(qa[:, :, sl], k, v, do_all[:, :, sl], 0.5, True,
                                  q_pos=rank * C + np.arange(C))
        dk_acc += dk
        dv_acc += dv
    _, rk, rv = autograd_ref(qa, k, v, do_all, 0.5, np.arange(P * C))
    assert np.allclose(dk_acc, rk, atol=1e-12) and np.allclose(dv_acc, rv, atol=1e-12)


# ---------------------------------------------------------------------------
# Schedule and accounting.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P", range(1, 10))
def test_schedule_visits_every_chunk_once_in_ring_order(P):
    for rank in range(P):
        sch = ring_schedule(rank, P, causal=False)
        assert [j for _, j, _ in sch] == [(rank - s) % P for s in range(P)]
        assert sorted(j for _, j, _ in sch) == list(range(P))
        assert sch[0][1] == rank
        csch = ring_schedule(rank, P, causal=True)
        assert csch[0][2] == "diag"
        vis = [j for _, j, kd in csch if kd != "skip"]
        assert vis == list(range(rank, -1, -1))
    tot_vis = sum(sum(kd != "skip" for *_, kd in ring_schedule(r, P, True)) for r in range(P))
    assert tot_vis == P * (P + 1) // 2
    assert P * P - tot_vis == P * (P - 1) // 2


def test_schedule_p8_counts():
    vis = sum(sum(kd != "skip" for *_, kd in ring_schedule(r, 8, True)) for r in range(8))
    assert (vis, 64 - vis) == (36, 28)


@pytest.mark.parametrize("C,P", [(1, 1), (3, 2), (5, 4), (7, 3)])
def test_visible_pairs_bruteforce(C, P):
    for rank in range(P):
        for causal in (False, True):
            n = 0
            for qi in range(C):
                for kk in range(P * C):
                    n += (not causal) or kk <= rank * C + qi
            assert visible_pairs(C, P, rank, causal) == n


def test_kv_bytes_match_worked_example():
    with open(os.path.join(GOLDEN, "context_parallelism_worked_example.json")) as f:
        g = json.load(f)
    C = g["S"] // g["P"]
    per_step = kv_bytes_per_step(C, g["d_k"])
    assert per_step == g["bytes_per_step_per_head"] == g["printed_MB_per_step"] * 2 ** 20
    assert per_step * g["rotations"] == g["bytes_per_layer_per_head"] == g["printed_MB_per_layer"] * 2 ** 20
    # 7B MHA: 32 layers x 32 heads x 128 x (K+V) x 2 bytes = 512 KB per token.
    per_token = 32 * kv_bytes_per_step(1, g["d_k"], H=g["heads"])
    assert per_token == g["kv_cache_per_token_bytes"]
    assert per_token * g["S"] == g["printed_kv_cache_GB_full"] * 2 ** 30
    assert per_token * C == g["printed_kv_cache_GB_per_gpu"] * 2 ** 30


# ---------------------------------------------------------------------------
# Planted mistakes: each altered oracle must fail at least one pin.
# ---------------------------------------------------------------------------

def _fwd_mutants():
    f = attention_fwd

    def no_scale(q, k, v, scale, causal, **kw):
        return f(q, k, v, 1.0, causal, **kw)

    def strict_mask(q, k, v, scale, causal, q_pos=None, **kw):
        qp = np.arange(q.shape[2]) if q_pos is None else np.asarray(q_pos)
        return f(q, k, v, scale, causal, q_pos=qp - 1, **kw)

    def lse_log2(q, k, v, scale, causal, **kw):
        o, lse = f(q, k, v, scale, causal, **kw)
        return o, lse / math.log(2.0)

    def q_k_swapped(q, k, v, scale, causal, **kw):
        if q.shape != k.shape:
            return f(q, k, v, scale, causal, **kw)
        return f(k, q, v, scale, causal, **kw)

    def v_time_reversed(q, k, v, scale, causal, **kw):
        return f(q, k, v[:, :, ::-1], scale, causal, **kw)

    def drop_last_key(q, k, v, scale, causal, **kw):
        kp = kw.pop("k_pos", None)
        if k.shape[2] < 2:
            return f(q, k, v, scale, causal, k_pos=kp, **kw)
        kp = None if kp is None else np.asarray(kp)[:-1]
        return f(q, k[:, :, :-1], v[:, :, :-1], scale, causal, k_pos=kp, **kw)

    def gqa_interleaved(q, k, v, scale, causal, **kw):
        """Query head h on key/value head h % Hk instead of h // (H / Hk)."""
        H, Hk = q.shape[1], k.shape[1]
        if Hk in (1, H):
            return f(q, k, v, scale, causal, **kw)
        idx = np.arange(H) % Hk
        return f(q, k[:, idx], v[:, idx], scale, causal, **kw)

    return [no_scale, strict_mask, lse_log2, q_k_swapped, v_time_reversed, drop_last_key, gqa_interleaved]


def _merge_mutants():
    def wrong_sign(o_a, lse_a, o_b, lse_b):
        """Wrong sign inside the weight of the second operand."""
        m = np.maximum(lse_a, lse_b)
        wa, wb = np.exp(lse_a - m), np.exp(m - lse_b)
        t = wa + wb
        return (wa / t)[..., None] * o_a + (wb / t)[..., None] * o_b, m + np.log(t)

    def unnormalised(o_a, lse_a, o_b, lse_b):
        m = np.maximum(lse_a, lse_b)
        wa, wb = np.exp(lse_a - m), np.exp(lse_b - m)
        return wa[..., None] * o_a + wb[..., None] * o_b, m + np.log(wa + wb)

    def keeps_first(o_a, lse_a, o_b, lse_b):
        return o_a, np.logaddexp(lse_a, lse_b)

    return [wrong_sign, unnormalised, keeps_first]


def _bwd_mutants():
    b = attention_bwd

    def dq_unscaled(q, k, v, do, scale, causal, **kw):
        dq, dk, dv = b(q, k, v, do, scale, causal, **kw)
        return dq / scale, dk, dv

    def no_D_term(q, k, v, do, scale, causal, q_pos=None, **kw):
        # dS = P * dP (the rowsum(dO * O) term dropped)
        qp = np.arange(q.shape[2]) if q_pos is None else np.asarray(q_pos)
        o, lse = attention_fwd(q, k, v, scale, causal, q_pos=qp)
        s = scale * np.einsum("bhqd,bhkd->bhqk", q, k)
        if causal:
            s = np.where(np.arange(k.shape[2])[None, :] <= qp[:, None], s, -np.inf)
        p = np.exp(s - lse[..., None])
        dp = np.einsum("bhqd,bhkd->bhqk", do, v)
        ds = p * dp
        return (scale * ds @ k, scale * np.swapaxes(ds, -1, -2) @ q, np.swapaxes(p, -1, -2) @ do)

    def dk_dv_swapped(q, k, v, do, scale, causal, **kw):
        dq, dk, dv = b(q, k, v, do, scale, causal, **kw)
        return dq, dv, dk

    def gqa_first_head_only(q, k, v, do, scale, causal, **kw):
        """A key/value head's gradient from the first query head of its group
        alone, not the group's sum."""
        H, Hk = q.shape[1], k.shape[1]
        if Hk == H:
            return b(q, k, v, do, scale, causal, **kw)
        grp = H // Hk
        idx = np.arange(H) // grp
        dq, dk_full, dv_full = b(q, k[:, idx], v[:, idx], do, scale, causal, **kw)
        return dq, dk_full[:, ::grp], dv_full[:, ::grp]

    return [dq_unscaled, no_D_term, dk_dv_swapped, gqa_first_head_only]


def _run_pin(pin, *args):
    """A pin's verdict on an altered oracle; a mutant that raises fails it."""
    try:
        return pin(*args)
    except Exception as e:  # noqa: BLE001 -- any exception is a failed pin
        return f"raised {type(e).__name__}"


def test_mutants_fail_a_pin():
    for m in _fwd_mutants():
        fails = [_run_pin(p, m) for p in (pin_sdpa, pin_sdpa_gqa, pin_bruteforce, pin_q_zero,
                                          pin_dominant_key, pin_v_constant)]
        fails.append(_run_pin(pin_chunk_merge, m, lse_merge))
        assert any(x is not None for x in fails), f"forward mutant {m.__name__} passed every pin"
    for m in _merge_mutants():
        fails = [_run_pin(pin_chunk_merge, attention_fwd, m), _run_pin(pin_merge_order, attention_fwd, m)]
        assert any(x is not None for x in fails), f"merge mutant {m.__name__} passed every pin"
    for m in _bwd_mutants():
        fails = [_run_pin(p, m) for p in (pin_bwd_autograd, pin_bwd_autograd_gqa, pin_bwd_sums)]
        assert any(x is not None for x in fails), f"backward mutant {m.__name__} passed every pin"


def test_gqa_mutants_fail_the_gqa_pins():
    """The grouping mistakes are caught by the GQA pins specifically."""
    fm = {m.__name__: m for m in _fwd_mutants()}
    bm = {m.__name__: m for m in _bwd_mutants()}
    assert _run_pin(pin_sdpa_gqa, fm["gqa_interleaved"]) is not None
    assert _run_pin(pin_bwd_autograd_gqa, bm["gqa_first_head_only"]) is not None


def test_oracle_header_marks_it_test_infrastructure():
    assert "TEST INFRASTRUCTURE" in oracle.__doc__
    assert "parity unpinned" in oracle.__doc__  # states that no function is unpinned
