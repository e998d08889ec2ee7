"""GPU parity at sizes the oracle finishes in seconds: several tiles, ragged
tails, both head dims, every rank, both ring modes.  HIP outputs are compared
element by element with the fp64 CPU oracle."""

import math

import numpy as np
import pytest
import torch

import long_context_exact_step_amd as ra
import oracle
from long_context_exact_step_amd import inputs
from parity import (TOL_GRAD, TOL_LSE, TOL_O, assert_close, dev, f64, gen, ring_tensors)

pytestmark = pytest.mark.gpu


def run_step(q, k, v, step, causal, scale):
    B, H, Sq, d = q.shape
    o = torch.full((B, H, Sq, d), float("nan"), device=dev())
    lse = torch.full((B, H, Sq), float("nan"), device=dev())
    ra.step_fwd(q.to(dev()), k.to(dev()), v.to(dev()), o, lse, step, causal, scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,H,Sq,Sk,d,diag", [
    (1, 1, 1, 1, 64, True),
    (1, 2, 3, 3, 128, True),
    (2, 2, 100, 100, 128, True),
    (1, 2, 129, 129, 64, True),
    (1, 3, 293, 293, 128, True),
    (1, 2, 100, 37, 128, False),
    (2, 1, 293, 517, 64, False),
    (1, 2, 1, 700, 128, False),
    (1, 1, 256, 256, 128, False),
    (1, 2, 600, 600, 128, True),
    (1, 1, 520, 1000, 64, False),
])
def test_step_fwd_matches_oracle(B, H, Sq, Sk, d, diag):
    print(f"step_fwd B={B} H={H} Sq={Sq} Sk={Sk} d={d} diag={diag}", flush=True)
    q = gen(101, inputs.Q, 0, B, H, Sq, d)
    k = gen(101, inputs.K, 0, B, H, Sk, d)
    v = gen(101, inputs.V, 0, B, H, Sk, d)
    scale = 1 / math.sqrt(d)
    o, lse = run_step(q, k, v, 0 if diag else 2, diag, scale)
    ro, rl = oracle.step_partial(f64(q), f64(k), f64(v), scale, diagonal=diag)
    assert_close(f64(o), ro, TOL_O, "o_partial")
    assert_close(f64(lse), rl, TOL_LSE, "lse_partial", rel=None)


def test_lse_merge_matches_oracle():
    print("lse_merge", flush=True)
    g = torch.Generator().manual_seed(5)
    B, H, S, d = 2, 3, 77, 128
    o = torch.randn(B, H, S, d, generator=g)
    op = torch.randn(B, H, S, d, generator=g)
    lse = torch.randn(B, H, S, generator=g) * 4
    lp = torch.randn(B, H, S, generator=g) * 4
    lse[0, 0, :5] = -math.inf
    lp[0, 0, 3:9] = -math.inf
    o[0, 0, :5] = 0
    op[0, 0, 3:9] = 0
    ro, rl = oracle.lse_merge(f64(o), f64(lse), f64(op), f64(lp))
    go, gl, gop, glp = (t.to(dev()) for t in (o, lse, op, lp))
    ra.lse_merge(go, gl, gop, glp)
    torch.cuda.synchronize()
    got_l = f64(gl)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.abs(got_l[fin] - rl[fin]).max() < 1e-5
    assert_close(f64(go), ro, 1e-5, "merged o")


def test_lse_merge_past_2_26_rows():
    """ra_lse_merge over 2^26 + 2000 rows at d = 128: the merge kernel's
    thread count, rows x 32, passes 2^31 there (the host accepts any
    B*H*S < 2^31).  Constant operands give closed forms for every row:
    o <- (e^la a + e^lb b) / (e^la + e^lb), lse <- ln(e^la + e^lb)."""
    B, H, S, d = 1, 2, (1 << 25) + 1000, 128
    print(f"lse_merge rows={B * H * S}", flush=True)
    a, b, la, lb = 1.0, 3.0, 0.5, -0.25
    o = torch.full((B, H, S, d), a, device=dev())
    op = torch.full((B, H, S, d), b, device=dev())
    lse = torch.full((B, H, S), la, device=dev())
    lp = torch.full((B, H, S), lb, device=dev())
    ra.lse_merge(o, lse, op, lp)
    torch.cuda.synchronize()
    del op, lp
    tot = math.exp(la) + math.exp(lb)
    o_ref = (math.exp(la) * a + math.exp(lb) * b) / tot
    lse_ref = math.log(tot)
    omin, omax = (x.item() for x in torch.aminmax(o))
    lmin, lmax = (x.item() for x in torch.aminmax(lse))
    del o, lse
    torch.cuda.empty_cache()
    assert abs(omin - o_ref) < 1e-5 and abs(omax - o_ref) < 1e-5, (omin, omax, o_ref)
    assert abs(lmin - lse_ref) < 1e-5 and abs(lmax - lse_ref) < 1e-5, (lmin, lmax, lse_ref)


@pytest.mark.parametrize("P,C,d,causal", [
    (1, 100, 128, True), (2, 3, 64, True), (4, 100, 128, True), (3, 129, 64, False),
    (4, 64, 128, False), (2, 200, 128, True),
])
@pytest.mark.parametrize("mode", ["resident", "double_buffer", "double_buffer_in_kernel"])
def test_ring_fwd_every_rank(P, C, d, causal, mode):
    """double_buffer_in_kernel: no copy stream given, so each step's kernel
    stages the next chunk into the idle slot itself (a wrong or late copy
    would show up in the next step's result)."""
    B, H = 1, 2
    q, k, v, _ = ring_tensors(102, B, H, P, C, d)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    copy_stream = torch.cuda.Stream() if mode == "double_buffer" else None
    ring_mode = "resident" if mode == "resident" else "double_buffer"
    for rank in range(P):
        print(f"ring_fwd P={P} C={C} d={d} causal={causal} mode={mode} rank={rank}", flush=True)
        o = torch.full((B, H, C, d), float("nan"), device=dev())
        lse = torch.full((B, H, C), float("nan"), device=dev())
        ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, causal, scale, ring_mode=ring_mode,
                    copy_stream=copy_stream)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, causal, q_pos=rank * C + np.arange(C))
        assert_close(f64(o), ro, TOL_O, f"o rank {rank}")
        assert_close(f64(lse), rl, TOL_LSE, f"lse rank {rank}", rel=None)


@pytest.mark.parametrize("P,C,d,causal,H_kv,B,H", [
    (4, 128, 128, True, None, 1, 2), (3, 192, 64, True, None, 1, 2), (3, 192, 64, False, None, 1, 2),
    (2, 256, 128, True, 1, 1, 2), (16, 64, 128, True, None, 1, 2), (3, 128, 128, True, 2, 2, 4),
])
def test_ring_fwd_fused_every_rank(P, C, d, causal, H_kv, B, H):
    """RA_RING_FUSED: the visible chunks walked by one launch.  Every rank
    against the oracle, and against the per-step resident walk (the same
    exact result, summed in another order)."""
    q, k, v, _ = ring_tensors(115, B, H, P, C, d, H_kv=H_kv)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    for rank in range(P):
        print(f"ring_fwd fused P={P} C={C} d={d} causal={causal} H_kv={H_kv} B={B} H={H} rank={rank}", flush=True)
        outs = {}
        for mode in ("fused", "resident"):
            o = torch.full((B, H, C, d), float("nan"), device=dev())
            lse = torch.full((B, H, C), float("nan"), device=dev())
            ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, causal, scale, ring_mode=mode)
            torch.cuda.synchronize()
            outs[mode] = (f64(o), f64(lse))
        ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, causal, q_pos=rank * C + np.arange(C))
        assert_close(outs["fused"][0], ro, TOL_O, f"o rank {rank}")
        assert_close(outs["fused"][1], rl, TOL_LSE, f"lse rank {rank}", rel=None)
        assert_close(outs["fused"][0], outs["resident"][0], 2e-3, "fused vs resident o", rel=None)
        assert_close(outs["fused"][1], outs["resident"][1], 1e-4, "fused vs resident lse", rel=None)


@pytest.mark.parametrize("P,C,d,H,Hk,causal,B", [(3, 8192, 64, 32, 32, True, 1), (3, 8192, 128, 32, 8, True, 1),
                                                 (2, 8212, 64, 32, 32, False, 1), (2, 8192, 64, 16, 4, True, 2)])
def test_ring_fwd_persistent_steps_match_static(P, C, d, H, Hk, causal, B):
    """The double-buffer walk's full-chunk steps, with at least four (head,
    query tile) units per compute unit, run persistent blocks that take
    units from per-XCD work queues; the resident walk runs one block per
    unit.  Each unit is computed the same way whichever block takes it, so
    the two are bit-identical: every rank, both stagings (C = 8212 has
    ragged query and key tiles; B = 2 puts the batch index in the units).
    Sampled rows against the oracle."""
    ncu, _ = ra.device_info()
    assert B * H * -(-C // 256) >= 4 * ncu, "the case needs four units per compute unit"
    q, k, v, _ = ring_tensors(117, B, H, P, C, d, H_kv=Hk)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    rows = np.array([0, 37, 255, 256, C // 2, C - 1])
    copy_stream = torch.cuda.Stream()
    for rank in range(P):
        qd = q[rank].to(dev())
        outs = {}
        for mode, cs in (("resident", None), ("double_buffer", copy_stream), ("double_buffer", None)):
            print(f"persistent steps B={B} P={P} C={C} d={d} H={H} Hk={Hk} causal={causal} rank={rank} {mode} "
                  f"copy_stream={cs is not None}", flush=True)
            o = torch.full((B, H, C, d), float("nan"), device=dev())
            lse = torch.full((B, H, C), float("nan"), device=dev())
            ra.ring_fwd(qd, kd, vd, o, lse, rank, causal, scale, ring_mode=mode, copy_stream=cs)
            torch.cuda.synchronize()
            outs[(mode, cs is not None)] = (o.cpu(), lse.cpu())
        ro, rl = outs[("resident", False)]
        for key, (o, lse) in outs.items():
            assert torch.equal(o, ro) and torch.equal(lse, rl), f"{key} differs from the resident walk"
        po, pl = oracle.attention_fwd(f64(q[rank][:, :, rows]), kf, vf, scale, causal, q_pos=rank * C + rows)
        assert_close(f64(ro[:, :, rows]), po, TOL_O, f"o rank {rank}")
        assert_close(f64(rl[:, :, rows]), pl, TOL_LSE, f"lse rank {rank}", rel=None)


@pytest.mark.parametrize("P,C", [(3, 100), (17, 64)])
def test_ring_fwd_fused_falls_back(P, C):
    """Chunk lengths that are not a multiple of 64, or more than 16 visible
    chunks, run the per-step resident walk: bit-identical to it."""
    B, H, d, rank = 1, 2, 128, P - 1
    print(f"ring_fwd fused fallback P={P} C={C}", flush=True)
    q, k, v, _ = ring_tensors(116, B, H, P, C, d, ranks=[rank])
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    outs = []
    for mode in ("fused", "resident"):
        o = torch.empty(B, H, C, d, device=dev())
        lse = torch.empty(B, H, C, device=dev())
        ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, True, ring_mode=mode)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("d", [128, 64])
def test_maximum_chunk_length(d):
    """A key chunk longer than 2^32 bytes (2^24 + 100 tokens at d = 128,
    2^25 + 100 at d = 64; the host accepts any B*H*S < 2^31).  Every key is
    zero except keys 100..127, which carry k = 2 and v = 1 against q = 1: their
    score s = 2 sqrt(d) dominates, and with 28 such keys among N
        O = 28 e^s / (28 e^s + N - 28),  lse = ln(28 e^s + N - 28).
    Those keys sit in the second 64-key tile, whose rows counted from the
    tile to the end of the chunk are just past 2^32 bytes: a tile resource
    sized by the rows left in the matrix would wrap there and read them as
    zeros (O = 0, lse = ln N)."""
    n = (1 << (32 - (d * 2).bit_length() + 1)) + 100
    print(f"maximum chunk length d={d} keys={n}", flush=True)
    assert n * d * 2 > 1 << 32
    q = torch.ones(1, 1, 256, d, dtype=torch.bfloat16, device=dev())
    k = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=dev())
    v = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=dev())
    k[:, :, 100:128] = 2
    v[:, :, 100:128] = 1
    scale = 1 / math.sqrt(d)
    o = torch.full((1, 1, 256, d), float("nan"), device=dev())
    lse = torch.full((1, 1, 256), float("nan"), device=dev())
    ra.step_fwd(q, k, v, o, lse, 1, False, scale)
    torch.cuda.synchronize()
    del k, v
    torch.cuda.empty_cache()
    s = 2 * d * scale
    big = 28 * math.exp(s)
    o_ref = big / (big + n - 28)
    lse_ref = math.log(big + n - 28)
    assert_close(f64(o), np.full((1, 1, 256, d), o_ref), TOL_O, "o")
    assert_close(f64(lse), np.full((1, 1, 256), lse_ref), TOL_LSE, "lse", rel=None)


def test_steps_plus_merge_equal_fused_ring():
    """The unfused path (ra_step_fwd per chunk + ra_lse_merge) and the fused
    ring walk agree, and merge order does not matter."""
    print("steps+merge vs fused ring", flush=True)
    B, H, P, C, d, rank = 1, 2, 4, 160, 128, 3
    q, k, v, _ = ring_tensors(103, B, H, P, C, d, ranks=[rank])
    qd = q[rank].to(dev())
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, True, ring_mode="resident")
    parts = []
    for s in range(P):
        j = (rank - s) % P
        op = torch.empty(B, H, C, d, device=dev())
        lp = torch.empty(B, H, C, device=dev())
        ra.step_fwd(qd, kd[j], vd[j], op, lp, s, True)
        parts.append((op, lp))
    results = []
    for order in ([0, 1, 2, 3], [3, 1, 0, 2], [2, 3, 1, 0]):
        mo, ml = parts[order[0]][0].clone(), parts[order[0]][1].clone()
        for n in order[1:]:
            ra.lse_merge(mo, ml, parts[n][0], parts[n][1])
        results.append((mo, ml))
    torch.cuda.synchronize()
    for mo, ml in results:
        assert_close(f64(mo), f64(o), 1e-5, "unfused vs fused o", rel=None)
        assert_close(f64(ml), f64(lse), 1e-5, "unfused vs fused lse", rel=None)


def test_future_chunks_do_not_matter():
    """Causal: contents of chunks j > rank leave the outputs bit-identical."""
    print("skip invariance", flush=True)
    B, H, P, C, d, rank = 1, 2, 4, 96, 128, 1
    q, k, v, _ = ring_tensors(104, B, H, P, C, d, ranks=[rank])
    outs = []
    for trial in range(2):
        kk = [t.clone() for t in k]
        vv = [t.clone() for t in v]
        if trial:
            for j in range(rank + 1, P):
                kk[j] = gen(999, inputs.K, j, B, H, C, d)
                vv[j] = gen(999, inputs.V, j, B, H, C, d)
        o = torch.empty(B, H, C, d, device=dev())
        lse = torch.empty(B, H, C, device=dev())
        ra.ring_fwd(q[rank].to(dev()), [t.to(dev()) for t in kk], [t.to(dev()) for t in vv], o, lse, rank, True)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def _bwd_case(P, C, d, causal, rank, B=1, H=2, wid=105):
    q, k, v, do = ring_tensors(wid, B, H, P, C, d, with_do=True, ranks=[rank])
    scale = 1 / math.sqrt(d)
    qd, dod = q[rank].to(dev()), do[rank].to(dev())
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, causal, scale, ring_mode="resident")
    dq = torch.full((B, H, C, d), float("nan"), device=dev())
    dk = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    dv = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, causal, scale)
    torch.cuda.synchronize()
    return q, k, v, do, scale, dq, dk, dv


@pytest.mark.parametrize("P,C,d,causal", [(3, 100, 128, True), (2, 129, 64, True), (3, 64, 128, False),
                                          (1, 200, 128, True),
                                          # several 256-row blocks and 64-row tiles, ragged tails
                                          (2, 600, 128, True), (2, 300, 64, True), (2, 520, 128, False),
                                          # chunks shorter than a 32-query unit or a 32-key wave: one
                                          # tile, most units and keys masked or absent
                                          (3, 1, 128, True), (3, 1, 64, False), (2, 5, 64, True),
                                          (3, 31, 128, True), (2, 33, 64, False), (4, 17, 128, True)])
def test_ring_bwd_matches_oracle(P, C, d, causal):
    for rank in range(P):
        print(f"ring_bwd P={P} C={C} d={d} causal={causal} rank={rank}", flush=True)
        q, k, v, do, scale, dq, dk, dv = _bwd_case(P, C, d, causal, rank)
        kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
        rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, causal,
                                          q_pos=rank * C + np.arange(C))
        assert_close(f64(dq), rq, TOL_GRAD, "dq")
        for j in range(P):
            sl = slice(j * C, (j + 1) * C)
            if causal and j > rank:
                assert not dk[j].any() and not dv[j].any(), "skipped chunk was touched"
                continue
            assert_close(f64(dk[j]), rk[:, :, sl], TOL_GRAD, f"dk chunk {j}")
            assert_close(f64(dv[j]), rv[:, :, sl], TOL_GRAD, f"dv chunk {j}")


@pytest.mark.parametrize("scale", [0.03, 0.5])
@pytest.mark.parametrize("d", [64, 128])
def test_ring_walk_other_scales(scale, d):
    """The softmax scale is an argument: forward and backward at scales far
    from 1/sqrt(d) (flat and peaked softmax).  At the peaked scale the
    gradients reach ~18 and P and dS are rounded to bf16 for the MFMAs, so
    the gradients' max-abs bound is 3e-2 of the largest reference gradient
    when that exceeds 1 (the relative Frobenius bound of 1e-2 applies as
    everywhere)."""
    B, H, P, C, rank = 1, 2, 3, 150, 2
    print(f"ring fwd/bwd scale={scale} d={d}", flush=True)
    q, k, v, do = ring_tensors(112, B, H, P, C, d, with_do=True, ranks=[rank])
    qd, dod = q[rank].to(dev()), do[rank].to(dev())
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, True, scale, ring_mode="resident")
    dq = torch.empty(B, H, C, d, device=dev())
    dk = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    dv = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, True, scale)
    torch.cuda.synchronize()
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    pos = rank * C + np.arange(C)
    ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, True, q_pos=pos)
    rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, True, q_pos=pos)
    assert_close(f64(o), ro, TOL_O, "o")
    assert_close(f64(lse), rl, TOL_LSE, "lse", rel=None)
    bound = lambda ref: TOL_GRAD * max(1.0, float(np.abs(ref).max()))
    assert_close(f64(dq), rq, bound(rq), "dq")
    assert_close(f64(torch.cat(dk, dim=2)), rk, bound(rk), "dk")
    assert_close(f64(torch.cat(dv, dim=2)), rv, bound(rv), "dv")


def test_ring_bwd_accumulates_over_ranks():
    """Walking every rank's share into the same dK_j/dV_j accumulators gives
    the full-sequence gradient."""
    print("ring_bwd accumulation over ranks", flush=True)
    B, H, P, C, d = 1, 2, 3, 80, 128
    q, k, v, do = ring_tensors(106, B, H, P, C, d, with_do=True)
    scale = 1 / math.sqrt(d)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    dk = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    dv = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    for rank in range(P):
        o = torch.empty(B, H, C, d, device=dev())
        lse = torch.empty(B, H, C, device=dev())
        dq = torch.empty(B, H, C, d, device=dev())
        ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, True, scale)
        ra.ring_bwd(q[rank].to(dev()), kd, vd, o, lse, do[rank].to(dev()), dq, dk, dv, rank, True, scale)
    torch.cuda.synchronize()
    qa = f64(torch.cat([q[r] for r in range(P)], dim=2))
    doa = f64(torch.cat([do[r] for r in range(P)], dim=2))
    _, rk, rv = oracle.attention_bwd(qa, f64(torch.cat(k, 2)), f64(torch.cat(v, 2)), doa, scale, True)
    assert_close(f64(torch.cat(dk, 2)), rk, TOL_GRAD, "dk accumulated")
    assert_close(f64(torch.cat(dv, 2)), rv, TOL_GRAD, "dv accumulated")


def test_repeat_runs_bit_identical():
    print("determinism", flush=True)
    outs = []
    for _ in range(2):
        q, k, v, do, scale, dq, dk, dv = _bwd_case(2, 150, 128, True, 1, wid=107)
        outs.append([t.cpu() for t in [dq, *dk, *dv]])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Scores that grow along the sequence.  The forward kernels take exponentials
# against the running maximum without first taking each tile's maximum and
# fall back to an exact pass (tile maximum, recomputed P, rescaled O) when a
# tile's row sum against that reference exceeds 2^8.  N(0,1) inputs at scale
# 1/sqrt(d) never get there past a row's first tile; these inputs do, on
# most tiles.
# ---------------------------------------------------------------------------

def _growing_scores(q, k, P, C, spike=4.0):
    """Host-side rescaling of seeded bf16 chunks (no attention arithmetic):
    Q x 3; key t of the sequence, at offset u in its chunk, x (1 + u / 64)
    (1 + t / S), so that within every chunk the keys grow by about one unit of
    scale per 64-key tile; the last 16 keys of chunk P-2 x `spike` on top.
    Scaled scores reach hundreds of nats, the running maximum rises tile
    after tile (a lazy pass against it overflows its 2^8 bound on about
    three tiles of four), and at the spike the lazy exponentials overflow
    fp32 outright."""
    S = P * C
    q = {r: (t.float() * 3).bfloat16() for r, t in q.items()}
    out = []
    for j, t in enumerate(k):
        pos = torch.arange(j * C, (j + 1) * C, dtype=torch.float32)
        ramp = (1 + (pos - j * C) / 64) * (1 + pos / S)
        if j == P - 2:
            ramp[-16:] *= spike
        out.append((t.float() * ramp[None, None, :, None]).bfloat16())
    return q, out


@pytest.mark.parametrize("P,C,d,causal", [(4, 300, 128, True), (4, 300, 128, False), (3, 200, 64, True),
                                          (2, 520, 64, False)])
def test_ring_fwd_growing_scores_every_rank(P, C, d, causal):
    B, H = 1, 2
    q, k, v, _ = ring_tensors(108, B, H, P, C, d)
    q, k = _growing_scores(q, k, P, C)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    for rank in range(P):
        print(f"ring_fwd growing scores P={P} C={C} d={d} causal={causal} rank={rank}", flush=True)
        o = torch.full((B, H, C, d), float("nan"), device=dev())
        lse = torch.full((B, H, C), float("nan"), device=dev())
        ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, causal, scale, ring_mode="resident")
        torch.cuda.synchronize()
        ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, causal, q_pos=rank * C + np.arange(C))
        if rank == P - 1:
            assert rl.max() > 100, "the inputs no longer reach large scores"
        eo = assert_close(f64(o), ro, TOL_O, f"o rank {rank}")
        el = assert_close(f64(lse), rl, TOL_LSE, f"lse rank {rank}", rel=None)
        print(f"  max-abs err o {eo:.2e} lse {el:.2e} (lse up to {rl.max():.0f})", flush=True)


@pytest.mark.parametrize("P,C,d,causal", [(3, 200, 128, True), (2, 300, 64, False)])
def test_ring_bwd_growing_scores(P, C, d, causal):
    """Backward on the same inputs.  Gradients here reach tens, and the
    step kernels round P and dS to bf16 for the MFMAs, so the max-abs bound
    is 3e-2 relative to the largest reference gradient (the relative
    Frobenius bound of 1e-2 applies as everywhere)."""
    B, H = 1, 2
    rank = P - 1
    print(f"ring_bwd growing scores P={P} C={C} d={d} causal={causal} rank={rank}", flush=True)
    q, k, v, do = ring_tensors(109, B, H, P, C, d, with_do=True, ranks=[rank])
    q, k = _growing_scores(q, k, P, C)
    scale = 1 / math.sqrt(d)
    qd, dod = q[rank].to(dev()), do[rank].to(dev())
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, causal, scale, ring_mode="resident")
    dq = torch.full((B, H, C, d), float("nan"), device=dev())
    dk = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    dv = [torch.zeros(B, H, C, d, device=dev()) for _ in range(P)]
    ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, causal, scale)
    torch.cuda.synchronize()
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, causal,
                                      q_pos=rank * C + np.arange(C))
    bound = lambda ref: TOL_GRAD * max(1.0, float(np.abs(ref).max()))
    eq = assert_close(f64(dq), rq, bound(rq), "dq")
    dkg, dvg = f64(torch.cat(dk, dim=2)), f64(torch.cat(dv, dim=2))
    ek = assert_close(dkg, rk, bound(rk), "dk")
    ev = assert_close(dvg, rv, bound(rv), "dv")
    print(f"  max-abs err dq {eq:.2e} (|dq| up to {np.abs(rq).max():.1f}), dk {ek:.2e}, dv {ev:.2e}", flush=True)


# ---------------------------------------------------------------------------
# Grouped-query attention: key/value chunks with fewer heads than the queries.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,Hk,Sq,Sk,d,diag", [
    (4, 2, 100, 100, 128, True), (6, 3, 293, 517, 64, False), (4, 1, 300, 300, 128, True),
])
def test_step_fwd_gqa_matches_oracle(H, Hk, Sq, Sk, d, diag):
    print(f"step_fwd gqa H={H} Hk={Hk} Sq={Sq} Sk={Sk} d={d} diag={diag}", flush=True)
    q = gen(108, inputs.Q, 0, 1, H, Sq, d)
    k = gen(108, inputs.K, 0, 1, Hk, Sk, d)
    v = gen(108, inputs.V, 0, 1, Hk, Sk, d)
    scale = 1 / math.sqrt(d)
    o, lse = run_step(q, k, v, 0 if diag else 2, diag, scale)
    ro, rl = oracle.step_partial(f64(q), f64(k), f64(v), scale, diagonal=diag)
    assert_close(f64(o), ro, TOL_O, "o_partial")
    assert_close(f64(lse), rl, TOL_LSE, "lse_partial", rel=None)


@pytest.mark.parametrize("mode", ["resident", "double_buffer"])
def test_ring_fwd_gqa_every_rank(mode):
    P, C, d, H, Hk = 3, 300, 128, 4, 2
    q, k, v, _ = ring_tensors(109, 1, H, P, C, d, H_kv=Hk)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    for rank in range(P):
        print(f"ring_fwd gqa mode={mode} rank={rank}", flush=True)
        o = torch.full((1, H, C, d), float("nan"), device=dev())
        lse = torch.full((1, H, C), float("nan"), device=dev())
        ra.ring_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, True, scale, ring_mode=mode)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, True, q_pos=rank * C + np.arange(C))
        assert_close(f64(o), ro, TOL_O, f"o rank {rank}")
        assert_close(f64(lse), rl, TOL_LSE, f"lse rank {rank}", rel=None)


@pytest.mark.parametrize("P,C,d,H,Hk", [(2, 300, 128, 4, 2), (3, 100, 64, 6, 3), (2, 130, 128, 4, 1),
                                        # several key blocks per head, grouped heads, d = 64
                                        (2, 600, 64, 8, 2), (2, 520, 128, 8, 2)])
def test_ring_bwd_gqa_matches_oracle(P, C, d, H, Hk):
    q, k, v, do = ring_tensors(110, 1, H, P, C, d, with_do=True, H_kv=Hk)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    for rank in range(P):
        print(f"ring_bwd gqa P={P} C={C} d={d} H={H} Hk={Hk} rank={rank}", flush=True)
        qd = q[rank].to(dev())
        o = torch.empty(1, H, C, d, device=dev())
        lse = torch.empty(1, H, C, device=dev())
        ra.ring_fwd(qd, kd, vd, o, lse, rank, True, scale, ring_mode="resident")
        dq = torch.full((1, H, C, d), float("nan"), device=dev())
        dk = [torch.zeros(1, Hk, C, d, device=dev()) for _ in range(P)]
        dv = [torch.zeros(1, Hk, C, d, device=dev()) for _ in range(P)]
        ra.ring_bwd(qd, kd, vd, o, lse, do[rank].to(dev()), dq, dk, dv, rank, True, scale)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, True,
                                          q_pos=rank * C + np.arange(C))
        assert_close(f64(dq), rq, TOL_GRAD, "dq")
        for j in range(P):
            if j > rank:
                assert not dk[j].any() and not dv[j].any(), "skipped chunk was touched"
                continue
            sl = slice(j * C, (j + 1) * C)
            assert_close(f64(dk[j]), rk[:, :, sl], TOL_GRAD, f"dk chunk {j}")
            assert_close(f64(dv[j]), rv[:, :, sl], TOL_GRAD, f"dv chunk {j}")



@pytest.mark.parametrize("P,C,d,H,Hk,causal", [(3, 130, 128, 4, 4, True), (3, 130, 128, 4, 2, True),
                                               (2, 192, 64, 4, 1, False)])
def test_ring_batch_of_two_every_rank(P, C, d, H, Hk, causal):
    """B = 2: the batch index enters every kernel's row and chunk offsets
    (queries, running output, lse, D, dq, and each key chunk of H_kv heads).
    Ragged chunks (130) and whole tiles (192, where the fused walk runs rather
    than falling back to the per-step walk).  Every forward walk (resident, double-buffered with a copy stream and with
    in-kernel staging, fused) and the backward walk, every rank, against the
    oracle."""
    B = 2
    q, k, v, do = ring_tensors(118, B, H, P, C, d, with_do=True, H_kv=Hk)
    kf, vf = f64(torch.cat(k, dim=2)), f64(torch.cat(v, dim=2))
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    copy_stream = torch.cuda.Stream()
    modes = [("resident", None), ("double_buffer", copy_stream), ("double_buffer", None), ("fused", None)]
    for rank in range(P):
        pos = rank * C + np.arange(C)
        qd, dod = q[rank].to(dev()), do[rank].to(dev())
        ro, rl = oracle.attention_fwd(f64(q[rank]), kf, vf, scale, causal, q_pos=pos)
        for mode, cs in modes:
            print(f"ring B=2 P={P} C={C} d={d} H={H} Hk={Hk} causal={causal} rank={rank} "
                  f"fwd {mode} copy_stream={cs is not None}", flush=True)
            o = torch.full((B, H, C, d), float("nan"), device=dev())
            lse = torch.full((B, H, C), float("nan"), device=dev())
            ra.ring_fwd(qd, kd, vd, o, lse, rank, causal, scale, ring_mode=mode, copy_stream=cs)
            torch.cuda.synchronize()
            assert_close(f64(o), ro, TOL_O, f"o {mode}")
            assert_close(f64(lse), rl, TOL_LSE, f"lse {mode}", rel=None)
        print(f"ring B=2 P={P} C={C} d={d} H={H} Hk={Hk} causal={causal} rank={rank} bwd", flush=True)
        dq = torch.full((B, H, C, d), float("nan"), device=dev())
        dk = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
        dv = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
        ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, causal, scale)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_bwd(f64(q[rank]), kf, vf, f64(do[rank]), scale, causal, q_pos=pos)
        assert_close(f64(dq), rq, TOL_GRAD, "dq")
        for j in range(P):
            if causal and j > rank:
                assert not dk[j].any() and not dv[j].any(), "skipped chunk was touched"
                continue
            sl = slice(j * C, (j + 1) * C)
            assert_close(f64(dk[j]), rk[:, :, sl], TOL_GRAD, f"dk chunk {j}")
            assert_close(f64(dv[j]), rv[:, :, sl], TOL_GRAD, f"dv chunk {j}")

# ---------------------------------------------------------------------------
# Head-partitioned (Ulysses) share: regroup by head, full-sequence attention.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,C,H,d,causal", [(2, 100, 4, 128, True), (4, 37, 8, 64, True),
                                            (3, 129, 3, 128, False), (2, 300, 2, 128, True)])
def test_ulysses_share_every_rank(P, C, H, d, causal):
    from oracle.ulysses import ulysses_share
    q, k, v, _ = ring_tensors(111, 1, H, P, C, d)
    qc = [q[r] for r in range(P)]
    qd, kd, vd = ([t.to(dev()) for t in x] for x in (qc, k, v))
    scale = 1 / math.sqrt(d)
    for rank in range(P):
        print(f"ulysses P={P} C={C} H={H} d={d} causal={causal} rank={rank}", flush=True)
        o = torch.full((1, H // P, P * C, d), float("nan"), device=dev())
        lse = torch.full((1, H // P, P * C), float("nan"), device=dev())
        ra.ulysses_fwd(qd, kd, vd, o, lse, rank, causal, scale)
        torch.cuda.synchronize()
        ro, rl = ulysses_share([f64(t) for t in qc], [f64(t) for t in k], [f64(t) for t in v], rank, causal, scale)
        assert_close(f64(o), ro, TOL_O, f"o rank {rank}")
        assert_close(f64(lse), rl, TOL_LSE, f"lse rank {rank}", rel=None)


@pytest.mark.parametrize("P,C,H,d,causal", [(2, 100, 4, 128, True), (4, 37, 8, 64, True), (3, 129, 3, 128, False)])
def test_ulysses_bwd_every_rank(P, C, H, d, causal):
    from oracle.ulysses import ulysses_gather
    q, k, v, do = ring_tensors(112, 1, H, P, C, d, with_do=True)
    qc, dc = [q[r] for r in range(P)], [do[r] for r in range(P)]
    qd, kd, vd, dd = ([t.to(dev()) for t in x] for x in (qc, k, v, dc))
    scale = 1 / math.sqrt(d)
    Hs, S = H // P, P * C
    for rank in range(P):
        print(f"ulysses bwd P={P} C={C} H={H} d={d} causal={causal} rank={rank}", flush=True)
        o = torch.empty(1, Hs, S, d, device=dev())
        lse = torch.empty(1, Hs, S, device=dev())
        ra.ulysses_fwd(qd, kd, vd, o, lse, rank, causal, scale)
        dq, dk, dv = (torch.full((1, Hs, S, d), float("nan"), device=dev()) for _ in range(3))
        ra.ulysses_bwd(qd, kd, vd, dd, o, lse, dq, dk, dv, rank, causal, scale)
        torch.cuda.synchronize()
        g = lambda cs: ulysses_gather([f64(t) for t in cs], rank)
        rq, rk, rv = oracle.attention_bwd(g(qc), g(k), g(v), g(dc), scale, causal)
        assert_close(f64(dq), rq, TOL_GRAD, "dq")
        assert_close(f64(dk), rk, TOL_GRAD, "dk")
        assert_close(f64(dv), rv, TOL_GRAD, "dv")


# ---------------------------------------------------------------------------
# All-gather share: gathered K/V, one pass at a causal offset.
# ---------------------------------------------------------------------------

# Ragged chunk sizes put the causal offset rank*C off the 64-token tiles;
# (2, 300) has key blocks that no query of rank 0 sees.
# The last two run two sequences (B = 2) through one gather.
AG_CASES = [(2, 100, 2, 2, 128, True, 1), (4, 37, 4, 2, 64, True, 1), (3, 129, 2, 2, 128, False, 1),
            (2, 300, 2, 1, 128, True, 1), (4, 1, 2, 2, 128, True, 1), (3, 70, 4, 4, 64, False, 1),
            (3, 90, 4, 2, 128, True, 2), (2, 65, 2, 1, 64, False, 2)]


@pytest.mark.parametrize("P,C,H,Hk,d,causal,B", AG_CASES)
def test_allgather_share_every_rank(P, C, H, Hk, d, causal, B):
    from oracle.allgather import allgather_share_fwd
    q, k, v, _ = ring_tensors(113, B, H, P, C, d, H_kv=Hk)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    for rank in range(P):
        print(f"allgather P={P} C={C} B={B} H={H} Hk={Hk} d={d} causal={causal} rank={rank}", flush=True)
        o = torch.full((B, H, C, d), float("nan"), device=dev())
        lse = torch.full((B, H, C), float("nan"), device=dev())
        ra.allgather_fwd(q[rank].to(dev()), kd, vd, o, lse, rank, causal, scale)
        torch.cuda.synchronize()
        ro, rl = allgather_share_fwd(f64(q[rank]), [f64(t) for t in k], [f64(t) for t in v], rank, causal, scale)
        assert_close(f64(o), ro, TOL_O, f"o rank {rank}")
        assert_close(f64(lse), rl, TOL_LSE, f"lse rank {rank}", rel=None)


@pytest.mark.parametrize("P,C,H,Hk,d,causal,B", AG_CASES)
def test_allgather_bwd_every_rank(P, C, H, Hk, d, causal, B):
    from oracle.allgather import allgather_share_bwd
    q, k, v, do = ring_tensors(114, B, H, P, C, d, with_do=True, H_kv=Hk)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    scale = 1 / math.sqrt(d)
    for rank in range(P):
        print(f"allgather bwd P={P} C={C} B={B} H={H} Hk={Hk} d={d} causal={causal} rank={rank}", flush=True)
        qd, dd = q[rank].to(dev()), do[rank].to(dev())
        o = torch.empty(B, H, C, d, device=dev())
        lse = torch.empty(B, H, C, device=dev())
        ra.allgather_fwd(qd, kd, vd, o, lse, rank, causal, scale)
        dq = torch.full((B, H, C, d), float("nan"), device=dev())
        dk, dv = (torch.full((B, Hk, P * C, d), float("nan"), device=dev()) for _ in range(2))
        ra.allgather_bwd(qd, kd, vd, o, lse, dd, dq, dk, dv, rank, causal, scale)
        torch.cuda.synchronize()
        rq, rk, rv = allgather_share_bwd(f64(q[rank]), [f64(t) for t in k], [f64(t) for t in v], f64(do[rank]),
                                         rank, causal, scale)
        assert_close(f64(dq), rq, TOL_GRAD, "dq")
        assert_close(f64(dk), rk, TOL_GRAD, "dk")
        assert_close(f64(dv), rv, TOL_GRAD, "dv")
        if causal:
            assert not dk[:, :, (rank + 1) * C:].any() and not dv[:, :, (rank + 1) * C:].any(), \
                "keys past the rank's chunk got a gradient"


def test_allgather_equals_ring_walk():
    """The two methods reach the same exact attention: the all-gather share
    and the ring walk of the same rank agree to rounding."""
    P, C, H, d = 4, 200, 2, 128
    q, k, v, _ = ring_tensors(115, 1, H, P, C, d)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    for rank in range(P):
        print(f"allgather vs ring rank={rank}", flush=True)
        qd = q[rank].to(dev())
        o1, o2 = (torch.empty(1, H, C, d, device=dev()) for _ in range(2))
        l1, l2 = (torch.empty(1, H, C, device=dev()) for _ in range(2))
        ra.allgather_fwd(qd, kd, vd, o1, l1, rank, True)
        ra.ring_fwd(qd, kd, vd, o2, l2, rank, True, ring_mode="resident")
        torch.cuda.synchronize()
        assert_close(f64(o1), f64(o2), 1e-2, "o all-gather vs ring")
        assert_close(f64(l1), f64(l2), 1e-3, "lse all-gather vs ring", rel=None)


def test_mfma_probe_runs_within_the_derived_peak():
    """The throughput probe: zero operands give zero sums, random ones finite
    sums, and the measured rate stays under the peak derived from the CU count
    and clock."""
    cus, clk_khz = ra.device_info()
    print(f"mfma probe: {cus} CUs, {clk_khz / 1e3:.0f} MHz", flush=True)
    assert cus > 0 and clk_khz > 0
    peak = cus * 4096 * clk_khz * 1e3
    sink = torch.full((cus * 512,), float("nan"), device=dev())
    clocks = torch.zeros(2, dtype=torch.int64, device=dev())
    ra.mfma_probe(torch.zeros(8192, dtype=torch.bfloat16, device=dev()), sink, clocks, cus, 100)
    torch.cuda.synchronize()
    assert not sink.any() and clocks[0].item() > 0 and clocks[1].item() > 0
    ops = torch.randn(8192, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(dev())
    iters = 20000
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    ra.mfma_probe(ops, sink, clocks, cus, iters)
    t1.record()
    torch.cuda.synchronize()
    rate = cus * 8 * iters * 16 * 32768 / (t0.elapsed_time(t1) * 1e-3)
    print(f"  random operands: {rate / 1e12:.0f} TFLOP/s of a derived {peak / 1e12:.0f}", flush=True)
    assert torch.isfinite(sink).all() and 0 < rate <= 1.02 * peak


def test_fwd_ladder_probe_runs_within_the_derived_peak():
    """Every level of the ladder probe runs, gives finite sums on random
    operands, records a clock, and stays under the derived peak."""
    cus, clk_khz = ra.device_info()
    peak = cus * 4096 * clk_khz * 1e3
    gen = torch.Generator().manual_seed(5)
    ops = torch.randn(10240, generator=gen).to(torch.bfloat16).to(dev())
    tiles = torch.randn(524288, generator=gen).to(torch.bfloat16).to(dev())
    sink = torch.full((cus * 512,), float("nan"), device=dev())
    clocks = torch.zeros(2, dtype=torch.int64, device=dev())
    iters = 200
    for level in range(11):
        print(f"ladder level {level}", flush=True)
        ra.fwd_ladder_probe(level, ops, tiles, sink, clocks, cus, 20, 0.1275)  # warm-up
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        ra.fwd_ladder_probe(level, ops, tiles, sink, clocks, cus, iters, 0.1275)
        t1.record()
        torch.cuda.synchronize()
        rate = cus * 8 * iters * 4194304 / (t0.elapsed_time(t1) * 1e-3)
        print(f"  {rate / 1e12:.0f} TFLOP/s of a derived {peak / 1e12:.0f}", flush=True)
        assert torch.isfinite(sink).all() and clocks[0].item() > 0 and clocks[1].item() > 0
        assert 0 < rate <= 1.02 * peak
