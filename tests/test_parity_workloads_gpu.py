"""GPU parity on the five ring-attention workloads at their full sizes, in the
launch configuration bench.py times (double-buffered ring walk with a copy
stream).

* Tiny ring (S=512, P=4, d=64, non-causal) and the full ring (S=32K, P=8,
  every rank): every row of O and lse against the fp64 oracle.
* 128K/CP=4 and 1M/CP=8 local shares: 256 seeded query rows per head against
  the oracle, plus closed forms checked on every row: Q = 0 makes every
  visible score 0, so lse_p = ln(p + 1) and O_p is the mean of V over the
  visible prefix; V = 1 makes O = 1.
* Training share (C=16K, P=4, rank 3): O/lse and dQ on 256 sampled query
  rows per head, dK/dV on 256 sampled key rows per (head, chunk) for every
  head, and on every key the sums that hold exactly: sum_k dK_k = 0 and
  sum_k dV_k = sum_q dO_q.
* Head-partitioned (Ulysses) share of the 128K/CP=4 sequence: ranks 0 and 3,
  H/4 = 8 heads over all 131072 tokens, 256 sampled rows per head; its
  backward: dQ on 256 sampled rows per head and the gradient sums on every
  key.
* Grouped-query attention (key/value chunks of H/4 heads): the 128K/CP=4
  share on sampled rows, and the training share's dQ on sampled rows, dK/dV
  (summed over each group's query heads) on sampled key rows of every
  key/value head, and the gradient sums on every key.
* All-gather share: the 128K/CP=4 forward on sampled rows (MHA and grouped
  heads); the training share's forward and dQ on sampled rows, dK/dV on
  sampled key rows of every head over the gathered sequence, and the
  gradient sums.
* Head size 64: the 128K/CP=4 share and the training share again at H = 64,
  d = 64 (the same flops and bytes), with the same checks.

The oracle runs on the host, fanned out over heads with one BLAS thread per
task.
"""

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import long_context_exact_step_amd as ra
import oracle
from long_context_exact_step_amd import inputs
from long_context_exact_step_amd.workloads import WORKLOADS
from parity import TOL_GRAD, TOL_LSE, TOL_O, TOL_REL, assert_close, dev, f64, workers

pytestmark = pytest.mark.gpu

# The full-size shares checked below, by key: the workloads themselves and
# their head-size-64 variants (H = 64, d = 64).
SHARES = {
    2: WORKLOADS[2],
    4: WORKLOADS[4],
    "2_d64": dataclasses.replace(WORKLOADS[2], H=64, d=64,
                                 name="128K/CP=4 local share, rank 3, H=64, d=64, causal fwd"),
}
TRAINS = {
    5: WORKLOADS[5],
    "5_d64": dataclasses.replace(WORKLOADS[5], H=64, d=64,
                                 name="training share C=16K, P=4, rank 3, H=64, d=64, causal fwd+bwd"),
}


def say(msg):
    print(msg, flush=True)


def gen_workload(w, ranks=None, with_do=False, H_kv=None):
    ranks = w.ranks if ranks is None else ranks
    Hk = w.H if H_kv is None else H_kv
    q = {r: inputs.chunk(w.id, inputs.Q, r, w.B, w.H, w.C, w.d) for r in ranks}
    k = [inputs.chunk(w.id, inputs.K, j, w.B, Hk, w.C, w.d) for j in range(w.P)]
    v = [inputs.chunk(w.id, inputs.V, j, w.B, Hk, w.C, w.d) for j in range(w.P)]
    do = {r: inputs.chunk(w.id, inputs.DO, r, w.B, w.H, w.C, w.d) for r in ranks} if with_do else None
    return q, k, v, do


def gpu_ring_fwd(w, rank, q, kd, vd, mode="double_buffer"):
    o = torch.full((w.B, w.H, w.C, w.d), float("nan"), device=dev())
    lse = torch.full((w.B, w.H, w.C), float("nan"), device=dev())
    # "double_buffer_in_kernel": no copy stream, each step kernel stages the next chunk.
    cs = torch.cuda.Stream(dev()) if mode == "double_buffer" else None
    ring_mode = "double_buffer" if mode == "double_buffer_in_kernel" else mode
    ra.ring_fwd(q.to(dev()), kd, vd, o, lse, rank, w.causal, w.scale, ring_mode=ring_mode, copy_stream=cs)
    torch.cuda.synchronize()
    return o, lse


def head_full(chunks, h):
    """fp64 [1, 1, P*C, d] of one head over the unchunked sequence."""
    return np.concatenate([f64(c[:, h:h + 1]) for c in chunks], axis=2)


def fan_out(fn, items):
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, items))


def check_rows(w, rank, q, k, v, o, lse, rows_of_head, label, grp=1, more=()):
    """Oracle on rows_of_head(h) of every head vs the GPU (o, lse), and vs each
    further (o, lse, label) in `more` (one oracle evaluation for all).  grp > 1:
    grouped-query key/value chunks, query head h reads key/value head h // grp."""
    outs = [(o.cpu(), lse.cpu(), label)] + [(a.cpu(), b.cpu(), n) for a, b, n in more]

    def one(h):
        rows = rows_of_head(h)
        kh, vh = head_full(k, h // grp), head_full(v, h // grp)
        qh = f64(q[:, h:h + 1, rows])
        ro, rl = oracle.attention_fwd(qh, kh, vh, w.scale, w.causal, q_pos=rank * w.C + rows)
        res = []
        for o_c, l_c, _ in outs:
            go, gl = f64(o_c[:, h:h + 1, rows]), f64(l_c[:, h:h + 1, rows])
            res.append((np.abs(go - ro).max(), np.abs(gl - rl).max(),
                        np.linalg.norm(go - ro) ** 2, np.linalg.norm(ro) ** 2, np.isfinite(go).all()))
        return res

    per_head = fan_out(one, range(w.H))
    for n, (_, _, name) in enumerate(outs):
        res = [r[n] for r in per_head]
        err_o = max(r[0] for r in res)
        err_l = max(r[1] for r in res)
        rel = math.sqrt(sum(r[2] for r in res) / sum(r[3] for r in res))
        say(f"{name}: max|dO|={err_o:.2e} max|dlse|={err_l:.2e} rel={rel:.2e}")
        assert all(r[4] for r in res), f"{name}: non-finite output"
        assert err_o <= TOL_O, f"{name}: O max abs err {err_o}"
        assert err_l <= TOL_LSE, f"{name}: lse max abs err {err_l}"
        assert rel <= TOL_REL, f"{name}: O relative err {rel}"


# ---------------------------------------------------------------------------
# Tiny ring, every rank, every row, both ring modes.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["double_buffer", "resident"])
def test_tiny_ring_all_rows(mode):
    w = WORKLOADS[1]
    q, k, v, _ = gen_workload(w)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    for r in w.ranks:
        say(f"tiny ring rank {r} mode {mode}")
        o, lse = gpu_ring_fwd(w, r, q[r], kd, vd, mode)
        check_rows(w, r, q[r], k, v, o, lse, lambda h: np.arange(w.C), f"tiny rank {r}")


# ---------------------------------------------------------------------------
# Full ring S=32K, P=8: every rank, every row.
# ---------------------------------------------------------------------------

@pytest.mark.timeout(600)
def test_full_ring_all_rows():
    w = WORKLOADS[3]
    q, k, v, _ = gen_workload(w)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    for r in w.ranks:
        say(f"full ring rank {r}: GPU walk (double buffer with a copy stream, with in-kernel staging, "
            f"resident, and fused), then oracle on all {w.C} rows x {w.H} heads")
        o, lse = gpu_ring_fwd(w, r, q[r], kd, vd)
        io, il = gpu_ring_fwd(w, r, q[r], kd, vd, "double_buffer_in_kernel")
        ro, rl = gpu_ring_fwd(w, r, q[r], kd, vd, "resident")
        fo, fl = gpu_ring_fwd(w, r, q[r], kd, vd, "fused")
        check_rows(w, r, q[r], k, v, o, lse, lambda h: np.arange(w.C), f"full ring rank {r}",
                   more=[(io, il, f"full ring rank {r} in-kernel staging"), (ro, rl, f"full ring rank {r} resident"),
                         (fo, fl, f"full ring rank {r} fused")])


@pytest.mark.timeout(600)
def test_full_ring_ranks_concurrent_bit_identical():
    """Every rank of the 32K full ring walked at once, each on a stream and
    with staging slots of its own (in-kernel staging, as the ranks of a real
    ring run): bit-identical to the same walks run one after another."""
    w = WORKLOADS[3]
    q, _, _, _ = gen_workload(w)
    k = [inputs.chunk(w.id, inputs.K, j, w.B, w.H, w.C, w.d).to(dev()) for j in range(w.P)]
    v = [inputs.chunk(w.id, inputs.V, j, w.B, w.H, w.C, w.d).to(dev()) for j in range(w.P)]
    qd = {r: q[r].to(dev()) for r in w.ranks}
    seq = {r: gpu_ring_fwd(w, r, qd[r], k, v, "double_buffer_in_kernel") for r in w.ranks}
    need = ra.workspace_bytes(w.P, w.B, w.H, w.C, w.d, "double_buffer")
    wss = {r: torch.empty(need, dtype=torch.uint8, device=dev()) for r in w.ranks}
    streams = {r: torch.cuda.Stream(dev()) for r in w.ranks}
    out = {r: (torch.full((w.B, w.H, w.C, w.d), float("nan"), device=dev()),
               torch.full((w.B, w.H, w.C), float("nan"), device=dev())) for r in w.ranks}
    torch.cuda.synchronize()
    say(f"full ring: {len(w.ranks)} ranks walked concurrently")
    for r in w.ranks:
        ra.ring_fwd(qd[r], k, v, out[r][0], out[r][1], r, w.causal, w.scale, ring_mode="double_buffer",
                    workspace=wss[r], stream=streams[r], copy_stream=None)
    torch.cuda.synchronize()
    for r in w.ranks:
        assert torch.equal(out[r][0], seq[r][0]) and torch.equal(out[r][1], seq[r][1]), f"rank {r}"


# ---------------------------------------------------------------------------
# 128K/CP=4 and 1M/CP=8 local shares.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def share_inputs():
    cache = {}

    def get(wid):
        if wid not in cache:
            cache.clear()
            w = SHARES[wid]
            say(f"generating inputs of {w.name}")
            q, k, v, _ = gen_workload(w)
            cache[wid] = (q, k, v, [t.to(dev()) for t in k], [t.to(dev()) for t in v])
        return cache[wid]

    yield get
    cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 4, "2_d64"])
def test_local_share_sampled_rows(wid, share_inputs):
    w = SHARES[wid]
    r = w.ranks[0]
    q, k, v, kd, vd = share_inputs(wid)
    say(f"{w.name}: GPU walk (copy stream, and in-kernel staging)")
    o, lse = gpu_ring_fwd(w, r, q[r], kd, vd)
    io, il = gpu_ring_fwd(w, r, q[r], kd, vd, "double_buffer_in_kernel")
    check_rows(w, r, q[r], k, v, o, lse, lambda h: inputs.query_row_sample(w.id, h, w.C),
               f"{w.name} sampled rows", more=[(io, il, f"{w.name} in-kernel staging sampled rows")])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 4, "2_d64"])
def test_local_share_closed_forms_every_row(wid, share_inputs):
    w = SHARES[wid]
    r = w.ranks[0]
    q, k, v, kd, vd = share_inputs(wid)
    pos = r * w.C + np.arange(w.C)

    say(f"{w.name}: Q = 0 (lse = ln(p+1), O = prefix mean of V)")
    o, lse = gpu_ring_fwd(w, r, torch.zeros_like(q[r]), kd, vd)
    o_c, l_c = o.cpu(), lse.cpu()
    want_l = np.log(pos + 1.0)

    def one(h):
        vh = head_full(v, h)[0, 0]
        pref = (np.cumsum(vh, axis=0)[pos] / (pos + 1)[:, None])
        return (np.abs(f64(o_c[0, h]) - pref).max(), np.abs(f64(l_c[0, h]) - want_l).max())

    res = fan_out(one, range(w.H))
    err_o, err_l = max(x[0] for x in res), max(x[1] for x in res)
    say(f"  max|O - prefix mean|={err_o:.2e} max|lse - ln(p+1)|={err_l:.2e}")
    assert err_o <= TOL_O and err_l <= TOL_LSE

    say(f"{w.name}: V = 1 (O = 1)")
    ones = [torch.ones_like(t) for t in vd]
    o, lse = gpu_ring_fwd(w, r, q[r], kd, ones)
    err = (o - 1).abs().max().item()
    say(f"  max|O - 1|={err:.2e}")
    assert err <= TOL_O
    assert torch.isfinite(lse).all()


@pytest.mark.timeout(600)
def test_local_share_walk_bit_repeatable(share_inputs):
    """The 128K/CP=4 walk at full size, run twice in each staging mode: the
    copy stream's event-ordered copies and the in-kernel staging must give
    bit-identical O and lse from run to run (the kernels are deterministic,
    and every staged chunk is complete before a step reads it), and the two
    stagings must agree with each other bit for bit."""
    w = WORKLOADS[2]
    r = w.ranks[0]
    q, k, v, kd, vd = share_inputs(2)
    runs = {}
    for mode in ("double_buffer", "double_buffer_in_kernel"):
        for rep in range(2):
            say(f"{w.name}: {mode} run {rep}")
            runs[(mode, rep)] = tuple(t.cpu() for t in gpu_ring_fwd(w, r, q[r], kd, vd, mode))
    ref = runs[("double_buffer", 0)]
    for key, (o, lse) in runs.items():
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"{key} differs from the first run"


# ---------------------------------------------------------------------------
# Training share: forward + backward.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module", params=list(TRAINS))
def train_run(request):
    w = TRAINS[request.param]
    r = w.ranks[0]
    say(f"{w.name}: inputs")
    q, k, v, do = gen_workload(w, with_do=True)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o, lse = gpu_ring_fwd(w, r, q[r], kd, vd)
    dq = torch.full_like(o, float("nan"))
    dk = [torch.zeros(w.B, w.H, w.C, w.d, device=dev()) for _ in range(w.P)]
    dv = [torch.zeros(w.B, w.H, w.C, w.d, device=dev()) for _ in range(w.P)]
    say(f"{w.name}: GPU backward walk")
    ra.ring_bwd(q[r].to(dev()), kd, vd, o, lse, do[r].to(dev()), dq, dk, dv, r, w.causal, w.scale)
    torch.cuda.synchronize()
    out = dict(w=w, r=r, q=q[r], k=k, v=v, do=do[r], o=o.cpu(), lse=lse.cpu(), dq=dq.cpu(),
               dk=[t.cpu() for t in dk], dv=[t.cpu() for t in dv])
    del kd, vd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(600)
def test_train_forward_and_dq_sampled_rows(train_run):
    t = train_run
    w, r = t["w"], t["r"]

    def one(h):
        rows = inputs.query_row_sample(w.id, h, w.C)
        kh, vh = head_full(t["k"], h), head_full(t["v"], h)
        qh, doh = f64(t["q"][:, h:h + 1, rows]), f64(t["do"][:, h:h + 1, rows])
        pos = r * w.C + rows
        ro, rl = oracle.attention_fwd(qh, kh, vh, w.scale, True, q_pos=pos)
        rq, _, _ = oracle.attention_bwd(qh, kh, vh, doh, w.scale, True, q_pos=pos)
        go, gl, gq = (f64(t[n][:, h:h + 1, rows]) for n in ("o", "lse", "dq"))
        return (np.abs(go - ro).max(), np.abs(gl - rl).max(), np.abs(gq - rq).max(),
                np.linalg.norm(gq - rq) ** 2, np.linalg.norm(rq) ** 2)

    say(f"{w.name}: oracle forward + dQ on 256 rows x {w.H} heads")
    res = fan_out(one, range(w.H))
    e_o, e_l, e_q = (max(x[i] for x in res) for i in range(3))
    rel_q = math.sqrt(sum(x[3] for x in res) / sum(x[4] for x in res))
    say(f"  max|dO|={e_o:.2e} max|dlse|={e_l:.2e} max|ddQ|={e_q:.2e} rel dQ={rel_q:.2e}")
    assert e_o <= TOL_O and e_l <= TOL_LSE and e_q <= TOL_GRAD and rel_q <= TOL_REL


@pytest.mark.timeout(900)
def test_train_dk_dv_sampled_key_rows(train_run):
    t = train_run
    w, r = t["w"], t["r"]
    heads = range(w.H)
    pos = r * w.C + np.arange(w.C)

    def one(h):
        kh, vh = head_full(t["k"], h), head_full(t["v"], h)
        qh, doh = f64(t["q"][:, h:h + 1]), f64(t["do"][:, h:h + 1])
        per_chunk = [inputs.key_row_sample(w.id, h, j, w.C) for j in range(w.P)]
        all_rows = np.concatenate([j * w.C + rows for j, rows in enumerate(per_chunk)])
        rk, rv = oracle.attention_bwd_key_rows(qh, kh, vh, doh, w.scale, True, all_rows, q_pos=pos)
        errs = []
        n0 = 0
        for j, rows in enumerate(per_chunk):
            sl = slice(n0, n0 + len(rows))
            n0 += len(rows)
            gk, gv = f64(t["dk"][j][:, h:h + 1, rows]), f64(t["dv"][j][:, h:h + 1, rows])
            errs.append((np.abs(gk - rk[:, :, sl]).max(), np.abs(gv - rv[:, :, sl]).max(),
                         np.linalg.norm(gk - rk[:, :, sl]) ** 2 + np.linalg.norm(gv - rv[:, :, sl]) ** 2,
                         np.linalg.norm(rk[:, :, sl]) ** 2 + np.linalg.norm(rv[:, :, sl]) ** 2))
        return errs

    say(f"{w.name}: oracle dK/dV on 256 key rows x {w.P} chunks x all {w.H} heads")
    res = [e for per_head in fan_out(one, heads) for e in per_head]
    e_k, e_v = max(x[0] for x in res), max(x[1] for x in res)
    rel = math.sqrt(sum(x[2] for x in res) / sum(x[3] for x in res))
    say(f"  max|ddK|={e_k:.2e} max|ddV|={e_v:.2e} rel={rel:.2e}")
    assert e_k <= TOL_GRAD and e_v <= TOL_GRAD and rel <= TOL_REL


@pytest.mark.timeout(600)
def test_train_backward_bit_repeatable(train_run):
    """The training share's backward walk at full size, run again on the
    same forward output: dQ, dK and dV are bit-identical (no atomics)."""
    t = train_run
    w, r = t["w"], t["r"]
    kd = [x.to(dev()) for x in t["k"]]
    vd = [x.to(dev()) for x in t["v"]]
    o, lse = t["o"].to(dev()), t["lse"].to(dev())
    dq = torch.full_like(o, float("nan"))
    dk = [torch.zeros(w.B, w.H, w.C, w.d, device=dev()) for _ in range(w.P)]
    dv = [torch.zeros(w.B, w.H, w.C, w.d, device=dev()) for _ in range(w.P)]
    say(f"{w.name}: second backward walk")
    ra.ring_bwd(t["q"].to(dev()), kd, vd, o, lse, t["do"].to(dev()), dq, dk, dv, r, w.causal, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(dq.cpu(), t["dq"])
    for j in range(w.P):
        assert torch.equal(dk[j].cpu(), t["dk"][j]) and torch.equal(dv[j].cpu(), t["dv"][j]), f"chunk {j}"
    del kd, vd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_train_gradient_sums_every_key(train_run):
    t = train_run
    w = t["w"]
    dk = torch.cat(t["dk"], dim=2).double()
    dv = torch.cat(t["dv"], dim=2).double()
    sum_dk = dk.sum(dim=2)
    scale_k = dk.abs().sum(dim=2)
    sum_dv = dv.sum(dim=2)
    sum_do = t["do"].double().sum(dim=2)
    r_k = (sum_dk.abs() / scale_k.clamp_min(1e-30)).max().item()
    r_v = ((sum_dv - sum_do).abs().max() / sum_do.abs().max()).item()
    say(f"{w.name}: max|sum dK|/sum|dK|={r_k:.2e}  max|sum dV - sum dO|/max|sum dO|={r_v:.2e}")
    assert r_k <= 1e-3 and r_v <= 1e-3


# ---------------------------------------------------------------------------
# Grouped-query attention at full size: the 128K/CP=4 share and the training
# share with key/value chunks of H/4 = 8 heads (the bench's gqa runs).
# ---------------------------------------------------------------------------

GQA_GROUP = 4


@pytest.mark.timeout(600)
def test_gqa_local_share_sampled_rows():
    w = WORKLOADS[2]
    r = w.ranks[0]
    Hk = w.H // GQA_GROUP
    say(f"{w.name}, H_kv={Hk}: inputs and GPU walk")
    q, k, v, _ = gen_workload(w, H_kv=Hk)
    kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
    o, lse = gpu_ring_fwd(w, r, q[r], kd, vd)
    del kd, vd
    check_rows(w, r, q[r], k, v, o, lse, lambda h: inputs.query_row_sample(w.id, h, w.C),
               f"{w.name} H_kv={Hk} sampled rows", grp=GQA_GROUP)


@pytest.fixture(scope="module")
def train_run_gqa():
    w = WORKLOADS[5]
    r = w.ranks[0]
    Hk = w.H // GQA_GROUP
    say(f"{w.name}, H_kv={Hk}: inputs")
    q, k, v, do = gen_workload(w, with_do=True, H_kv=Hk)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o, lse = gpu_ring_fwd(w, r, q[r], kd, vd)
    dq = torch.full_like(o, float("nan"))
    dk = [torch.zeros(w.B, Hk, w.C, w.d, device=dev()) for _ in range(w.P)]
    dv = [torch.zeros(w.B, Hk, w.C, w.d, device=dev()) for _ in range(w.P)]
    say(f"{w.name}, H_kv={Hk}: GPU backward walk")
    ra.ring_bwd(q[r].to(dev()), kd, vd, o, lse, do[r].to(dev()), dq, dk, dv, r, w.causal, w.scale)
    torch.cuda.synchronize()
    out = dict(w=w, r=r, Hk=Hk, q=q[r], k=k, v=v, do=do[r], o=o.cpu(), lse=lse.cpu(), dq=dq.cpu(),
               dk=[t.cpu() for t in dk], dv=[t.cpu() for t in dv])
    del kd, vd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(600)
def test_gqa_train_dq_sampled_rows(train_run_gqa):
    t = train_run_gqa
    w, r = t["w"], t["r"]

    def one(h):
        rows = inputs.query_row_sample(w.id, h, w.C)
        kh, vh = head_full(t["k"], h // GQA_GROUP), head_full(t["v"], h // GQA_GROUP)
        qh, doh = f64(t["q"][:, h:h + 1, rows]), f64(t["do"][:, h:h + 1, rows])
        pos = r * w.C + rows
        rq, _, _ = oracle.attention_bwd(qh, kh, vh, doh, w.scale, True, q_pos=pos)
        gq = f64(t["dq"][:, h:h + 1, rows])
        return np.abs(gq - rq).max(), np.linalg.norm(gq - rq) ** 2, np.linalg.norm(rq) ** 2

    say(f"{w.name}, H_kv={t['Hk']}: oracle dQ on 256 rows x {w.H} heads")
    res = fan_out(one, range(w.H))
    e_q = max(x[0] for x in res)
    rel = math.sqrt(sum(x[1] for x in res) / sum(x[2] for x in res))
    say(f"  max|ddQ|={e_q:.2e} rel={rel:.2e}")
    assert e_q <= TOL_GRAD and rel <= TOL_REL


@pytest.mark.timeout(900)
def test_gqa_train_dk_dv_sampled_key_rows(train_run_gqa):
    """dK/dV of every key/value head, which sum over the 4 query heads of its
    group: the oracle runs once per query head (its contribution to its
    key/value head at that head's sampled key rows) and the contributions of
    a group are added."""
    t = train_run_gqa
    w, r = t["w"], t["r"]
    Hk = t["Hk"]
    pos = r * w.C + np.arange(w.C)
    key_rows = {hk: [inputs.key_row_sample(w.id, hk, j, w.C) for j in range(w.P)] for hk in range(Hk)}

    def one(h):
        hk = h // GQA_GROUP
        kh, vh = head_full(t["k"], hk), head_full(t["v"], hk)
        qh, doh = f64(t["q"][:, h:h + 1]), f64(t["do"][:, h:h + 1])
        all_rows = np.concatenate([j * w.C + rows for j, rows in enumerate(key_rows[hk])])
        return oracle.attention_bwd_key_rows(qh, kh, vh, doh, w.scale, True, all_rows, q_pos=pos)

    say(f"{w.name}, H_kv={Hk}: oracle dK/dV on 256 key rows x {w.P} chunks x all {Hk} key/value heads "
        f"({w.H} query heads)")
    per_q = fan_out(one, range(w.H))
    res = []
    for hk in range(Hk):
        rk = sum(per_q[h][0] for h in range(hk * GQA_GROUP, (hk + 1) * GQA_GROUP))
        rv = sum(per_q[h][1] for h in range(hk * GQA_GROUP, (hk + 1) * GQA_GROUP))
        n0 = 0
        for j, rows in enumerate(key_rows[hk]):
            sl = slice(n0, n0 + len(rows))
            n0 += len(rows)
            gk, gv = f64(t["dk"][j][:, hk:hk + 1, rows]), f64(t["dv"][j][:, hk:hk + 1, rows])
            res.append((np.abs(gk - rk[:, :, sl]).max(), np.abs(gv - rv[:, :, sl]).max(),
                        np.linalg.norm(gk - rk[:, :, sl]) ** 2 + np.linalg.norm(gv - rv[:, :, sl]) ** 2,
                        np.linalg.norm(rk[:, :, sl]) ** 2 + np.linalg.norm(rv[:, :, sl]) ** 2))
    e_k, e_v = max(x[0] for x in res), max(x[1] for x in res)
    rel = math.sqrt(sum(x[2] for x in res) / sum(x[3] for x in res))
    say(f"  max|ddK|={e_k:.2e} max|ddV|={e_v:.2e} rel={rel:.2e}")
    assert e_k <= TOL_GRAD and e_v <= TOL_GRAD and rel <= TOL_REL


def test_gqa_train_gradient_sums_every_key(train_run_gqa):
    """Per key/value head: sum_k dK_k = 0, and sum_k dV_k = the sum of dO over
    the query rows of every query head in its group."""
    t = train_run_gqa
    w = t["w"]
    dk = torch.cat(t["dk"], dim=2).double()
    dv = torch.cat(t["dv"], dim=2).double()
    sum_dk = dk.sum(dim=2)
    scale_k = dk.abs().sum(dim=2)
    do = t["do"].double()
    sum_do = do.reshape(w.B, t["Hk"], GQA_GROUP, w.C, w.d).sum(dim=(2, 3))
    r_k = (sum_dk.abs() / scale_k.clamp_min(1e-30)).max().item()
    r_v = ((dv.sum(dim=2) - sum_do).abs().max() / sum_do.abs().max()).item()
    say(f"{w.name}, H_kv={t['Hk']}: max|sum dK|/sum|dK|={r_k:.2e}  max|sum dV - sum dO|/max|sum dO|={r_v:.2e}")
    assert r_k <= 1e-3 and r_v <= 1e-3


# ---------------------------------------------------------------------------
# Head-partitioned (Ulysses) share of the 128K/CP=4 sequence.
# ---------------------------------------------------------------------------

@pytest.mark.timeout(600)
def test_ulysses_share_128k_sampled_rows():
    w = WORKLOADS[2]
    P, C = w.P, w.C
    S = P * C
    Hs = w.H // P
    say(f"{w.name}: Ulysses inputs (every chunk)")
    q, k, v, _ = gen_workload(w, ranks=range(P))
    qc = [q[r] for r in range(P)]
    qd, kd, vd = ([t.to(dev()) for t in x] for x in (qc, k, v))
    for rank in (0, P - 1):
        say(f"{w.name}: Ulysses share of rank {rank} ({Hs} heads x {S} tokens)")
        o = torch.full((w.B, Hs, S, w.d), float("nan"), device=dev())
        lse = torch.full((w.B, Hs, S), float("nan"), device=dev())
        ra.ulysses_fwd(qd, kd, vd, o, lse, rank, w.causal, w.scale)
        torch.cuda.synchronize()
        o_c, l_c = o.cpu(), lse.cpu()

        def one(i):
            h = rank * Hs + i  # global head
            rows = inputs.query_row_sample(w.id, h, S)
            kh, vh = head_full(k, h), head_full(v, h)
            qh = np.concatenate([f64(c[:, h:h + 1]) for c in qc], axis=2)[:, :, rows]
            ro, rl = oracle.attention_fwd(qh, kh, vh, w.scale, w.causal, q_pos=rows)
            go, gl = f64(o_c[:, i:i + 1, rows]), f64(l_c[:, i:i + 1, rows])
            return np.abs(go - ro).max(), np.abs(gl - rl).max(), np.isfinite(go).all()

        res = fan_out(one, range(Hs))
        e_o, e_l = max(r_[0] for r_ in res), max(r_[1] for r_ in res)
        say(f"  max|dO|={e_o:.2e} max|dlse|={e_l:.2e}")
        assert all(r_[2] for r_ in res) and e_o <= TOL_O and e_l <= TOL_LSE
        del o, lse
    del qd, kd, vd
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_ulysses_bwd_128k_sampled_rows_and_sums():
    from oracle.ulysses import ulysses_gather
    w = WORKLOADS[2]
    P, C = w.P, w.C
    S, Hs, rank = P * C, w.H // P, 1
    say(f"{w.name}: Ulysses backward inputs (every chunk)")
    q, k, v, do = gen_workload(w, ranks=range(P), with_do=True)
    qc, dc = [q[r] for r in range(P)], [do[r] for r in range(P)]
    qd, kd, vd, dd = ([t.to(dev()) for t in x] for x in (qc, k, v, dc))
    o = torch.empty(w.B, Hs, S, w.d, device=dev())
    lse = torch.empty(w.B, Hs, S, device=dev())
    ra.ulysses_fwd(qd, kd, vd, o, lse, rank, w.causal, w.scale)
    dq, dk, dv = (torch.full((w.B, Hs, S, w.d), float("nan"), device=dev()) for _ in range(3))
    say(f"{w.name}: Ulysses backward of rank {rank} ({Hs} heads x {S} tokens)")
    ra.ulysses_bwd(qd, kd, vd, dd, o, lse, dq, dk, dv, rank, w.causal, w.scale)
    torch.cuda.synchronize()
    dq_c, dk_c, dv_c = dq.cpu(), dk.double().cpu(), dv.double().cpu()
    del qd, kd, vd, dd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    gq, gk, gv, gd = (ulysses_gather([f64(t) for t in cs], rank) for cs in (qc, k, v, dc))

    def one(i):
        rows = inputs.query_row_sample(w.id, rank * Hs + i, S)
        rq, _, _ = oracle.attention_bwd(gq[:, i:i + 1, rows], gk[:, i:i + 1], gv[:, i:i + 1], gd[:, i:i + 1, rows],
                                        w.scale, w.causal, q_pos=rows)
        got = f64(dq_c[:, i:i + 1, rows])
        return np.abs(got - rq).max(), np.linalg.norm(got - rq) ** 2, np.linalg.norm(rq) ** 2

    res = fan_out(one, range(Hs))
    e_q = max(x[0] for x in res)
    rel = math.sqrt(sum(x[1] for x in res) / sum(x[2] for x in res))
    r_k = (dk_c.sum(dim=2).abs() / dk_c.abs().sum(dim=2).clamp_min(1e-30)).max().item()
    sum_do = torch.from_numpy(gd).sum(dim=2)
    r_v = ((dv_c.sum(dim=2) - sum_do).abs().max() / sum_do.abs().max()).item()
    say(f"  max|ddQ|={e_q:.2e} rel={rel:.2e}  max|sum dK|/sum|dK|={r_k:.2e}  sum dV vs sum dO={r_v:.2e}")
    assert e_q <= TOL_GRAD and rel <= TOL_REL and r_k <= 1e-3 and r_v <= 1e-3


# ---------------------------------------------------------------------------
# All-gather share: the rank's queries over the gathered sequence in one pass.
# ---------------------------------------------------------------------------

@pytest.mark.timeout(600)
def test_allgather_share_128k_sampled_rows():
    """Rank 3's share of the 128K/CP=4 sequence (MHA, then key/value chunks
    of H/4 heads) against the oracle on 256 sampled rows per head."""
    w = WORKLOADS[2]
    r = w.ranks[0]
    for Hk in (w.H, w.H // GQA_GROUP):
        say(f"{w.name}, H_kv={Hk}: all-gather inputs")
        q, k, v, _ = gen_workload(w, H_kv=Hk)
        kd, vd = [t.to(dev()) for t in k], [t.to(dev()) for t in v]
        o = torch.full((w.B, w.H, w.C, w.d), float("nan"), device=dev())
        lse = torch.full((w.B, w.H, w.C), float("nan"), device=dev())
        say(f"{w.name}, H_kv={Hk}: all-gather share of rank {r}")
        ra.allgather_fwd(q[r].to(dev()), kd, vd, o, lse, r, w.causal, w.scale)
        torch.cuda.synchronize()
        del kd, vd
        torch.cuda.empty_cache()
        check_rows(w, r, q[r], k, v, o, lse, lambda h: inputs.query_row_sample(w.id, h, w.C),
                   f"{w.name} all-gather H_kv={Hk} sampled rows", grp=w.H // Hk)


@pytest.fixture(scope="module")
def train_run_allgather():
    w = WORKLOADS[5]
    r = w.ranks[0]
    say(f"{w.name}: all-gather training inputs")
    q, k, v, do = gen_workload(w, with_do=True)
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    qd, dd = q[r].to(dev()), do[r].to(dev())
    o = torch.full((w.B, w.H, w.C, w.d), float("nan"), device=dev())
    lse = torch.full((w.B, w.H, w.C), float("nan"), device=dev())
    ra.allgather_fwd(qd, kd, vd, o, lse, r, w.causal, w.scale)
    dq = torch.full_like(o, float("nan"))
    dk, dv = (torch.full((w.B, w.H, w.P * w.C, w.d), float("nan"), device=dev()) for _ in range(2))
    say(f"{w.name}: all-gather backward of rank {r}")
    ra.allgather_bwd(qd, kd, vd, o, lse, dd, dq, dk, dv, r, w.causal, w.scale)
    torch.cuda.synchronize()
    out = dict(w=w, r=r, q=q[r], k=k, v=v, do=do[r], o=o.cpu(), lse=lse.cpu(), dq=dq.cpu(), dk=dk.cpu(),
               dv=dv.cpu())
    del kd, vd, qd, dd, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(600)
def test_allgather_train_forward_and_dq_sampled_rows(train_run_allgather):
    t = train_run_allgather
    w, r = t["w"], t["r"]
    check_rows(w, r, t["q"], t["k"], t["v"], t["o"], t["lse"], lambda h: inputs.query_row_sample(w.id, h, w.C),
               f"{w.name} all-gather forward sampled rows")

    def one(h):
        rows = inputs.query_row_sample(w.id, h, w.C)
        kh, vh = head_full(t["k"], h), head_full(t["v"], h)
        qh, doh = f64(t["q"][:, h:h + 1, rows]), f64(t["do"][:, h:h + 1, rows])
        rq, _, _ = oracle.attention_bwd(qh, kh, vh, doh, w.scale, True, q_pos=r * w.C + rows)
        gq = f64(t["dq"][:, h:h + 1, rows])
        return np.abs(gq - rq).max(), np.linalg.norm(gq - rq) ** 2, np.linalg.norm(rq) ** 2

    say(f"{w.name}: all-gather oracle dQ on 256 rows x {w.H} heads")
    res = fan_out(one, range(w.H))
    e_q = max(x[0] for x in res)
    rel = math.sqrt(sum(x[1] for x in res) / sum(x[2] for x in res))
    say(f"  max|ddQ|={e_q:.2e} rel={rel:.2e}")
    assert e_q <= TOL_GRAD and rel <= TOL_REL


@pytest.mark.timeout(900)
def test_allgather_train_dk_dv_sampled_key_rows(train_run_allgather):
    t = train_run_allgather
    w, r = t["w"], t["r"]
    heads = range(w.H)
    pos = r * w.C + np.arange(w.C)

    def one(h):
        kh, vh = head_full(t["k"], h), head_full(t["v"], h)
        qh, doh = f64(t["q"][:, h:h + 1]), f64(t["do"][:, h:h + 1])
        rows = np.concatenate([j * w.C + inputs.key_row_sample(w.id, h, j, w.C) for j in range(w.P)])
        rk, rv = oracle.attention_bwd_key_rows(qh, kh, vh, doh, w.scale, True, rows, q_pos=pos)
        gk, gv = f64(t["dk"][:, h:h + 1, rows]), f64(t["dv"][:, h:h + 1, rows])
        return (np.abs(gk - rk).max(), np.abs(gv - rv).max(),
                np.linalg.norm(gk - rk) ** 2 + np.linalg.norm(gv - rv) ** 2,
                np.linalg.norm(rk) ** 2 + np.linalg.norm(rv) ** 2)

    say(f"{w.name}: all-gather oracle dK/dV on 256 key rows x {w.P} chunks x all {w.H} heads")
    res = fan_out(one, heads)
    e_k, e_v = max(x[0] for x in res), max(x[1] for x in res)
    rel = math.sqrt(sum(x[2] for x in res) / sum(x[3] for x in res))
    say(f"  max|ddK|={e_k:.2e} max|ddV|={e_v:.2e} rel={rel:.2e}")
    assert e_k <= TOL_GRAD and e_v <= TOL_GRAD and rel <= TOL_REL


def test_allgather_train_gradient_sums_every_key(train_run_allgather):
    """Over the whole gathered sequence: sum_k dK_k = 0 and sum_k dV_k = sum_q dO_q."""
    t = train_run_allgather
    w = t["w"]
    dk, dv = t["dk"].double(), t["dv"].double()
    r_k = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
    sum_do = t["do"].double().sum(dim=2)
    r_v = ((dv.sum(dim=2) - sum_do).abs().max() / sum_do.abs().max()).item()
    say(f"{w.name}: all-gather max|sum dK|/sum|dK|={r_k:.2e}  max|sum dV - sum dO|/max|sum dO|={r_v:.2e}")
    assert r_k <= 1e-3 and r_v <= 1e-3
