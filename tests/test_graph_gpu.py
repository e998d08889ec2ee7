"""The library's calls captured in a HIP graph.  The library launches kernels
and device-to-device copies on the caller's streams and orders the staging
slots with events; it enqueues no memset, allocation or synchronisation, so a
caller may capture a whole training step (forward walk in double-buffer mode
with its copy stream, backward walk; or the Ulysses or all-gather share's
forward and backward) and replay it.  Every replay must give
the eager result bit for bit, with the program's own eager work and
synchronisations between replays, and a replay after the inputs change in
place must match an eager run on the new inputs."""

import math

import pytest
import torch

import long_context_exact_step_amd as ra
from long_context_exact_step_amd import inputs
from parity import dev, gen, ring_tensors

pytestmark = pytest.mark.gpu


class Step:
    """Static buffers of one rank's training step and the calls that fill them."""

    def __init__(self, B, H, P, C, d, rank, causal, H_kv=None):
        Hk = H if H_kv is None else H_kv
        q, k, v, do = ring_tensors(110, B, H, P, C, d, with_do=True, ranks=[rank], H_kv=Hk)
        self.q, self.do = q[rank].to(dev()), do[rank].to(dev())
        self.k = [t.to(dev()) for t in k]
        self.v = [t.to(dev()) for t in v]
        self.rank, self.causal, self.scale = rank, causal, 1 / math.sqrt(d)
        self.o = torch.empty(B, H, C, d, device=dev())
        self.lse = torch.empty(B, H, C, device=dev())
        self.dq = torch.empty(B, H, C, d, device=dev())
        self.dk = [torch.empty(B, Hk, C, d, device=dev()) for _ in range(P)]
        self.dv = [torch.empty(B, Hk, C, d, device=dev()) for _ in range(P)]
        self.ws_f = torch.empty(ra.workspace_bytes(P, B, H, C, d, "double_buffer", H_kv=Hk), dtype=torch.uint8,
                                device=dev())
        self.ws_b = torch.empty(ra.workspace_bytes(P, B, H, C, d, "resident", bwd=True, H_kv=Hk),
                                dtype=torch.uint8, device=dev())
        self.copy_stream = torch.cuda.Stream(dev())

    def run(self):
        for t in self.dk + self.dv:
            t.zero_()  # a fill kernel, not a memset node
        ra.ring_fwd(self.q, self.k, self.v, self.o, self.lse, self.rank, self.causal, self.scale,
                    ring_mode="double_buffer", workspace=self.ws_f, copy_stream=self.copy_stream)
        ra.ring_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.dq, self.dk, self.dv, self.rank,
                    self.causal, self.scale, workspace=self.ws_b)

    def outputs(self):
        return [t.clone() for t in [self.o, self.lse, self.dq, *self.dk, *self.dv]]


def _same(got, want, what):
    for n, (a, b) in enumerate(zip(got, want)):
        assert torch.equal(a, b), f"{what}: output {n} differs from the eager run"


@pytest.mark.parametrize("B,H,H_kv,P,C,d,rank,causal", [
    (1, 2, None, 4, 200, 128, 3, True),
    (2, 4, 2, 3, 130, 64, 1, False),
    # four (head, query tile) units per compute unit: the full-chunk steps
    # run persistent blocks whose work-queue counters the kernels re-zero
    (1, 32, 8, 3, 8192, 64, 2, True),
])
def test_captured_training_step_replays_bit_identical(B, H, H_kv, P, C, d, rank, causal):
    print(f"graph B={B} H={H} H_kv={H_kv} P={P} C={C} d={d} rank={rank} causal={causal}", flush=True)
    s = Step(B, H, P, C, d, rank, causal, H_kv)
    s.run()  # eager warm-up: the library's per-thread events exist before capture
    torch.cuda.synchronize()
    want = s.outputs()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.run()
    torch.cuda.synchronize()

    # Another eager walk on other buffers between replays.
    other = Step(B, H, P, C, d, (rank + 1) % P, causal, H_kv)
    for rep in range(3):
        for t in [s.o, s.lse, s.dq, *s.dk, *s.dv]:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(s.outputs(), want, f"replay {rep}")
        other.run()
        torch.cuda.synchronize()

    # New inputs, copied into the captured buffers in place.
    Hk = H if H_kv is None else H_kv
    s.q.copy_(gen(111, inputs.Q, rank, B, H, C, d).to(dev()))
    for j in range(P):
        s.k[j].copy_(gen(111, inputs.K, j, B, Hk, C, d).to(dev()))
        s.v[j].copy_(gen(111, inputs.V, j, B, Hk, C, d).to(dev()))
    g.replay()
    torch.cuda.synchronize()
    got = s.outputs()
    s.run()
    torch.cuda.synchronize()
    _same(got, s.outputs(), "replay on new inputs")
    assert not torch.equal(got[0], want[0]), "the replay did not read the new inputs"


def _replays_match(run, outputs, reps=3):
    """Eager run, capture, then replays with eager work between them: every
    replay must reproduce the eager outputs bit for bit."""
    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in outputs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same([t.clone() for t in outputs], want, f"replay {rep}")
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_captured_ulysses_and_allgather_shares():
    """The other two parallel shares (2D regroup / gather copies, the row
    pre-pass and the step kernels) captured and replayed likewise."""
    B, H, Hk, P, C, d, rank = 1, 4, 2, 2, 130, 128, 1
    print(f"graph ulysses/allgather B={B} H={H} H_kv={Hk} P={P} C={C} d={d} rank={rank}", flush=True)
    scale = 1 / math.sqrt(d)
    q, k, v, do = ring_tensors(114, B, H, P, C, d, with_do=True)
    qc = [q[r].to(dev()) for r in range(P)]
    dc = [do[r].to(dev()) for r in range(P)]
    kc = [t.to(dev()) for t in k]
    vc = [t.to(dev()) for t in v]
    S, Hs = P * C, H // P
    uo = torch.empty(B, Hs, S, d, device=dev())
    ul = torch.empty(B, Hs, S, device=dev())
    udq, udk, udv = (torch.empty(B, Hs, S, d, device=dev()) for _ in range(3))
    uws_f = torch.empty(ra.ulysses_workspace_bytes(P, B, H, C, d), dtype=torch.uint8, device=dev())
    uws_b = torch.empty(ra.ulysses_workspace_bytes(P, B, H, C, d, bwd=True), dtype=torch.uint8, device=dev())

    def ulysses():
        ra.ulysses_fwd(qc, kc, vc, uo, ul, rank, True, scale, workspace=uws_f)
        ra.ulysses_bwd(qc, kc, vc, dc, uo, ul, udq, udk, udv, rank, True, scale, workspace=uws_b)

    _replays_match(ulysses, [uo, ul, udq, udk, udv])

    kg = [gen(114, inputs.K, j, B, Hk, C, d).to(dev()) for j in range(P)]
    vg = [gen(114, inputs.V, j, B, Hk, C, d).to(dev()) for j in range(P)]
    ao = torch.empty(B, H, C, d, device=dev())
    al = torch.empty(B, H, C, device=dev())
    adq = torch.empty(B, H, C, d, device=dev())
    adk, adv = (torch.empty(B, Hk, S, d, device=dev()) for _ in range(2))
    aws_f = torch.empty(ra.allgather_workspace_bytes(P, B, H, C, d, H_kv=Hk), dtype=torch.uint8, device=dev())
    aws_b = torch.empty(ra.allgather_workspace_bytes(P, B, H, C, d, H_kv=Hk, bwd=True), dtype=torch.uint8,
                        device=dev())

    def allgather():
        ra.allgather_fwd(qc[rank], kg, vg, ao, al, rank, True, scale, workspace=aws_f)
        ra.allgather_bwd(qc[rank], kg, vg, ao, al, dc[rank], adq, adk, adv, rank, True, scale, workspace=aws_b)

    _replays_match(allgather, [ao, al, adq, adk, adv])
