"""The five synthetic ring-attention workloads and their work counts.

Each workload is one GPU's share of Ring Attention: a local query block of C
tokens (rank r) walking P KV chunks of C tokens each, B = 1.  "ranks" lists the
query blocks a run walks (all of them for the full-ring workloads).
"""

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    P: int
    C: int
    H: int
    d: int
    causal: bool
    ranks: tuple
    train: bool = False
    B: int = 1

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def S(self):
        return self.P * self.C


WORKLOADS = {
    1: Workload(1, "tiny ring fwd, S=512, P=4, H=2, d=64, non-causal, all ranks",
                P=4, C=128, H=2, d=64, causal=False, ranks=(0, 1, 2, 3)),
    2: Workload(2, "128K/CP=4 local share, rank 3, H=32, d=128, causal fwd",
                P=4, C=32768, H=32, d=128, causal=True, ranks=(3,)),
    3: Workload(3, "full ring S=32K, P=8, H=32, d=128, causal fwd, all ranks",
                P=8, C=4096, H=32, d=128, causal=True, ranks=tuple(range(8))),
    4: Workload(4, "1M/CP=8/TP=4 local share, rank 7, H=8, d=128, causal fwd",
                P=8, C=131072, H=8, d=128, causal=True, ranks=(7,)),
    5: Workload(5, "training share C=16K, P=4, rank 3, H=32, d=128, causal fwd+bwd",
                P=4, C=16384, H=32, d=128, causal=True, ranks=(3,), train=True),
}


def step_kinds(rank, P, causal):
    """Per ring step s: chunk j = (rank - s) mod P and whether it is the
    masked diagonal chunk, a full chunk, or skipped (causal, j > rank)."""
    out = []
    for s in range(P):
        j = (rank - s) % P
        if causal and s == 0:
            out.append((s, j, "diag"))
        elif causal and j > rank:
            out.append((s, j, "skip"))
        else:
            out.append((s, j, "full"))
    return out


MAX_WALK_CHUNKS = 16  # chunks one fused-walk launch can hold (ra_kernels.h kMaxWalkChunks)


def fused_walk_applies(w, rank):
    """Whether ra_ring_fwd in RA_RING_FUSED mode walks this rank's visible
    chunks in one launch (the library's rule: C a multiple of 64, at most 16
    visible chunks, visible chunks * C < 2^30); otherwise it runs the
    per-step resident walk."""
    nvis = sum(kind != "skip" for *_, kind in step_kinds(rank, w.P, w.causal))
    return w.C % 64 == 0 and nvis <= MAX_WALK_CHUNKS and nvis * w.C < 2 ** 30


def queue_steps_apply(w, ring_mode, cus):
    """Whether ra_ring_fwd runs the walk's full-chunk steps on persistent
    blocks with per-XCD work queues (the library's rule: the double-buffer
    walk, whose workspace holds the queue counters, with at least four
    (head, query tile) units of 256 query rows per compute unit)."""
    units = w.B * w.H * -(-w.C // 256)
    return ring_mode == "double_buffer" and units >= 4 * cus


def visible_pairs_per_head(w, rank):
    """(query, key) pairs a rank's walk evaluates per (batch, head)."""
    n = 0
    for _, _, kind in step_kinds(rank, w.P, w.causal):
        if kind == "full":
            n += w.C * w.C
        elif kind == "diag":
            n += w.C * (w.C + 1) // 2
    return n


def fwd_flops(w, ranks=None):
    """Algorithmic forward flops: 4*d per visible pair (QK^T and PV)."""
    ranks = w.ranks if ranks is None else ranks
    return sum(4 * w.d * w.B * w.H * visible_pairs_per_head(w, r) for r in ranks)


def bwd_flops(w, ranks=None):
    """Algorithmic backward flops: 10*d per visible pair (S recompute, dP, dV,
    dK, dQ)."""
    ranks = w.ranks if ranks is None else ranks
    return sum(10 * w.d * w.B * w.H * visible_pairs_per_head(w, r) for r in ranks)
