"""Ring schedule and KV-rotation accounting (test infrastructure; see
``oracle/__init__.py``)."""


def ring_schedule(rank, P, causal):
    """The ring walk of one rank: a list of (step, chunk, kind).

    Step s uses KV chunk j = (rank - s) mod P: step 0 is the local chunk, step 1
    the chunk received from the left neighbour, and so on until every chunk has
    been seen once after P - 1 rotations ("Context Parallelism", 2 "Ring
    Attention", "How It Works"; "Training Long-Context Models Without OOM: Ring
    Attention", "Ring Attention Demystified", items 2-5).

    kind: "diag" for step 0 under causal masking (the chunk holding the query
    block's own positions), "skip" for a chunk wholly in the future of every
    query (j > rank, causal only), "full" otherwise.
    """
    out = []
    for s in range(P):
        j = (rank - s) % P
        if causal and s == 0:
            kind = "diag"
        elif causal and j > rank:
            kind = "skip"
        else:
            kind = "full"
        out.append((s, j, kind))
    return out


def kv_bytes_per_step(C, d_k, H=1, B=1, elem_bytes=2):
    """Bytes of K plus V that one rotation moves: 2 x (S/P) x d_k x 2 bytes per
    head in bf16 ("Context Parallelism", 2 "Communication", per-step formula).
    The page's formula is per head; H heads and B sequences multiply it."""
    return 2 * B * H * C * d_k * elem_bytes


def visible_pairs(C, P, rank, causal):
    """Number of (query, key) pairs one rank's walk evaluates per (batch, head),
    counted by brute force over the schedule: C*C for a full chunk,
    C*(C+1)/2 for the diagonal chunk, 0 for a skipped one."""
    total = 0
    for _, _, kind in ring_schedule(rank, P, causal):
        if kind == "full":
            total += C * C
        elif kind == "diag":
            total += sum(t + 1 for t in range(C))
    return total
