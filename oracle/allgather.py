"""fp64 reference of one GPU's share of all-gather sequence parallelism
(test infrastructure; see ``oracle/__init__.py``).

The page on sequence parallelism for 1M-token training, section "How
Sequence Parallelism Works": every GPU holds a
contiguous chunk of L/S tokens; the key/value chunks of all GPUs are
collected on every GPU by an all-gather, and each GPU computes attention for
its own query chunk against them.  The same page's "SP Methods: Head-to-Head
Comparison" table sets it beside Ulysses and Ring Attention.

Readings (the page leaves them open): the gathered sequence is the chunks in
index order, chunk j holding global tokens [j*C, (j+1)*C); causality is over
global positions, so rank r's query t sits at r*C + t; the backward returns
the gradient of the whole gathered key/value sequence from this rank's
queries (a reduce-scatter across ranks would hand each owner its slice).
"""

import numpy as np

from .attention import attention_bwd, attention_fwd


def allgather_kv(chunks):
    """The all-gather for one tensor: chunks[j] [B, Hk, C, d] in index order,
    concatenated along the sequence -> [B, Hk, P*C, d]."""
    return np.concatenate(list(chunks), axis=2)


def allgather_positions(rank, C):
    """Global positions of rank `rank`'s local query rows."""
    return rank * C + np.arange(C)


def allgather_share_fwd(q, k_chunks, v_chunks, rank, causal, scale):
    """(O, lse) of the rank's local queries q [B, H, C, d] over the gathered
    keys and values: [B, H, C, d] and [B, H, C]."""
    C = q.shape[2]
    return attention_fwd(q, allgather_kv(k_chunks), allgather_kv(v_chunks), scale, causal,
                         q_pos=allgather_positions(rank, C))


def allgather_share_bwd(q, k_chunks, v_chunks, do, rank, causal, scale):
    """Gradients of sum(dO * O) for the share above: dq [B, H, C, d] and dk,
    dv [B, Hk, P*C, d] over the whole gathered sequence (zero for keys no
    local query sees)."""
    C = q.shape[2]
    return attention_bwd(q, allgather_kv(k_chunks), allgather_kv(v_chunks), do, scale, causal,
                         q_pos=allgather_positions(rank, C))
