"""fp64 reference of one GPU's share of head-partitioned (Ulysses) sequence
parallelism (test infrastructure; see ``oracle/__init__.py``).

"Context Parallelism", section 3 "Ulysses (DeepSpeed)": every GPU starts with
Q, K, V of its S/P tokens (step 1); an all-to-all regroups them by head, so a
GPU holds all S tokens of N_h/P heads (step 2); it computes full attention for
those heads (step 3); a second all-to-all restores the split by sequence
(step 4).  "Training Long-Context Models Without OOM: Ring Attention", "Ring
Attention vs. DeepSpeed Ulysses (All-to-All)", describes the same exchange.

Readings (the pages leave them open): rank r receives the contiguous heads
r*H/P .. (r+1)*H/P - 1; queries are regrouped like keys and values (full
attention over all S tokens needs every query of those heads); positions are
global, chunk j holding tokens [j*C, (j+1)*C).
"""

import numpy as np

from .attention import attention_fwd


def ulysses_heads(rank, P, H):
    """The heads rank `rank` of P computes: a contiguous block of H/P."""
    if H % P:
        raise ValueError(f"{H} heads do not split over {P} ranks")
    hs = H // P
    return np.arange(rank * hs, (rank + 1) * hs)


def ulysses_gather(chunks, rank):
    """Step 2 for one rank: its heads of every sequence chunk, concatenated
    along the sequence.  chunks[j]: [B, H, C, d] -> [B, H/P, P*C, d]."""
    P = len(chunks)
    heads = ulysses_heads(rank, P, chunks[0].shape[1])
    return np.concatenate([c[:, heads] for c in chunks], axis=2)


def ulysses_share(q_chunks, k_chunks, v_chunks, rank, causal, scale):
    """Steps 2 and 3 for one rank: (O, lse) of its heads over the whole
    sequence, [B, H/P, P*C, d] and [B, H/P, P*C]."""
    q = ulysses_gather(q_chunks, rank)
    k = ulysses_gather(k_chunks, rank)
    v = ulysses_gather(v_chunks, rank)
    return attention_fwd(q, k, v, scale, causal)


def ulysses_scatter(o_shares, C):
    """Step 4: the ranks' head-partitioned outputs o_shares[r] ([B, H/P, P*C, d])
    back to sequence chunks: chunk j is [B, H, C, d] with every head."""
    P = len(o_shares)
    return [np.concatenate([o[:, :, j * C:(j + 1) * C] for o in o_shares], axis=1) for j in range(P)]
