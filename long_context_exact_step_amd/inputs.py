"""Seeded synthetic inputs for the ring-attention workloads.

This module only draws random numbers; it holds none of the attention
arithmetic, so both the HIP path's tests/bench and the CPU oracle can use it.

Values are i.i.d. N(0, 1) drawn in fp32 by torch's CPU generator and rounded to
bf16 with round-to-nearest-even.  Each tensor chunk has its own seed, so any
chunk can be regenerated on its own:

    seed = 1_000_000 * workload + 1_000 * kind + chunk

with kind 0 = Q, 1 = K, 2 = V, 3 = dO and chunk the chunk index (the query
block of rank r is chunk r).  Shapes are [B, H, C, d] (BHSD).
"""

import numpy as np
import torch

Q, K, V, DO = 0, 1, 2, 3


def chunk_seed(workload, kind, chunk):
    return 1_000_000 * int(workload) + 1_000 * int(kind) + int(chunk)


def randn_bf16(shape, seed):
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(torch.bfloat16)


def chunk(workload, kind, j, B, H, C, d):
    """One [B, H, C, d] bf16 CPU tensor of the given kind and chunk index."""
    return randn_bf16((B, H, C, d), chunk_seed(workload, kind, j))


def sample_rows(n, count, seed):
    """Sorted distinct row indices in [0, n): the first and last row plus a
    seeded uniform sample of count - 2 rows in between.  All rows if
    count >= n."""
    if count >= n:
        return np.arange(n)
    if count < 2:
        raise ValueError("count must be >= 2")
    rng = np.random.default_rng(int(seed))
    mid = rng.choice(n - 2, size=count - 2, replace=False) + 1
    return np.sort(np.concatenate([np.array([0, n - 1]), mid]))


def query_row_sample(workload, h, C, count=256):
    return sample_rows(C, count, 1_000_000 * int(workload) + 900 + int(h))


def key_row_sample(workload, h, j, C, count=256):
    return sample_rows(C, count, 1_000_000 * int(workload) + 950 + 8 * int(h) + int(j))
