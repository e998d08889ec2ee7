"""Plain fp64 CPU oracle for one GPU's share of Ring Attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library never routes through
it, and it imports nothing from the HIP side (no kernels, headers, tables or
helpers are shared).

What it computes, and the passage each function follows:

* ``attention.attention_fwd`` -- exact softmax attention of query rows over the
  unchunked key/value sequence.  Ring Attention is exact: after the walk every
  query block has attended to the whole global sequence ("Training Long-Context
  Models Without OOM: Ring Attention", section "Ring Attention Demystified",
  item 5 "Ring Completion"; "Context Parallelism", section 2 "Ring Attention",
  "How It Works").  The oracle therefore is the plain definition, not the ring.
  Key/value tensors may carry fewer heads than the queries (grouped-query
  attention, named in "Training Long-Context Models Without OOM: Ring
  Attention", "Ring Attention vs. DeepSpeed Ulysses (All-to-All)"): query
  head h reads key/value head h // (H / Hk), and the backward sums a key/value
  head's gradient over its group.  Pinned against the library's attention
  with grouped heads, forward and autograd.
* ``attention.attention_bwd`` / ``attention_bwd_key_rows`` -- the textbook
  gradient of softmax attention.  The pages give no backward formula; this
  is the plain one, with P recomputed from the final log-sum-exp of each
  query row.
* ``attention.lse_merge`` / ``ring_fwd_chunked`` -- the online-softmax merge of
  partial results ("Training Long-Context Models Without OOM: Ring
  Attention", "Ring Attention Demystified", paragraph on running softmax
  statistics; "Context Parallelism", 2 "How It Works", last sentence).  Used by
  the tests only to check invariants of the method, never as the expected
  value of a GPU output.
* ``ulysses.ulysses_share`` / ``ulysses_gather`` / ``ulysses_scatter`` -- one
  rank's share of head-partitioned (Ulysses) sequence parallelism: the
  all-to-all regrouping by head, full attention for the rank's heads over the
  whole sequence, and the regrouping back ("Context Parallelism", 3 "Ulysses
  (DeepSpeed)", steps 1-4).  Pinned against the library's attention and
  against the ring walk (``tests/test_oracle_ulysses.py``).
* ``allgather.allgather_share_fwd`` / ``allgather_share_bwd`` /
  ``allgather_kv`` -- one rank's share of all-gather sequence parallelism:
  the key/value chunks gathered in index order, then exact attention of the
  rank's query chunk (at its global positions) over them, and its gradient
  (the page on sequence parallelism for 1M-token training, "How Sequence
  Parallelism Works").  Pinned against the library's attention, its
  autograd and the ring walk (``tests/test_oracle_allgather.py``).
* ``schedule.ring_schedule`` -- which KV chunk a rank uses at each step
  ("Context Parallelism", 2 "How It Works": step s uses K_{i-s}, V_{i-s};
  "Training Long-Context Models Without OOM", "Ring Attention Demystified",
  items 2-5).
* ``schedule.kv_bytes_per_step`` -- KV rotation bytes ("Context Parallelism",
  2 "Communication" and "Worked Example").

Every function here is pinned by ``tests/test_oracle.py`` against something
other than itself (a library routine, brute force, closed forms, invariants,
or numbers the pages print).  No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_fwd,
    attention_bwd,
    attention_bwd_key_rows,
    lse_merge,
    step_partial,
    ring_fwd_chunked,
)
from .schedule import ring_schedule, kv_bytes_per_step, visible_pairs  # noqa: F401
