"""fp64 reference attention (test infrastructure; see ``oracle/__init__.py``).

All arrays are NumPy float64 with layout [B, H, S, d] (lse: [B, H, S]).  The
bf16 inputs the GPU consumes convert exactly to float64, so input rounding is
not error on either side.

Causality is over *global* positions: a query at global position p sees key
positions k <= p (diagonal inclusive).  The pages never say "causal"; this is
the plain decoder reading, with contiguous equal chunks (chunk j holds global
tokens [j*C, (j+1)*C)), following "Training Long-Context Models Without OOM:
Ring Attention", "Ring Attention Demystified", item 1 (the sequence is split
equally, each GPU holds a contiguous block of length s/N).
"""

import numpy as np

NEG_INF = -np.inf


def _kv_group(H, Hk):
    """Query heads per key/value head.  Grouped-query attention: query head h
    reads key/value head h // (H / Hk) (contiguous groups; the pages name GQA
    in "Training Long-Context Models Without OOM: Ring Attention", "Ring
    Attention vs. DeepSpeed Ulysses (All-to-All)", but not its head order).
    Hk == H is ordinary multi-head attention."""
    if Hk < 1 or H % Hk:
        raise ValueError(f"{H} query heads do not split into groups over {Hk} key/value heads")
    return H // Hk


def _visible_mask(q_pos, k_pos):
    """[nq, nk] bool: key k visible to query q under causal masking (k <= q)."""
    return k_pos[None, :] <= q_pos[:, None]


def attention_fwd(q, k, v, scale, causal, q_pos=None, k_pos=None, block=512):
    """Exact softmax attention over the whole (unchunked) key sequence.

    For every query row: s_k = scale * <q, k_k> over visible keys,
    lse = ln(sum_k exp(s_k)) (taken as m + ln sum exp(s - m), m = max),
    P_k = exp(s_k - lse), O = sum_k P_k v_k.

    This is what Ring Attention reaches exactly ("Training Long-Context Models
    Without OOM: Ring Attention", "Ring Attention Demystified": exact attention,
    the global s-by-s matrix never materialised on a GPU).  Here there is no
    chunking and no merge: each block of query rows meets every visible key at
    once.

    q: [B, H, Sq, d]; k, v: [B, Hk, Sk, d] with H a multiple of Hk (query
    head h uses key/value head h // (H / Hk)).
    q_pos: [Sq] global positions of the query rows (default 0..Sq-1).
    k_pos: [Sk] global positions of the keys (default 0..Sk-1).
    Returns (O [B, H, Sq, d], lse [B, H, Sq]).  A row with no visible key gets
    O = 0, lse = -inf (only possible when q_pos precedes every key).
    """
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    grp = _kv_group(H, k.shape[1])
    if q_pos is None:
        q_pos = np.arange(Sq)
    if k_pos is None:
        k_pos = np.arange(Sk)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    o = np.zeros((B, H, Sq, d), dtype=np.float64)
    lse = np.full((B, H, Sq), NEG_INF, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, block):
                r1 = min(Sq, r0 + block)
                qb = q[b, h, r0:r1]
                if causal:
                    # Only keys that some row of this block can see.
                    order = np.nonzero(k_pos <= q_pos[r0:r1].max())[0]
                else:
                    order = np.arange(Sk)
                if order.size == 0:
                    continue
                kb = k[b, h // grp, order]
                vb = v[b, h // grp, order]
                s = scale * (qb @ kb.T)
                if causal:
                    vis = _visible_mask(q_pos[r0:r1], k_pos[order])
                    s = np.where(vis, s, NEG_INF)
                m = s.max(axis=1)
                has = np.isfinite(m)
                m_safe = np.where(has, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                l = e.sum(axis=1)
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = np.where(has, m_safe + np.log(l), NEG_INF)
                p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
                o[b, h, r0:r1] = p @ vb
    return o, lse


def step_partial(q, k_chunk, v_chunk, scale, diagonal):
    """One ring step's partial: attention of the local query block against one
    KV chunk ("Context Parallelism", 2 "How It Works": step s, GPU i computes
    attention(Q_i, K_{i-s}, V_{i-s})).

    diagonal=True is the step-0 chunk under causal masking: local query t sees
    local key t' <= t.  Otherwise every key of the chunk is visible.
    Returns (o_partial, lse_partial), normalised within the chunk.
    """
    Sq = q.shape[2]
    Sk = k_chunk.shape[2]
    return attention_fwd(q, k_chunk, v_chunk, scale, causal=diagonal,
                         q_pos=np.arange(Sq), k_pos=np.arange(Sk))


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two normalised partials of the same query rows.

    The running softmax statistics (row maximum and running sum of
    exponentials) let a partial result be updated incrementally ("Training
    Long-Context Models Without OOM: Ring Attention", "Ring Attention
    Demystified"; "Context Parallelism", 2 "How It Works", last sentence).  In
    log-sum-exp form: lse = ln(e^lse_a + e^lse_b) and
    O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.
    An operand with lse = -inf contributes nothing; both -inf gives (0, -inf).
    """
    m = np.maximum(lse_a, lse_b)
    fin = np.isfinite(m)
    m_safe = np.where(fin, m, 0.0)
    wa = np.where(fin, np.exp(np.where(fin, lse_a - m_safe, 0.0)), 0.0)
    wb = np.where(fin, np.exp(np.where(fin, lse_b - m_safe, 0.0)), 0.0)
    wa = np.where(np.isneginf(lse_a), 0.0, wa)
    wb = np.where(np.isneginf(lse_b), 0.0, wb)
    tot = wa + wb
    with np.errstate(divide="ignore"):
        lse = np.where(fin, m_safe + np.log(np.where(fin, tot, 1.0)), NEG_INF)
    tot_safe = np.where(tot > 0, tot, 1.0)
    o = (wa / tot_safe)[..., None] * o_a + (wb / tot_safe)[..., None] * o_b
    return o, lse


def ring_fwd_chunked(q, k_chunks, v_chunks, rank, causal, scale):
    """The ring walk done on the CPU: per visible step a partial against chunk
    j = (rank - s) mod P, merged into the running (O, lse).

    Secondary reference for invariants only ("chunked with merge equals
    unchunked"); the expected value of a GPU ring output is
    ``attention_fwd`` over the unchunked sequence.
    """
    from .schedule import ring_schedule

    P = len(k_chunks)
    o = None
    lse = None
    for s, j, kind in ring_schedule(rank, P, causal):
        if kind == "skip":
            continue
        op, lp = step_partial(q, k_chunks[j], v_chunks[j], scale, diagonal=(kind == "diag"))
        if o is None:
            o, lse = op, lp
        else:
            o, lse = lse_merge(o, lse, op, lp)
    return o, lse


def _fwd_block_stats(qb, kb, vb, scale, vis):
    s = scale * (qb @ kb.T)
    if vis is not None:
        s = np.where(vis, s, NEG_INF)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    lse = m + np.log(l)
    p = e / l[:, None]
    return s, p, lse, p @ vb


def attention_bwd(q, k, v, do, scale, causal, q_pos=None, block=512):
    """Gradient of L = sum(dO * O) for O = attention_fwd(q, k, v).

    Textbook softmax-attention backward (the pages give none): with
    P = softmax(scale q k^T) over visible keys,
      dV = P^T dO;  dP = dO V^T;  D = rowsum(dO * O) = rowsum(P * dP);
      dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
    q, do: [B, H, Sq, d] (the local rows); k, v: [B, Hk, Sk, d] (the global
    sequence; query head h uses key/value head h // (H / Hk)).  Returns
    (dq [B,H,Sq,d], dk [B,Hk,Sk,d], dv [B,Hk,Sk,d]); only the given query rows
    contribute to dk, dv, and a key/value head's gradient sums over the query
    heads of its group.  Every query row must see at least one key.
    """
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    grp = _kv_group(H, k.shape[1])
    if q_pos is None:
        q_pos = np.arange(Sq)
    q_pos = np.asarray(q_pos)
    k_pos = np.arange(Sk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, block):
                r1 = min(Sq, r0 + block)
                nk = int(q_pos[r0:r1].max()) + 1 if causal else Sk
                nk = min(nk, Sk)
                kh = h // grp
                kb, vb = k[b, kh, :nk], v[b, kh, :nk]
                vis = _visible_mask(q_pos[r0:r1], k_pos[:nk]) if causal else None
                _, p, _, ob = _fwd_block_stats(q[b, h, r0:r1], kb, vb, scale, vis)
                dob = do[b, h, r0:r1]
                dp = dob @ vb.T
                D = (dob * ob).sum(axis=1)
                ds = p * (dp - D[:, None])
                dq[b, h, r0:r1] = scale * (ds @ kb)
                dk[b, kh, :nk] += scale * (ds.T @ q[b, h, r0:r1])
                dv[b, kh, :nk] += p.T @ dob
    return dq, dk, dv


def attention_bwd_key_rows(q, k, v, do, scale, causal, key_rows, q_pos=None, block=512):
    """dK and dV at selected key positions only (same definition as
    ``attention_bwd``).  Needs lse and D of every query row, so the full
    forward over all query rows is computed; only the columns of P, dP and dS
    that belong to ``key_rows`` are formed.

    Returns (dk_rows [B,Hk,len(key_rows),d], dv_rows [B,Hk,len(key_rows),d]).
    """
    B, H, Sq, d = q.shape
    Hk = k.shape[1]
    grp = _kv_group(H, Hk)
    if q_pos is None:
        q_pos = np.arange(Sq)
    q_pos = np.asarray(q_pos)
    key_rows = np.asarray(key_rows)
    o, lse = attention_fwd(q, k, v, scale, causal, q_pos=q_pos, block=block)
    nr = key_rows.size
    dk_r = np.zeros((B, Hk, nr, d))
    dv_r = np.zeros((B, Hk, nr, d))
    for b in range(B):
        for h in range(H):
            kh = h // grp
            ks = k[b, kh, key_rows]
            vs = v[b, kh, key_rows]
            for r0 in range(0, Sq, block):
                r1 = min(Sq, r0 + block)
                s = scale * (q[b, h, r0:r1] @ ks.T)
                if causal:
                    s = np.where(_visible_mask(q_pos[r0:r1], key_rows), s, NEG_INF)
                p = np.exp(s - lse[b, h, r0:r1, None])
                dob = do[b, h, r0:r1]
                dp = dob @ vs.T
                D = (dob * o[b, h, r0:r1]).sum(axis=1)
                ds = p * (dp - D[:, None])
                dk_r[b, kh] += scale * (ds.T @ q[b, h, r0:r1])
                dv_r[b, kh] += p.T @ dob
    return dk_r, dv_r
