/*
 * ra.h -- one GPU's share of Ring Attention, hand-written HIP for MI355X
 * (gfx950).  C ABI: plain pointers, sizes and status codes; no C++ or torch
 * types cross it.
 *
 * The method.  The sequence is split into P equal contiguous chunks; the GPU
 * of rank r keeps its query chunk Q_r while the key/value chunks travel round
 * a ring.  At step s it computes exact attention of Q_r against chunk
 * j = (r - s) mod P and folds the result into running softmax statistics, so
 * after P - 1 rotations Q_r has attended to the whole sequence without the
 * global score matrix ever being formed ("Training Long-Context Models
 * Without OOM: Ring Attention", section "Ring Attention Demystified", items
 * 1-5; "Context Parallelism", section 2 "Ring Attention", "How It Works").
 * The per-step kernel is FlashAttention-style tiling: scores live only in
 * on-chip tiles, with a running row maximum and running sum of exponentials
 * (same section of the first page).  On one GPU the rotation is emulated: all
 * P chunks are resident and the ring walk is a double-buffered copy into a
 * two-slot staging area.
 *
 * Conventions shared by every entry point.
 *   Layout: q, k, v, dO are bf16 [B, H, S, d] contiguous ("BHSD"), the
 *     d values of one token adjacent.  o, o_partial, dq, dk, dv are fp32 in
 *     the same layout; lse and lse_partial are fp32 [B, H, S].
 *   lse is the natural logarithm of sum_k exp(scale * q . k_k) over the keys
 *     a row has seen; o is normalised (the softmax-weighted mean of v).  A
 *     row that has seen no key has o = 0 and lse = -inf.
 *   d must be 64 or 128; B, H and every sequence length must be >= 1 (any
 *     length: ragged tails are masked in the kernels).  B * H * S must stay
 *     below 2^31 for every tensor (RA_ERR_SHAPE otherwise); a single chunk
 *     may exceed 4 GiB.
 *   Every device pointer must be 16-byte aligned.
 *   Causality is over global positions with the diagonal included: query at
 *     global position p sees key positions <= p.  Chunk j holds global
 *     tokens [j*C, (j+1)*C).  So under causal masking chunk j < r is fully
 *     visible to rank r, chunk r is lower-triangular, chunks j > r are
 *     skipped.
 *   stream / copy_stream: a hipStream_t passed as void* (NULL = the null
 *     stream).  Work is enqueued asynchronously on it; device faults surface
 *     at the caller's next synchronisation.
 *   Ownership: the caller owns every buffer.  Hot calls allocate no device
 *     memory; they only read and write the buffers passed in.
 *   Errors: arguments are validated on the host before anything is
 *     enqueued; on any non-zero status nothing has been enqueued, except
 *     RA_ERR_HIP which reports a failed launch or runtime call (work
 *     enqueued before it may still run).  ra_last_error() then holds a
 *     message for the calling thread.  No C++ exception crosses the ABI.
 *   Thread safety: calls on distinct streams may run concurrently.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_VERSION 6

enum ra_status {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL */
  RA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  RA_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  RA_ERR_UNSUPPORTED = 4, /* d is not 64 or 128, or an unknown mode */
  RA_ERR_RANK = 5,        /* rank outside [0, P) */
  RA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  RA_ERR_HIP = 7          /* a HIP runtime call or launch failed */
};

enum ra_ring_mode {
  RA_RING_RESIDENT = 0,      /* walk the resident chunks in ring order, no copies */
  RA_RING_DOUBLE_BUFFER = 1, /* stage each chunk into a 2-slot buffer first (the
                                emulated receive), overlapped with the previous
                                step's compute: on copy_stream when given, else
                                by the previous step's kernel itself */
  RA_RING_FUSED = 2          /* resident chunks walked by one launch: the
                                online-softmax state runs on from chunk to
                                chunk in registers and no partial crosses HBM.
                                Needs C % 64 == 0, at most 16 visible
                                chunks and (visible chunks) * C < 2^30;
                                otherwise the call runs as RA_RING_RESIDENT.  Chunks are visited in index
                                order, so results differ from the ring order's
                                by rounding only. */
};

/* Library version (RA_VERSION). */
int ra_version(void);

/* Human-readable name of a status code; never NULL. */
const char* ra_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* ra_last_error(void);

/*
 * ra_step_fwd -- one ring step's attention partial.
 *
 * Exact attention of the query block q [B,H,Sq,d] against one KV chunk
 * k, v [B,H,Sk,d] ("Context Parallelism", 2 "How It Works": at step s GPU i
 * computes attention(Q_i, K_{i-s}, V_{i-s})).  Writes the normalised partial
 * o_partial [B,H,Sq,d] and its log-sum-exp lse_partial [B,H,Sq] (both fp32,
 * overwritten).  scale multiplies q . k before the softmax.
 *
 * The diagonal mask (local query t sees local keys <= t) applies iff
 * causal != 0 and step == 0; that case needs Sq == Sk.  Every other call is
 * unmasked: skipping chunks in the future of the query block is the
 * caller's business (ra_ring_fwd does it).  step < 0 is RA_ERR_SHAPE.
 */
int ra_step_fwd(const void* q, const void* k, const void* v,
                float* o_partial, float* lse_partial,
                int B, int H, int Sq, int Sk, int d,
                float scale, int step, int causal, void* stream);

/*
 * ra_lse_merge -- fold a partial into a running result, in place.
 *
 * With lse' = ln(e^lse + e^lse_p):
 *   o <- e^(lse - lse') o + e^(lse_p - lse') o_partial,  lse <- lse'
 * This is the online-softmax update that lets partial outputs against
 * separate KV chunks be combined incrementally ("Training Long-Context Models
 * Without OOM: Ring Attention", "Ring Attention Demystified"; "Context
 * Parallelism", 2 "How It Works").  An operand with lse = -inf contributes
 * nothing; both -inf leaves o = 0, lse = -inf.  o, o_partial [B,H,S,d],
 * lse, lse_partial [B,H,S], fp32.  o/lse may not alias the partial.
 */
int ra_lse_merge(float* o, float* lse, const float* o_partial,
                 const float* lse_partial, int B, int H, int S, int d,
                 void* stream);

/*
 * Device workspace bytes ra_ring_fwd (bwd == 0) or ra_ring_bwd (bwd != 0)
 * needs for these sizes.  Double-buffer forward: two slots of one K and one
 * V chunk, 4 * B*H*C*d * 2 bytes, then 1024 bytes of work-queue counters.
 * Resident forward: 0.  Backward: two fp32 values per row, -rowsum(dO * O)
 * and lse * log2(e), 2 * B*H*C * 4 bytes.  Returns 0 for invalid sizes.
 */
size_t ra_ring_workspace_bytes(int P, int B, int H, int C, int d,
                               int ring_mode, int bwd);

/*
 * ra_ring_fwd -- rank `rank`'s whole ring walk, forward.
 *
 * q [B,H,C,d] is the local query chunk (global tokens [rank*C, (rank+1)*C)).
 * k_chunks and v_chunks are HOST arrays of P device pointers, chunk j at
 * index j, each [B,H,C,d] bf16.  Step s = 0..P-1 uses chunk
 * j = (rank - s) mod P ("Context Parallelism", 2 "How It Works").  Under
 * causal masking step 0 is the diagonal chunk and chunks j > rank are skipped
 * (no copy, no launch).  Each visible step runs one kernel that computes the
 * step's partial in on-chip tiles and merges it with the running (o, lse) in
 * its epilogue, so only o and lse touch memory between steps.
 * o [B,H,C,d] and lse [B,H,C] (fp32) are overwritten with the final result.
 *
 * ring_mode RA_RING_DOUBLE_BUFFER needs ra_ring_workspace_bytes(...) of
 * workspace: the chunk of step s >= 1 is copied into slot (s-1) & 1 while
 * step s-1 computes -- the stand-in for the ring's receive from the left
 * neighbour ("Training Long-Context Models Without OOM: Ring Attention",
 * "Ring Attention Demystified", items 3-4).  With a copy_stream the copies
 * run there, with events ordering slot reuse.  With copy_stream NULL the
 * kernel of step s-1 makes the copy itself: each of its blocks copies a
 * share of the chunk once its own tiles are done, so the walk is one
 * stream of kernels with no copies or events elsewhere (cheaper per step
 * for short chunks).  The workspace also holds the work-queue counters of
 * the full-chunk steps: with at least four (head, query tile) units per
 * compute unit, such a step runs one persistent block per compute unit, taking
 * units from its XCD's queue first and then from the other XCDs', so that
 * a slower XCD does not set the step's length.  Results are the same bits
 * as with one block per unit.
 * RA_RING_RESIDENT reads the chunks in place and needs no workspace.
 * When the call returns, all work is ordered on `stream` (copy_stream work
 * is joined back into it).
 */
int ra_ring_fwd(const void* q, const void* const* k_chunks,
                const void* const* v_chunks, int P, float* o, float* lse,
                int rank, int causal, float scale, int B, int H, int C, int d,
                int ring_mode, void* workspace, size_t workspace_bytes,
                void* stream, void* copy_stream);

/*
 * ra_ring_bwd -- rank `rank`'s ring walk, backward.
 *
 * Gradient of L = sum(dO * o) for the o that ra_ring_fwd produced.  The pages
 * give no backward; this is the textbook softmax-attention gradient with the
 * probabilities recomputed from the final lse (no merge is needed):
 *   P = exp(scale q k^T - lse), dV_j += P^T dO, dP = dO v_j^T,
 *   D = rowsum(dO * o), dS = P (dP - D), dq += scale dS k_j,
 *   dK_j += scale dS^T q.
 * q, dO [B,H,C,d] bf16; o [B,H,C,d] and lse [B,H,C] fp32 from the forward;
 * dq [B,H,C,d] fp32 is overwritten.  dk_chunks and dv_chunks are HOST arrays
 * of P device pointers to fp32 [B,H,C,d] accumulators that are ADDED TO
 * (the caller zeroes them once), so walking every rank's share accumulates
 * the full-sequence gradient.  Skipped chunks are not touched.  workspace
 * must hold ra_ring_workspace_bytes(P,B,H,C,d,0,1) bytes.
 */
int ra_ring_bwd(const void* q, const void* const* k_chunks,
                const void* const* v_chunks, int P, const float* o,
                const float* lse, const void* dO, float* dq,
                float* const* dk_chunks, float* const* dv_chunks, int rank,
                int causal, float scale, int B, int H, int C, int d,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query attention (GQA): key/value tensors carry H_kv heads for the
 * H query heads, H_kv dividing H, and query head h reads key/value head
 * h / (H / H_kv) (contiguous groups).  Ring attention's per-GPU work does not
 * depend on the head count, which is its stated advantage over all-to-all
 * sequence parallelism for GQA models ("Training Long-Context Models Without
 * OOM: Ring Attention", "Ring Attention vs. DeepSpeed Ulysses (All-to-All)").
 * Each *_gqa entry point is the call of the same name without the suffix,
 * with H_kv inserted after H; the suffix-free calls are these with
 * H_kv == H.  The differences:
 *   - k, v, k_chunks[j], v_chunks[j] are [B,H_kv,*,d] bf16; q, dO, o, lse,
 *     dq, o_partial, lse_partial keep H heads.
 *   - dk_chunks[j], dv_chunks[j] are [B,H_kv,C,d] fp32 accumulators; each
 *     key/value head's gradient sums over the query heads of its group.
 *   - The double-buffer workspace holds H_kv-head chunks:
 *     4 * B*H_kv*C*d * 2 + 1024 bytes.  The backward workspace is unchanged
 *     (2 * B*H*C * 4 bytes).
 *   - H_kv < 1, or H not a multiple of H_kv, is RA_ERR_SHAPE (and 0 bytes
 *     from ra_ring_workspace_bytes_gqa).  Every other contract (ownership,
 *     validation before enqueueing, asynchrony, status codes) is as for the
 *     suffix-free call.
 */
int ra_step_fwd_gqa(const void* q, const void* k, const void* v,
                    float* o_partial, float* lse_partial,
                    int B, int H, int H_kv, int Sq, int Sk, int d,
                    float scale, int step, int causal, void* stream);
size_t ra_ring_workspace_bytes_gqa(int P, int B, int H, int H_kv, int C,
                                   int d, int ring_mode, int bwd);
int ra_ring_fwd_gqa(const void* q, const void* const* k_chunks,
                    const void* const* v_chunks, int P, float* o, float* lse,
                    int rank, int causal, float scale, int B, int H, int H_kv,
                    int C, int d, int ring_mode, void* workspace,
                    size_t workspace_bytes, void* stream, void* copy_stream);
int ra_ring_bwd_gqa(const void* q, const void* const* k_chunks,
                    const void* const* v_chunks, int P, const float* o,
                    const float* lse, const void* dO, float* dq,
                    float* const* dk_chunks, float* const* dv_chunks, int rank,
                    int causal, float scale, int B, int H, int H_kv, int C,
                    int d, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * ra_ring_bwd_noalloc -- ra_ring_bwd_gqa for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, or
 * harnesses that forbid hipMalloc.  Same arguments, results and contracts as
 * ra_ring_bwd_gqa (H_kv == H for multi-head attention), minus the workspace:
 * the row terms the backward needs (-rowsum(dO * o) and lse in base 2, two
 * floats per query row) live in a static device array of the library,
 * sized for RA_NOALLOC_MAX_ROWS query rows (16 MiB), of which each device
 * keeps its own copy until the process ends.  The call allocates and frees
 * nothing.
 *   - B*H*C above RA_NOALLOC_MAX_ROWS is RA_ERR_WORKSPACE, before anything
 *     is enqueued.
 *   - The first call on a device looks up the array's address there
 *     (RA_ERR_HIP if that fails).
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents (each call writes every row it reads before
 *     reading it, so nothing needs clearing).  Calls that overlap on one
 *     device -- on different streams, or from different threads -- race on
 *     it and must be ordered by the caller.
 */
#define RA_NOALLOC_MAX_ROWS (1 << 21)
int ra_ring_bwd_noalloc(const void* q, const void* const* k_chunks,
                        const void* const* v_chunks, int P, const float* o,
                        const float* lse, const void* dO, float* dq,
                        float* const* dk_chunks, float* const* dv_chunks,
                        int rank, int causal, float scale, int B, int H,
                        int H_kv, int C, int d, void* stream);

/*
 * ra_ulysses_fwd -- one GPU's share of head-partitioned (Ulysses) sequence
 * parallelism, forward ("Context Parallelism", 3 "Ulysses (DeepSpeed)";
 * "Training Long-Context Models Without OOM: Ring Attention", "Ring
 * Attention vs. DeepSpeed Ulysses (All-to-All)").  The sequence is split in
 * P chunks of C tokens (q_chunks[j], k_chunks[j], v_chunks[j]: HOST arrays of
 * P device pointers to [B,H,C,d] bf16, chunk j = global tokens [jC,(j+1)C)).
 * Rank `rank` regroups its heads rank*H/P .. (rank+1)*H/P-1 of every chunk
 * into workspace (on one GPU this stands in for the all-to-all of step 2),
 * then computes exact attention for those heads over the whole sequence of
 * S = P*C tokens (step 3; causal != 0 masks key positions after the query's).
 * Writes o [B,H/P,S,d] and lse [B,H/P,S] fp32 (overwritten), the rank's
 * head-partitioned output; step 4's all-to-all back to sequence chunks is the
 * exchange between GPUs and is not performed.  Needs H % P == 0
 * (RA_ERR_SHAPE) and ra_ulysses_workspace_bytes(P,B,H,C,d,0) bytes of
 * 16-byte-aligned workspace (RA_ERR_WORKSPACE).  Other contracts as for
 * ra_ring_fwd.
 *
 * ra_ulysses_bwd -- the same share's backward (the softmax-attention
 * gradient with P recomputed from the share's final lse, as ra_ring_bwd).
 * dO_chunks: HOST array of P device pointers to [B,H,C,d] bf16, split by
 * sequence like q_chunks and regrouped the same way; o [B,H/P,S,d] and lse
 * [B,H/P,S] are ra_ulysses_fwd's outputs.  dq, dk, dv [B,H/P,S,d] fp32 are
 * overwritten with the gradients of the rank's heads over the whole sequence
 * (complete: every query of those heads is local).  Workspace:
 * ra_ulysses_workspace_bytes(P,B,H,C,d,1) bytes.
 *
 * ra_ulysses_workspace_bytes: bwd == 0: regrouped Q, K, V,
 * 3 * B*(H/P)*P*C*d * 2 bytes; bwd != 0: regrouped Q, K, V, dO and two fp32
 * values per row, 4 * B*(H/P)*P*C*d * 2 + 2 * B*(H/P)*P*C * 4 bytes.  0 for
 * invalid sizes.
 */
size_t ra_ulysses_workspace_bytes(int P, int B, int H, int C, int d, int bwd);
int ra_ulysses_fwd(const void* const* q_chunks, const void* const* k_chunks,
                   const void* const* v_chunks, int P, float* o, float* lse,
                   int rank, int causal, float scale, int B, int H, int C,
                   int d, void* workspace, size_t workspace_bytes,
                   void* stream);
int ra_ulysses_bwd(const void* const* q_chunks, const void* const* k_chunks,
                   const void* const* v_chunks, const void* const* dO_chunks,
                   int P, const float* o, const float* lse, float* dq,
                   float* dk, float* dv, int rank, int causal, float scale,
                   int B, int H, int C, int d, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * ra_allgather_fwd -- one GPU's share of all-gather sequence parallelism,
 * forward (the page on sequence parallelism for 1M-token training, "How
 * Sequence Parallelism Works"; set beside Ulysses and Ring Attention in its
 * "SP Methods: Head-to-Head Comparison" table).  Every rank holds the
 * contiguous chunk `rank` of a sequence of S = P*C tokens; an all-gather
 * gives every rank all P key/value chunks, and the rank computes exact
 * attention of its own query chunk over the gathered sequence in one pass.
 * On one GPU the all-gather is emulated by 2D device copies of the P chunks
 * into the workspace (gathered [B,H_kv,S,d], chunk j at tokens
 * [j*C, (j+1)*C)); there is no ring walk and no merge.
 *   q: [B,H,C,d] bf16, the rank's queries; k_chunks / v_chunks: HOST arrays
 *   of P device pointers to [B,H_kv,C,d] bf16 (every chunk is gathered, as
 *   the collective would; under causal masking the kernels read only chunks
 *   0..rank).  Causal: local query t sits at global position rank*C + t and
 *   sees keys <= rank*C + t.  o [B,H,C,d], lse [B,H,C] fp32 are overwritten
 *   (same meaning as ra_ring_fwd's).  H_kv must divide H (grouped-query
 *   attention as for the *_gqa calls).  Needs
 *   ra_allgather_workspace_bytes(P,B,H,H_kv,C,d,0) bytes of 16-byte-aligned
 *   workspace (RA_ERR_WORKSPACE); NULL chunk pointers give RA_ERR_NULL.
 *   Other contracts as for ra_ring_fwd.
 *
 * ra_allgather_bwd -- the same share's backward (the softmax-attention
 * gradient with P recomputed from the final lse, as ra_ring_bwd).  o, lse
 * are ra_allgather_fwd's outputs, dO [B,H,C,d] bf16.  dq [B,H,C,d] fp32 and
 * dk, dv [B,H_kv,S,d] fp32 are overwritten: dk, dv hold the gradient of the
 * whole gathered sequence from this rank's queries (zero for keys no local
 * query sees); summing them over ranks and handing each owner its slice is
 * the reduce-scatter a multi-GPU run would do.  Workspace:
 * ra_allgather_workspace_bytes(P,B,H,H_kv,C,d,1) bytes.
 *
 * ra_allgather_workspace_bytes: bwd == 0: gathered K and V,
 * 2 * B*H_kv*P*C*d * 2 bytes; bwd != 0: those and two fp32 values per local
 * query row, + 2 * B*H*C * 4 bytes.  0 for invalid sizes.
 */
size_t ra_allgather_workspace_bytes(int P, int B, int H, int H_kv, int C, int d, int bwd);
int ra_allgather_fwd(const void* q, const void* const* k_chunks,
                     const void* const* v_chunks, int P, float* o, float* lse,
                     int rank, int causal, float scale, int B, int H, int H_kv,
                     int C, int d, void* workspace, size_t workspace_bytes,
                     void* stream);
int ra_allgather_bwd(const void* q, const void* const* k_chunks,
                     const void* const* v_chunks, int P, const float* o,
                     const float* lse, const void* dO, float* dq, float* dk,
                     float* dv, int rank, int causal, float scale, int B,
                     int H, int H_kv, int C, int d, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Per-launch tracing, for profiling.  The pages define no such facility; it
 * exists so that a caller can time each kernel of a ring walk with its own
 * events, on the stream the kernel runs on.
 *
 * ra_trace_begin arms tracing on the calling thread.  Every kernel that
 * ra_step_fwd, ra_lse_merge, ra_ring_fwd, ra_ring_bwd (or their *_gqa
 * forms), ra_ulysses_fwd, ra_ulysses_bwd, ra_allgather_fwd or
 * ra_allgather_bwd then launch on their
 * compute stream is bracketed by hipEventRecord(start_events[n], stream)
 * and hipEventRecord(end_events[n], stream), and kinds[n] receives its
 * RA_TRACE_* kind, for the n-th such launch while n < capacity (later
 * launches run untraced).  The events are hipEvent_t handles (as void*) the
 * caller created with timing enabled and still owns; kinds may be NULL.
 * ra_trace_end disarms tracing and returns the number of launches made while
 * armed (possibly more than capacity).  Staging copies are not traced.
 * ra_trace_begin returns RA_ERR_NULL for missing arrays with capacity > 0
 * and RA_ERR_SHAPE for capacity < 0.
 */
enum ra_trace_kind {
  RA_TRACE_FWD_DIAG = 1,       /* forward, causal-masked (diagonal chunk, or causal offset) */
  RA_TRACE_FWD_FULL = 2,       /* forward step, fully visible chunk */
  RA_TRACE_MERGE = 3,          /* standalone lse merge */
  RA_TRACE_BWD_ROWDOT = 4,     /* backward: D = rowsum(dO * o) */
  RA_TRACE_BWD_ZERO = 5,       /* backward: dq (and dk, dv where overwritten) <- 0 */
  RA_TRACE_BWD_DQ_DIAG = 6,    /* backward dq kernel, causal-masked */
  RA_TRACE_BWD_DQ_FULL = 7,    /* backward dq kernel, full chunk */
  RA_TRACE_BWD_DKDV_DIAG = 8,  /* backward dk/dv kernel, causal-masked */
  RA_TRACE_BWD_DKDV_FULL = 9   /* backward dk/dv kernel, full chunk */
};
int ra_trace_begin(void* const* start_events, void* const* end_events, int* kinds, int capacity);
int ra_trace_end(void);

/*
 * Measurement helpers (no page defines them): what the bf16 matrix cores of
 * the current device can deliver, to set the attention kernels' throughput
 * against.
 *
 * ra_device_info writes the current device's compute-unit count and its
 * maximum engine clock in kHz (hipDeviceGetAttribute).  A CU's four SIMDs
 * each finish one 32x32x16 bf16 MFMA (32768 flop) every 32 cycles, so the
 * dense bf16 peak is cu_count * 4096 flop * clock.  RA_ERR_NULL for NULL
 * outputs, RA_ERR_HIP if the runtime fails.
 *
 * ra_mfma_probe launches `blocks` workgroups of 8 waves, one per CU (each
 * reserves 96 KB of LDS), two waves per SIMD as in the attention kernels.
 * Every wave loads 16 operand registers from `operands` (device, at least
 * 16 * 64 * 16 = 16384 bytes of bf16 data, which sets what the matrix cores
 * multiply: random values draw more power than zeros) and issues
 * iters * 16 back-to-back 32x32x16 bf16 MFMAs into four independent
 * accumulators: 524288 * iters flop per wave.  `sink` (device, blocks * 512
 * floats) receives per-lane sums; `clocks` (device, 2 values) receives the
 * shader-clock cycles (s_memtime) and 100 MHz reference ticks
 * (s_memrealtime) that wave 0 of block 0 spent in its loop, whose ratio is
 * the clock the cores ran at.  Asynchronous on `stream`; RA_ERR_NULL,
 * RA_ERR_SHAPE (blocks or iters < 1), RA_ERR_HIP.
 */
/*
 * ra_fwd_ladder_probe rebuilds the forward step kernel's instruction stream
 * on synthetic data, one feature per level, to account for the distance
 * between ra_mfma_probe's rate and the attention kernel's.  Every level has
 * `blocks` workgroups of 8 waves (one per CU, 128 KB of LDS each, two waves
 * per SIMD) and each wave issues iters * 4 tiles of 32 bf16 32x32x16 MFMAs:
 * 4194304 * iters flop per wave.  Level 0: the dense probe (independent
 * accumulators, register operands); 1: the kernel's accumulator pattern
 * (four P V outputs, two score chains restarting every tile); 2: A operands
 * read from LDS as the kernel reads them (ds_read_b64_tr_b16 pairs and
 * ds_read_b128, three MFMAs ahead); 3: the online softmax of the previous
 * tile's scores in the MFMA slots (scores times c, exp2, row sum, bf16
 * pack into the next P V operand); 4: a workgroup barrier per tile; 5: the
 * tile loads (direct-to-LDS buffer loads two tiles ahead, waited for before
 * the barrier).  Levels 6-10 take the other layout, one wave per SIMD
 * (4 waves per block) holding 64 query rows so that each LDS operand read
 * feeds two MFMAs (output accumulators in AGPRs, scores in VGPRs, P
 * double-buffered): 6: operand reads only (as level 2); 7: everything (as
 * level 5); 8: the softmax only; 9: softmax and barrier; 10: as 7 with the
 * barrier every second tile.  operands: device, >= 20480 bytes of bf16
 * data for the register operands; tiles: device, >= 1 MiB of bf16 data for the LDS
 * tiles and the tile loads.  sink: blocks * 512 floats; clocks: 2 values,
 * as for ra_mfma_probe.  RA_ERR_NULL, RA_ERR_SHAPE (level outside [0, 10],
 * blocks or iters < 1), RA_ERR_HIP.
 */
int ra_fwd_ladder_probe(int level, const void* operands, const void* tiles, float* sink,
                        unsigned long long* clocks, int blocks, int iters, float c, void* stream);
int ra_device_info(int* cu_count, int* max_clock_khz);
int ra_mfma_probe(const void* operands, float* sink, unsigned long long* clocks, int blocks, int iters,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
