// Host-visible launch interface of the ring-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// One ring step, forward: query block [BH, Sq, d] against one KV chunk
// [BH / group, Sk, d] (bf16), written into (o, lse) fp32 -- overwritten when
// merge == false, folded into the running values when merge == true.  Query
// head row bh reads key/value head bh / group (grouped-query attention with
// `group` query heads per key/value head; 1 = multi-head).
// Resident key/value chunks walked by one launch, in order: chunk c holds
// keys [c*C, (c+1)*C) of the walked sequence; C is a multiple of 64.
constexpr int kMaxWalkChunks = 16;
struct ChunkTable {
  const uint16_t* k[kMaxWalkChunks];
  const uint16_t* v[kMaxWalkChunks];
  int n;  // chunks walked (1 .. kMaxWalkChunks)
  int C;  // tokens per chunk
};

// In-kernel staging of the ring's next key/value chunk: after its own work,
// every block of a step launch copies its share of `units` 16-byte units of
// each of the two tensors from src[t] to dst[t] (the idle slot of the double
// buffer).  units == 0: no copy.
struct StageCopy {
  const void* src[2];
  void* dst[2];
  size_t units;
};

// Unit counters of a persistent step launch: one per XCD, 64 bytes apart.
constexpr int kFwdQueueInts = 128;
constexpr size_t kFwdQueueBytes = kFwdQueueInts * sizeof(int);

struct FwdStepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;
  int BH, Sq, Sk, d;
  float scale;
  bool diag;   // causal mask: query t sees keys <= t + qoff
  bool merge;  // fold into the running (o, lse) instead of overwriting
  int group;   // query heads per key/value head (>= 1, divides BH)
  int qoff = 0;  // causal offset of the query rows against the keys (>= 0; 0 on the ring's diagonal chunk)
  // Non-null: the keys are walk->n resident chunks (k, v unused; Sk =
  // n * C; merge must be false).
  const ChunkTable* walk = nullptr;
  // Non-null: stage the next chunk from inside this launch (step kernels only).
  const StageCopy* stage = nullptr;
  // Non-null (full-chunk steps): kFwdQueueInts zeroed counters this launch
  // owns while it runs.  With at least four (head, query tile) units per
  // compute unit, the launch then runs one persistent block per compute
  // unit; a block takes units from its XCD's
  // queue, the same units in the same order as the static mapping, and once
  // that queue is empty from the other XCDs' queues, so that faster XCDs
  // take more units.  Null: one block per unit, statically mapped.
  int* queue = nullptr;
  // Non-null: kFwdQueueInts counters the launch sets to zero for the next
  // launch on the stream (which cannot start before this one ends).
  int* queue_next = nullptr;
};
hipError_t launch_fwd_step(const FwdStepArgs& a, hipStream_t stream);

// Row-wise online-softmax merge of a partial into (o, lse), in place.
hipError_t launch_lse_merge(float* o, float* lse, const float* op, const float* lp,
                            int rows, int d, hipStream_t stream);

// Backward: D = rowsum(dO * O) per row, and lse2 = lse * log2(e) per row
// (+inf where lse is -inf).
hipError_t launch_bwd_rowdot(const uint16_t* dO, const float* o, const float* lse, float* D, float* lse2,
                             int rows, int d, hipStream_t stream);

// Backward of one ring step against one KV chunk.  Uses the final lse (in
// base 2) and D.  Query head row bh reads key/value head bh / group; dk, dv
// ([BH / group, Sk, d]) sum over the group's query heads.
struct BwdStepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  const float* lse2;  // final lse * log2(e) per row, +inf for a row that saw no key
  const float* D;
  float* dq;   // accumulated (+=)
  float* dk;   // accumulated (+=)
  float* dv;   // accumulated (+=)
  int BH, Sq, Sk, d;
  float scale;
  bool diag;  // causal mask: query t sees keys <= t + qoff
  int group;  // query heads per key/value head (>= 1, divides BH)
  int qoff = 0;  // causal offset of the query rows against the keys (>= 0)
};
hipError_t launch_bwd_dq(const BwdStepArgs& a, hipStream_t stream);    // dq += ...
hipError_t launch_bwd_dkdv(const BwdStepArgs& a, hipStream_t stream);  // dk, dv += ...

// dq <- 0 over n floats (a small fill kernel, safe under graph capture).
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream);

}  // namespace ra
