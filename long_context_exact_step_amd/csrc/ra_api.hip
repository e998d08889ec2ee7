// C-ABI of the ring-attention library: host-side validation, the ring walk
// (schedule, causal skip, double-buffered staging of KV chunks) and kernel
// dispatch.  See include/ra.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <vector>

#include "ra.h"
#include "ra_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return RA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sizes of one [B, H, S, d] tensor must fit the kernels' 32-bit row indices
// (rows = B*H*S) and size_t byte counts.
int check_dims(int B, int H, int S, int d, const char* what) {
  if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "%s: d=%d (supported: 64, 128)", what, d);
  if (B < 1 || H < 1 || S < 1) return fail(RA_ERR_SHAPE, "%s: B=%d H=%d S=%d must all be >= 1", what, B, H, S);
  const long long rows = (long long)B * H * S;
  if (rows > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "%s: B*H*S=%lld exceeds 2^31-1", what, rows);
  return RA_OK;
}

// Grouped-query heads: H query heads over H_kv key/value heads, H_kv | H.
int check_groups(int H, int H_kv, const char* what) {
  if (H_kv < 1 || H % H_kv)
    return fail(RA_ERR_SHAPE, "%s: H=%d query heads do not split evenly over H_kv=%d key/value heads", what, H, H_kv);
  return RA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// One visible ring step: which chunk, and whether it is the masked diagonal.
struct Step {
  int s, j;
  bool diag;
};

// Step s of rank `rank` uses chunk j = (rank - s) mod P ("Context
// Parallelism", 2 "How It Works"); under causal masking step 0 is the
// diagonal chunk and chunks j > rank are skipped.
std::vector<Step> visible_steps(int rank, int P, bool causal) {
  std::vector<Step> out;
  for (int s = 0; s < P; ++s) {
    const int j = ((rank - s) % P + P) % P;
    if (causal && s > 0 && j > rank) continue;
    out.push_back(Step{s, j, causal && s == 0});
  }
  return out;
}

// Events for ordering slot reuse between the compute and copy streams,
// created once per (thread, device) and reused.
struct RingEvents {
  int device = -1;
  hipEvent_t start = nullptr, copied[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr};
};
thread_local RingEvents t_events;

hipError_t ring_events(RingEvents** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  RingEvents& ev = t_events;
  if (ev.device != dev) {
    hipEvent_t* all[5] = {&ev.start, &ev.copied[0], &ev.copied[1], &ev.consumed[0], &ev.consumed[1]};
    for (hipEvent_t* p : all) {
      if (*p != nullptr && ev.device >= 0) (void)hipEventDestroy(*p);
      *p = nullptr;
      e = hipEventCreateWithFlags(p, hipEventDisableTiming);
      if (e != hipSuccess) {
        ev.device = -1;
        return e;
      }
    }
    ev.device = dev;
  }
  *out = &ev;
  return hipSuccess;
}

// Per-launch tracing state of the calling thread (see ra_trace_begin).
struct Trace {
  void* const* start = nullptr;
  void* const* end = nullptr;
  int* kinds = nullptr;
  int capacity = 0;
  int count = 0;
  bool armed = false;
};
thread_local Trace t_trace;

// Launches one kernel through `launch`, bracketed by the caller's trace
// events when tracing is armed.
template <class F>
hipError_t traced(int kind, hipStream_t stream, F&& launch) {
  Trace& tr = t_trace;
  const bool rec = tr.armed && tr.count < tr.capacity;
  const int n = tr.count;
  if (tr.armed) ++tr.count;
  hipError_t e;
  if (rec) {
    if (tr.kinds) tr.kinds[n] = kind;
    if ((e = hipEventRecord(static_cast<hipEvent_t>(tr.start[n]), stream)) != hipSuccess) return e;
  }
  if ((e = launch()) != hipSuccess) return e;
  if (rec) e = hipEventRecord(static_cast<hipEvent_t>(tr.end[n]), stream);
  return e;
}

// Step 2 of the head-partitioned scheme for one rank: heads rank*Hs ..
// rank*Hs+Hs-1 of every sequence chunk of `chunks` into a [B, Hs, P*C, d] bf16
// buffer.  Within a chunk those heads are one contiguous run of Hs rows of
// C*d values; in the regrouped buffer each head's C tokens land at sequence
// offset j*C.
hipError_t ulysses_regroup(const void* const* chunks, uint8_t* dst0, int P, int rank, int B, int H, int C, int d,
                           hipStream_t s) {
  const int Hs = H / P;
  const size_t S = (size_t)P * C, tok = (size_t)d * 2;
  for (int j = 0; j < P; ++j) {
    for (int b = 0; b < B; ++b) {
      const uint8_t* src = static_cast<const uint8_t*>(chunks[j]) + ((size_t)b * H + (size_t)rank * Hs) * C * tok;
      uint8_t* dst = dst0 + ((size_t)b * Hs * S + (size_t)j * C) * tok;
      const hipError_t e = hipMemcpy2DAsync(dst, S * tok, src, C * tok, C * tok, Hs, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// The all-gather of one tensor, emulated: chunks[j] ([B, Hk, C, d] bf16) to
// its place in the gathered [B, Hk, P*C, d] sequence, one 2D copy per chunk.
hipError_t allgather_copy(const void* const* chunks, uint8_t* dst0, int P, int B, int Hk, int C, int d,
                          hipStream_t s) {
  const size_t S = (size_t)P * C, tok = (size_t)d * 2;
  for (int j = 0; j < P; ++j) {
    const hipError_t e = hipMemcpy2DAsync(dst0 + (size_t)j * C * tok, S * tok, chunks[j], C * tok, C * tok,
                                          (size_t)B * Hk, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Validation shared by the two all-gather entry points.
int allgather_check(const void* const* k_chunks, const void* const* v_chunks, int P, int rank, int B, int H,
                    int H_kv, int C, int d, const char* what) {
  if (P < 1) return fail(RA_ERR_SHAPE, "%s: P=%d < 1", what, P);
  int st = check_dims(B, H, C, d, what);
  if (st) return st;
  st = check_groups(H, H_kv, what);
  if (st) return st;
  if (rank < 0 || rank >= P) return fail(RA_ERR_RANK, "%s: rank=%d outside [0, %d)", what, rank, P);
  if ((long long)B * H_kv * P * C > 0x7fffffffLL || (long long)P * C + 1024 > 0x3fffffffLL)
    return fail(RA_ERR_SHAPE, "%s: gathered sequence B*H_kv*P*C too large", what);
  for (int j = 0; j < P; ++j) {
    if (!k_chunks[j] || !v_chunks[j]) return fail(RA_ERR_NULL, "%s: chunk %d pointer is NULL", what, j);
    if (!aligned16(k_chunks[j]) || !aligned16(v_chunks[j]))
      return fail(RA_ERR_ALIGN, "%s: chunk %d pointer not 16-byte aligned", what, j);
  }
  return RA_OK;
}

// Validation shared by the two head-partitioned entry points.
int ulysses_check(const void* const* const* chunk_sets, int n_sets, int P, int rank, int B, int H, int C, int d,
                  const char* what) {
  if (P < 1) return fail(RA_ERR_SHAPE, "%s: P=%d < 1", what, P);
  int st = check_dims(B, H, C, d, what);
  if (st) return st;
  if (H % P) return fail(RA_ERR_SHAPE, "%s: H=%d heads do not split over P=%d ranks", what, H, P);
  if (rank < 0 || rank >= P) return fail(RA_ERR_RANK, "%s: rank=%d outside [0, %d)", what, rank, P);
  if ((long long)B * (H / P) * P * C > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "%s: B*H/P*P*C exceeds 2^31-1", what);
  for (int x = 0; x < n_sets; ++x)
    for (int j = 0; j < P; ++j) {
      if (!chunk_sets[x][j]) return fail(RA_ERR_NULL, "%s: chunk %d pointer is NULL", what, j);
      if (!aligned16(chunk_sets[x][j])) return fail(RA_ERR_ALIGN, "%s: chunk %d pointer not 16-byte aligned", what, j);
    }
  return RA_OK;
}

hipError_t fwd_step(const ra::FwdStepArgs& a, hipStream_t s) {
  return traced(a.diag ? RA_TRACE_FWD_DIAG : RA_TRACE_FWD_FULL, s, [&] { return ra::launch_fwd_step(a, s); });
}

}  // namespace

extern "C" {

int ra_trace_begin(void* const* start_events, void* const* end_events, int* kinds, int capacity) {
  if (capacity < 0) return fail(RA_ERR_SHAPE, "ra_trace_begin: capacity=%d < 0", capacity);
  if (capacity > 0 && (!start_events || !end_events)) return fail(RA_ERR_NULL, "ra_trace_begin: NULL event array");
  t_trace = Trace{start_events, end_events, kinds, capacity, 0, true};
  return ok();
}

int ra_trace_end(void) {
  const int n = t_trace.count;
  t_trace = Trace{};
  return n;
}

int ra_version(void) { return RA_VERSION; }

const char* ra_status_string(int status) {
  switch (status) {
    case RA_OK: return "RA_OK";
    case RA_ERR_NULL: return "RA_ERR_NULL";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE";
    case RA_ERR_ALIGN: return "RA_ERR_ALIGN";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_RANK: return "RA_ERR_RANK";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    case RA_ERR_HIP: return "RA_ERR_HIP";
    default: return "RA_ERR_UNKNOWN";
  }
}

const char* ra_last_error(void) { return g_err; }

int ra_step_fwd_gqa(const void* q, const void* k, const void* v, float* o_partial, float* lse_partial, int B,
                    int H, int H_kv, int Sq, int Sk, int d, float scale, int step, int causal, void* stream) {
  if (!q || !k || !v || !o_partial || !lse_partial) return fail(RA_ERR_NULL, "ra_step_fwd: NULL pointer");
  int st = check_dims(B, H, Sq, d, "ra_step_fwd(q)");
  if (st) return st;
  st = check_dims(B, H_kv, Sk, d, "ra_step_fwd(k)");
  if (st) return st;
  st = check_groups(H, H_kv, "ra_step_fwd");
  if (st) return st;
  if (step < 0) return fail(RA_ERR_SHAPE, "ra_step_fwd: step=%d < 0", step);
  const bool diag = causal != 0 && step == 0;
  if (diag && Sq != Sk) return fail(RA_ERR_SHAPE, "ra_step_fwd: diagonal step needs Sq == Sk (%d vs %d)", Sq, Sk);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_partial) || !aligned16(lse_partial))
    return fail(RA_ERR_ALIGN, "ra_step_fwd: device pointers must be 16-byte aligned");
  ra::FwdStepArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                    static_cast<const uint16_t*>(v), o_partial, lse_partial, B * H, Sq, Sk, d, scale, diag, false,
                    H / H_kv};
  const hipError_t e = fwd_step(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ra_step_fwd launch");
  return ok();
}

int ra_step_fwd(const void* q, const void* k, const void* v, float* o_partial, float* lse_partial, int B, int H,
                int Sq, int Sk, int d, float scale, int step, int causal, void* stream) {
  return ra_step_fwd_gqa(q, k, v, o_partial, lse_partial, B, H, H, Sq, Sk, d, scale, step, causal, stream);
}

int ra_lse_merge(float* o, float* lse, const float* o_partial, const float* lse_partial, int B, int H, int S, int d,
                 void* stream) {
  if (!o || !lse || !o_partial || !lse_partial) return fail(RA_ERR_NULL, "ra_lse_merge: NULL pointer");
  int st = check_dims(B, H, S, d, "ra_lse_merge");
  if (st) return st;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(o_partial) || !aligned16(lse_partial))
    return fail(RA_ERR_ALIGN, "ra_lse_merge: device pointers must be 16-byte aligned");
  if (o == o_partial || lse == lse_partial) return fail(RA_ERR_SHAPE, "ra_lse_merge: output aliases the partial");
  hipStream_t st_ = static_cast<hipStream_t>(stream);
  const hipError_t e = traced(RA_TRACE_MERGE, st_, [&] {
    return ra::launch_lse_merge(o, lse, o_partial, lse_partial, B * H * S, d, st_);
  });
  if (e != hipSuccess) return hip_fail(e, "ra_lse_merge launch");
  return ok();
}

size_t ra_ring_workspace_bytes_gqa(int P, int B, int H, int H_kv, int C, int d, int ring_mode, int bwd) {
  if (P < 1 || B < 1 || H < 1 || H_kv < 1 || H % H_kv || C < 1 || (d != 64 && d != 128)) return 0;
  const size_t kv_elems = (size_t)B * H_kv * C * d;
  if (bwd) return 2 * (size_t)B * H * C * sizeof(float);  // D and lse2 per query row
  // 2 slots x (K, V) bf16, then two blocks of unit-queue counters.
  if (ring_mode == RA_RING_DOUBLE_BUFFER) return 4 * kv_elems * 2 + 2 * ra::kFwdQueueBytes;
  return 0;
}

size_t ra_ring_workspace_bytes(int P, int B, int H, int C, int d, int ring_mode, int bwd) {
  return ra_ring_workspace_bytes_gqa(P, B, H, H, C, d, ring_mode, bwd);
}

int ra_ring_fwd_gqa(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, float* o,
                    float* lse, int rank, int causal, float scale, int B, int H, int H_kv, int C, int d,
                    int ring_mode, void* workspace, size_t workspace_bytes, void* stream, void* copy_stream) {
  if (!q || !k_chunks || !v_chunks || !o || !lse) return fail(RA_ERR_NULL, "ra_ring_fwd: NULL pointer");
  if (P < 1) return fail(RA_ERR_SHAPE, "ra_ring_fwd: P=%d < 1", P);
  int st = check_dims(B, H, C, d, "ra_ring_fwd");
  if (st) return st;
  st = check_groups(H, H_kv, "ra_ring_fwd");
  if (st) return st;
  if (rank < 0 || rank >= P) return fail(RA_ERR_RANK, "ra_ring_fwd: rank=%d outside [0, %d)", rank, P);
  if (ring_mode != RA_RING_RESIDENT && ring_mode != RA_RING_DOUBLE_BUFFER && ring_mode != RA_RING_FUSED)
    return fail(RA_ERR_UNSUPPORTED, "ra_ring_fwd: ring_mode=%d", ring_mode);
  for (int j = 0; j < P; ++j) {
    if (!k_chunks[j] || !v_chunks[j]) return fail(RA_ERR_NULL, "ra_ring_fwd: chunk %d pointer is NULL", j);
    if (!aligned16(k_chunks[j]) || !aligned16(v_chunks[j]))
      return fail(RA_ERR_ALIGN, "ra_ring_fwd: chunk %d pointer not 16-byte aligned", j);
  }
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse))
    return fail(RA_ERR_ALIGN, "ra_ring_fwd: device pointers must be 16-byte aligned");
  const size_t need = ra_ring_workspace_bytes_gqa(P, B, H, H_kv, C, d, ring_mode, 0);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(RA_ERR_WORKSPACE, "ra_ring_fwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (need > 0 && !aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_ring_fwd: workspace not 16-byte aligned");

  hipStream_t cs = static_cast<hipStream_t>(stream);
  hipStream_t xs = static_cast<hipStream_t>(copy_stream);
  const std::vector<Step> steps = visible_steps(rank, P, causal != 0);
  const size_t chunk_bytes = (size_t)B * H_kv * C * d * 2;
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  auto step_args = [&](const void* kp, const void* vp, bool diag, bool merge) {
    return ra::FwdStepArgs{qh, static_cast<const uint16_t*>(kp), static_cast<const uint16_t*>(vp), o, lse, B * H,
                           C, C, d, scale, diag, merge, H / H_kv};
  };

  if (ring_mode == RA_RING_FUSED && C % 64 == 0 && (int)steps.size() <= ra::kMaxWalkChunks &&
      (long long)steps.size() * C <= 0x3fffffffLL) {
    // One pass over the visible chunks in index order; under causal masking
    // the diagonal chunk comes last and the local queries sit at rank * C.
    ra::ChunkTable t{};
    t.n = 0;
    t.C = C;
    for (int j = 0; j < P; ++j)
      if (!causal || j <= rank) {
        t.k[t.n] = static_cast<const uint16_t*>(k_chunks[j]);
        t.v[t.n] = static_cast<const uint16_t*>(v_chunks[j]);
        ++t.n;
      }
    ra::FwdStepArgs a = step_args(nullptr, nullptr, causal != 0, false);
    a.Sk = t.n * C;
    a.qoff = causal ? rank * C : 0;
    a.walk = &t;
    const hipError_t e = fwd_step(a, cs);
    if (e != hipSuccess) return hip_fail(e, "ra_ring_fwd fused walk");
    return ok();
  }
  if (ring_mode != RA_RING_DOUBLE_BUFFER) {
    for (size_t i = 0; i < steps.size(); ++i) {
      const Step& sp = steps[i];
      const hipError_t e = fwd_step(step_args(k_chunks[sp.j], v_chunks[sp.j], sp.diag, i > 0), cs);
      if (e != hipSuccess) return hip_fail(e, "ra_ring_fwd step launch");
    }
    return ok();
  }

  // Double buffer: step 0 reads the local chunk in place; the chunk of
  // visible step i >= 1 is staged into slot (i-1) & 1 while step i-1 runs.
  // Steps i >= 1 (full chunks) run persistent blocks on the unit queue in
  // counter block i & 1, which step i-1 zeroed (step 0, static, zeroes
  // block 1), so the counters need no launch of their own.
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto slot_k = [&](int slot) { return ws + (size_t)slot * 2 * chunk_bytes; };
  auto slot_v = [&](int slot) { return ws + (size_t)slot * 2 * chunk_bytes + chunk_bytes; };
  int* queues = reinterpret_cast<int*>(ws + 4 * chunk_bytes);
  const int n = (int)steps.size();
  auto with_queues = [&](ra::FwdStepArgs a, int i) {
    if (i > 0) a.queue = queues + (i & 1) * ra::kFwdQueueInts;
    if (i + 1 < n) a.queue_next = queues + ((i + 1) & 1) * ra::kFwdQueueInts;
    return a;
  };
  hipError_t e = hipSuccess;
  if (!copy_stream) {
    // No copy stream: step i's kernel itself copies the chunk of step i+1
    // into slot i & 1 once its blocks have done their own work.  That slot
    // was last read by step i-1's kernel and is next read by step i+1's,
    // both ordered by the stream, so no copy or event goes elsewhere.
    for (int i = 0; i < n; ++i) {
      const Step& sp = steps[i];
      ra::StageCopy sc{};
      if (i + 1 < n) {
        const int j = steps[i + 1].j;
        sc = ra::StageCopy{{k_chunks[j], v_chunks[j]}, {slot_k(i & 1), slot_v(i & 1)}, chunk_bytes / 16};
      }
      ra::FwdStepArgs a = with_queues(i == 0 ? step_args(k_chunks[sp.j], v_chunks[sp.j], sp.diag, false)
                                             : step_args(slot_k((i - 1) & 1), slot_v((i - 1) & 1), sp.diag, true),
                                      i);
      if (i + 1 < n) a.stage = &sc;
      if ((e = fwd_step(a, cs)) != hipSuccess) return hip_fail(e, "ra_ring_fwd step");
    }
    return ok();
  }

  // Copy stream: the staging copies run there, ordered by events.
  RingEvents* ev = nullptr;
  if ((e = ring_events(&ev)) != hipSuccess) return hip_fail(e, "ra_ring_fwd events");
  // Copies may start only after everything already queued on the compute
  // stream (the inputs, and any earlier user of the workspace).
  if ((e = hipEventRecord(ev->start, cs)) != hipSuccess) return hip_fail(e, "ra_ring_fwd record");
  if ((e = hipStreamWaitEvent(xs, ev->start, 0)) != hipSuccess) return hip_fail(e, "ra_ring_fwd wait");
  for (int i = 0; i < n; ++i) {
    // Stage the chunk for step i+1 (slot i & 1); that slot was last read by
    // step i-1 (step 0 reads the local chunk in place), so from i = 2 on the
    // copy waits for that step.
    if (i + 1 < n) {
      const int slot = i & 1;
      const int j = steps[i + 1].j;
      if (i >= 2 && (e = hipStreamWaitEvent(xs, ev->consumed[slot], 0)) != hipSuccess)
        return hip_fail(e, "ra_ring_fwd wait");
      if ((e = hipMemcpyAsync(slot_k(slot), k_chunks[j], chunk_bytes, hipMemcpyDeviceToDevice, xs)) != hipSuccess)
        return hip_fail(e, "ra_ring_fwd stage K");
      if ((e = hipMemcpyAsync(slot_v(slot), v_chunks[j], chunk_bytes, hipMemcpyDeviceToDevice, xs)) != hipSuccess)
        return hip_fail(e, "ra_ring_fwd stage V");
      if ((e = hipEventRecord(ev->copied[slot], xs)) != hipSuccess) return hip_fail(e, "ra_ring_fwd record");
    }
    const Step& sp = steps[i];
    if (i == 0) {
      e = fwd_step(with_queues(step_args(k_chunks[sp.j], v_chunks[sp.j], sp.diag, false), i), cs);
    } else {
      const int slot = (i - 1) & 1;
      if ((e = hipStreamWaitEvent(cs, ev->copied[slot], 0)) != hipSuccess) return hip_fail(e, "ra_ring_fwd wait");
      e = fwd_step(with_queues(step_args(slot_k(slot), slot_v(slot), sp.diag, true), i), cs);
      if (e == hipSuccess) e = hipEventRecord(ev->consumed[slot], cs);
    }
    if (e != hipSuccess) return hip_fail(e, "ra_ring_fwd step");
  }
  return ok();
}

int ra_ring_fwd(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, float* o, float* lse,
                int rank, int causal, float scale, int B, int H, int C, int d, int ring_mode, void* workspace,
                size_t workspace_bytes, void* stream, void* copy_stream) {
  return ra_ring_fwd_gqa(q, k_chunks, v_chunks, P, o, lse, rank, causal, scale, B, H, H, C, d, ring_mode, workspace,
                         workspace_bytes, stream, copy_stream);
}

}  // extern "C"

namespace {

// Argument checks of the backward walk, other than its workspace.
int ring_bwd_check(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, const float* o,
                   const float* lse, const void* dO, float* dq, float* const* dk_chunks, float* const* dv_chunks,
                   int rank, int causal, int B, int H, int H_kv, int C, int d, const char* what) {
  if (!q || !k_chunks || !v_chunks || !o || !lse || !dO || !dq || !dk_chunks || !dv_chunks)
    return fail(RA_ERR_NULL, "%s: NULL pointer", what);
  if (P < 1) return fail(RA_ERR_SHAPE, "%s: P=%d < 1", what, P);
  int st = check_dims(B, H, C, d, what);
  if (st) return st;
  st = check_groups(H, H_kv, what);
  if (st) return st;
  if (rank < 0 || rank >= P) return fail(RA_ERR_RANK, "%s: rank=%d outside [0, %d)", what, rank, P);
  for (const Step& sp : visible_steps(rank, P, causal != 0)) {
    const int j = sp.j;
    if (!k_chunks[j] || !v_chunks[j] || !dk_chunks[j] || !dv_chunks[j])
      return fail(RA_ERR_NULL, "%s: chunk %d pointer is NULL", what, j);
    if (!aligned16(k_chunks[j]) || !aligned16(v_chunks[j]) || !aligned16(dk_chunks[j]) || !aligned16(dv_chunks[j]))
      return fail(RA_ERR_ALIGN, "%s: chunk %d pointer not 16-byte aligned", what, j);
  }
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || !aligned16(dO) || !aligned16(dq))
    return fail(RA_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", what);
  return RA_OK;
}

// The backward walk on validated arguments; Dbuf holds 2 * B*H*C floats (D,
// then lse in base 2), both written by the row pre-pass before any use.
int ring_bwd_run(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, const float* o,
                 const float* lse, const void* dO, float* dq, float* const* dk_chunks, float* const* dv_chunks,
                 int rank, int causal, float scale, int B, int H, int H_kv, int C, int d, float* Dbuf,
                 hipStream_t cs, const char* what) {
  const int rows = B * H * C;
  float* lse2 = Dbuf + rows;
  hipError_t e = traced(RA_TRACE_BWD_ROWDOT, cs, [&] {
    return ra::launch_bwd_rowdot(static_cast<const uint16_t*>(dO), o, lse, Dbuf, lse2, rows, d, cs);
  });
  if (e == hipSuccess) e = traced(RA_TRACE_BWD_ZERO, cs, [&] { return ra::launch_zero_f32(dq, (size_t)rows * d, cs); });
  if (e != hipSuccess) return hip_fail(e, what);
  for (const Step& sp : visible_steps(rank, P, causal != 0)) {
    ra::BwdStepArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_chunks[sp.j]),
                      static_cast<const uint16_t*>(v_chunks[sp.j]), static_cast<const uint16_t*>(dO), lse2, Dbuf, dq,
                      dk_chunks[sp.j], dv_chunks[sp.j], B * H, C, C, d, scale, sp.diag, H / H_kv};
    e = traced(sp.diag ? RA_TRACE_BWD_DQ_DIAG : RA_TRACE_BWD_DQ_FULL, cs, [&] { return ra::launch_bwd_dq(a, cs); });
    if (e == hipSuccess)
      e = traced(sp.diag ? RA_TRACE_BWD_DKDV_DIAG : RA_TRACE_BWD_DKDV_FULL, cs,
                 [&] { return ra::launch_bwd_dkdv(a, cs); });
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return ok();
}

}  // namespace

// Device scratch of ra_ring_bwd_noalloc: D and lse2 (two floats) for up to
// RA_NOALLOC_MAX_ROWS query rows, 16 MiB.  Each device that runs the library
// holds its own copy until the process ends.  In host code this name is a
// host-side stand-in, not a device address: kernels and copies get the
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[2 * (size_t)RA_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per
// device (with that device current) and kept.
int scratch_on_device(float** out, const char* what) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, what);
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_HIP, "%s: device %d beyond the %d supported", what, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, what);
    if (!p) return fail(RA_ERR_HIP, "%s: scratch address lookup returned NULL", what);
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

int ra_ring_bwd_gqa(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, const float* o,
                    const float* lse, const void* dO, float* dq, float* const* dk_chunks, float* const* dv_chunks,
                    int rank, int causal, float scale, int B, int H, int H_kv, int C, int d, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = ring_bwd_check(q, k_chunks, v_chunks, P, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, B, H, H_kv, C,
                          d, "ra_ring_bwd");
  if (st) return st;
  const size_t need = ra_ring_workspace_bytes_gqa(P, B, H, H_kv, C, d, 0, 1);
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "ra_ring_bwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (!aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_ring_bwd: workspace not 16-byte aligned");
  return ring_bwd_run(q, k_chunks, v_chunks, P, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, scale, B, H, H_kv,
                      C, d, static_cast<float*>(workspace), static_cast<hipStream_t>(stream), "ra_ring_bwd");
}

int ra_ring_bwd_noalloc(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P,
                        const float* o, const float* lse, const void* dO, float* dq, float* const* dk_chunks,
                        float* const* dv_chunks, int rank, int causal, float scale, int B, int H, int H_kv, int C,
                        int d, void* stream) {
  int st = ring_bwd_check(q, k_chunks, v_chunks, P, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, B, H, H_kv, C,
                          d, "ra_ring_bwd_noalloc");
  if (st) return st;
  const long long rows = (long long)B * H * C;
  if (rows > RA_NOALLOC_MAX_ROWS)
    return fail(RA_ERR_WORKSPACE, "ra_ring_bwd_noalloc: B*H*C=%lld query rows exceed the static scratch's %d",
                rows, RA_NOALLOC_MAX_ROWS);
  float* sp = nullptr;
  st = scratch_on_device(&sp, "ra_ring_bwd_noalloc");
  if (st) return st;
  return ring_bwd_run(q, k_chunks, v_chunks, P, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, scale, B, H, H_kv,
                      C, d, sp, static_cast<hipStream_t>(stream), "ra_ring_bwd_noalloc");
}

int ra_ring_bwd(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, const float* o,
                const float* lse, const void* dO, float* dq, float* const* dk_chunks, float* const* dv_chunks,
                int rank, int causal, float scale, int B, int H, int C, int d, void* workspace,
                size_t workspace_bytes, void* stream) {
  return ra_ring_bwd_gqa(q, k_chunks, v_chunks, P, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, scale, B, H,
                         H, C, d, workspace, workspace_bytes, stream);
}

size_t ra_ulysses_workspace_bytes(int P, int B, int H, int C, int d, int bwd) {
  if (P < 1 || B < 1 || H < 1 || H % P || C < 1 || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * (H / P) * ((size_t)P * C);
  if (bwd) return 4 * rows * d * 2 + 2 * rows * sizeof(float);  // regrouped Q, K, V, dO; D and lse2 per row
  return 3 * rows * d * 2;                                        // regrouped Q, K, V (bf16)
}


int ra_ulysses_fwd(const void* const* q_chunks, const void* const* k_chunks, const void* const* v_chunks, int P,
                   float* o, float* lse, int rank, int causal, float scale, int B, int H, int C, int d,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_chunks || !k_chunks || !v_chunks || !o || !lse) return fail(RA_ERR_NULL, "ra_ulysses_fwd: NULL pointer");
  const void* const* sets[3] = {q_chunks, k_chunks, v_chunks};
  int st = ulysses_check(sets, 3, P, rank, B, H, C, d, "ra_ulysses_fwd");
  if (st) return st;
  if (!aligned16(o) || !aligned16(lse)) return fail(RA_ERR_ALIGN, "ra_ulysses_fwd: outputs not 16-byte aligned");
  const size_t need = ra_ulysses_workspace_bytes(P, B, H, C, d, 0);
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "ra_ulysses_fwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (!aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_ulysses_fwd: workspace not 16-byte aligned");

  hipStream_t cs = static_cast<hipStream_t>(stream);
  const int Hs = H / P, S = P * C;
  const size_t part = (size_t)B * Hs * S * d * 2;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int x = 0; x < 3; ++x) {
    const hipError_t e = ulysses_regroup(sets[x], ws + x * part, P, rank, B, H, C, d, cs);
    if (e != hipSuccess) return hip_fail(e, "ra_ulysses_fwd regroup");
  }
  // Step 3: full attention of the regrouped heads over the whole sequence
  // (the causal mask over global positions is the diagonal mask at S).
  const ra::FwdStepArgs a{reinterpret_cast<const uint16_t*>(ws), reinterpret_cast<const uint16_t*>(ws + part),
                          reinterpret_cast<const uint16_t*>(ws + 2 * part), o, lse, B * Hs, S, S, d, scale,
                          causal != 0, false, 1};
  const hipError_t e = fwd_step(a, cs);
  if (e != hipSuccess) return hip_fail(e, "ra_ulysses_fwd attention");
  return ok();
}

int ra_ulysses_bwd(const void* const* q_chunks, const void* const* k_chunks, const void* const* v_chunks,
                   const void* const* dO_chunks, int P, const float* o, const float* lse, float* dq, float* dk,
                   float* dv, int rank, int causal, float scale, int B, int H, int C, int d, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!q_chunks || !k_chunks || !v_chunks || !dO_chunks || !o || !lse || !dq || !dk || !dv)
    return fail(RA_ERR_NULL, "ra_ulysses_bwd: NULL pointer");
  const void* const* sets[4] = {q_chunks, k_chunks, v_chunks, dO_chunks};
  int st = ulysses_check(sets, 4, P, rank, B, H, C, d, "ra_ulysses_bwd");
  if (st) return st;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(RA_ERR_ALIGN, "ra_ulysses_bwd: device pointers must be 16-byte aligned");
  const size_t need = ra_ulysses_workspace_bytes(P, B, H, C, d, 1);
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "ra_ulysses_bwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (!aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_ulysses_bwd: workspace not 16-byte aligned");

  hipStream_t cs = static_cast<hipStream_t>(stream);
  const int Hs = H / P, S = P * C;
  const int rows = B * Hs * S;
  const size_t part = (size_t)rows * d * 2;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int x = 0; x < 4; ++x) {
    const hipError_t e = ulysses_regroup(sets[x], ws + x * part, P, rank, B, H, C, d, cs);
    if (e != hipSuccess) return hip_fail(e, "ra_ulysses_bwd regroup");
  }
  const uint16_t* qr = reinterpret_cast<const uint16_t*>(ws);
  const uint16_t* dOr = reinterpret_cast<const uint16_t*>(ws + 3 * part);
  float* Dbuf = reinterpret_cast<float*>(ws + 4 * part);
  float* lse2 = Dbuf + rows;
  hipError_t e = traced(RA_TRACE_BWD_ROWDOT, cs, [&] { return ra::launch_bwd_rowdot(dOr, o, lse, Dbuf, lse2, rows, d, cs); });
  for (float* g : {dq, dk, dv})
    if (e == hipSuccess) e = traced(RA_TRACE_BWD_ZERO, cs, [&] { return ra::launch_zero_f32(g, (size_t)rows * d, cs); });
  if (e != hipSuccess) return hip_fail(e, "ra_ulysses_bwd preprocess");
  // The whole sequence is one step: the diagonal (causal) or a full chunk.
  const ra::BwdStepArgs a{qr, reinterpret_cast<const uint16_t*>(ws + part),
                          reinterpret_cast<const uint16_t*>(ws + 2 * part), dOr, lse2, Dbuf, dq, dk, dv,
                          B * Hs, S, S, d, scale, causal != 0, 1};
  e = traced(causal ? RA_TRACE_BWD_DQ_DIAG : RA_TRACE_BWD_DQ_FULL, cs, [&] { return ra::launch_bwd_dq(a, cs); });
  if (e == hipSuccess)
    e = traced(causal ? RA_TRACE_BWD_DKDV_DIAG : RA_TRACE_BWD_DKDV_FULL, cs, [&] { return ra::launch_bwd_dkdv(a, cs); });
  if (e != hipSuccess) return hip_fail(e, "ra_ulysses_bwd step");
  return ok();
}

size_t ra_allgather_workspace_bytes(int P, int B, int H, int H_kv, int C, int d, int bwd) {
  if (P < 1 || B < 1 || H < 1 || H_kv < 1 || H % H_kv || C < 1 || (d != 64 && d != 128)) return 0;
  const size_t kv = 2 * (size_t)B * H_kv * ((size_t)P * C) * d * 2;  // gathered K and V (bf16)
  if (bwd) return kv + 2 * (size_t)B * H * C * sizeof(float);       // and D, lse2 per local row
  return kv;
}

int ra_allgather_fwd(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, float* o,
                     float* lse, int rank, int causal, float scale, int B, int H, int H_kv, int C, int d,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_chunks || !v_chunks || !o || !lse) return fail(RA_ERR_NULL, "ra_allgather_fwd: NULL pointer");
  int st = allgather_check(k_chunks, v_chunks, P, rank, B, H, H_kv, C, d, "ra_allgather_fwd");
  if (st) return st;
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse))
    return fail(RA_ERR_ALIGN, "ra_allgather_fwd: device pointers must be 16-byte aligned");
  const size_t need = ra_allgather_workspace_bytes(P, B, H, H_kv, C, d, 0);
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "ra_allgather_fwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (!aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_allgather_fwd: workspace not 16-byte aligned");

  hipStream_t cs = static_cast<hipStream_t>(stream);
  const int S = P * C;
  const size_t part = (size_t)B * H_kv * S * d * 2;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e = allgather_copy(k_chunks, ws, P, B, H_kv, C, d, cs);
  if (e == hipSuccess) e = allgather_copy(v_chunks, ws + part, P, B, H_kv, C, d, cs);
  if (e != hipSuccess) return hip_fail(e, "ra_allgather_fwd gather");
  // One pass of the local queries over the gathered sequence; causal: query
  // t sits at global position rank*C + t.
  ra::FwdStepArgs a{static_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(ws),
                    reinterpret_cast<const uint16_t*>(ws + part), o, lse, B * H, C, S, d, scale, causal != 0, false,
                    H / H_kv, causal ? rank * C : 0};
  e = fwd_step(a, cs);
  if (e != hipSuccess) return hip_fail(e, "ra_allgather_fwd attention");
  return ok();
}

int ra_allgather_bwd(const void* q, const void* const* k_chunks, const void* const* v_chunks, int P, const float* o,
                     const float* lse, const void* dO, float* dq, float* dk, float* dv, int rank, int causal,
                     float scale, int B, int H, int H_kv, int C, int d, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!q || !k_chunks || !v_chunks || !o || !lse || !dO || !dq || !dk || !dv)
    return fail(RA_ERR_NULL, "ra_allgather_bwd: NULL pointer");
  int st = allgather_check(k_chunks, v_chunks, P, rank, B, H, H_kv, C, d, "ra_allgather_bwd");
  if (st) return st;
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return fail(RA_ERR_ALIGN, "ra_allgather_bwd: device pointers must be 16-byte aligned");
  const size_t need = ra_allgather_workspace_bytes(P, B, H, H_kv, C, d, 1);
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "ra_allgather_bwd: workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                need);
  if (!aligned16(workspace)) return fail(RA_ERR_ALIGN, "ra_allgather_bwd: workspace not 16-byte aligned");

  hipStream_t cs = static_cast<hipStream_t>(stream);
  const int S = P * C, rows = B * H * C;
  const size_t part = (size_t)B * H_kv * S * d * 2;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* Dbuf = reinterpret_cast<float*>(ws + 2 * part);
  float* lse2 = Dbuf + rows;
  hipError_t e = allgather_copy(k_chunks, ws, P, B, H_kv, C, d, cs);
  if (e == hipSuccess) e = allgather_copy(v_chunks, ws + part, P, B, H_kv, C, d, cs);
  if (e != hipSuccess) return hip_fail(e, "ra_allgather_bwd gather");
  e = traced(RA_TRACE_BWD_ROWDOT, cs, [&] {
    return ra::launch_bwd_rowdot(static_cast<const uint16_t*>(dO), o, lse, Dbuf, lse2, rows, d, cs);
  });
  if (e == hipSuccess) e = traced(RA_TRACE_BWD_ZERO, cs, [&] { return ra::launch_zero_f32(dq, (size_t)rows * d, cs); });
  for (float* g : {dk, dv})
    if (e == hipSuccess)
      e = traced(RA_TRACE_BWD_ZERO, cs, [&] { return ra::launch_zero_f32(g, (size_t)B * H_kv * S * d, cs); });
  if (e != hipSuccess) return hip_fail(e, "ra_allgather_bwd preprocess");
  const ra::BwdStepArgs a{static_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(ws),
                          reinterpret_cast<const uint16_t*>(ws + part), static_cast<const uint16_t*>(dO), lse2, Dbuf,
                          dq, dk, dv, B * H, C, S, d, scale, causal != 0, H / H_kv, causal ? rank * C : 0};
  e = traced(causal ? RA_TRACE_BWD_DQ_DIAG : RA_TRACE_BWD_DQ_FULL, cs, [&] { return ra::launch_bwd_dq(a, cs); });
  if (e == hipSuccess)
    e = traced(causal ? RA_TRACE_BWD_DKDV_DIAG : RA_TRACE_BWD_DKDV_FULL, cs, [&] { return ra::launch_bwd_dkdv(a, cs); });
  if (e != hipSuccess) return hip_fail(e, "ra_allgather_bwd step");
  return ok();
}

}  // extern "C"
