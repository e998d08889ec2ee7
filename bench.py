#!/usr/bin/env python3
"""Benchmark of one GPU's share of Ring Attention on one MI355X.

Default workload: the 128K-token sequence at CP=4, local share of rank 3
(C = 32768 query tokens, P = 4 KV chunks of 32768, H = 32, d = 128, causal),
forward ring walk in double-buffer mode.  One step = one ra_ring_fwd call:
the ring schedule, the staged (emulated) KV receives, one fused step kernel
per visible chunk with the log-sum-exp merge in its epilogue.  Inputs are
seeded synthetic bf16 N(0,1) tensors resident in HBM before timing starts.

Also reported (unless --no-train): the training share (C = 16384, P = 4,
rank 3, H = 32, d = 128, causal), one step = forward walk + backward walk.
And (unless --no-gqa): both walks again with grouped-query key/value chunks of
H/4 heads (4 query heads per key/value head), under "gqa".  And (unless
--no-ulysses): one rank's share of head-partitioned (Ulysses) sequence
parallelism on the same sequence, under "ulysses".  And (unless
--no-allgather): the same rank's share of all-gather sequence parallelism
(gathered key/value chunks, one pass at a causal offset), forward and
training step, under "allgather".  And (unless --no-ceiling): the bf16 peak
derived from the device's CU count and clock, what a dense MFMA probe
sustains on random and on zero operands, and one full-chunk step kernel on
the workload's random inputs and on zeros, under "mfma_ceiling".

Prints ONE JSON line: throughput in algorithmic TFLOP/s (4*d flops per
visible (query, key) pair forward, 10*d backward), tokens/s, the roofline of
the dominant kernel timed live with HIP events on its own stream, and the
fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--no-train] [--no-cpu] [--no-gqa]
"""

import argparse
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring-attention fwd/bwd TFLOP/s and tokens/s on 1 MI355X (% of bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak (the roofline's peak)
# 256 CUs x 4096 flop per CU per clock x 2.4 GHz: the same peak derived from
# the chip's unit counts and clock, reported beside the published figure.
DERIVED_PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "fwd_full_step_128k_cp4_counters.json")
FWD_KERNEL_SOURCES = ["long_context_exact_step_amd/csrc/ra_fwd.hip", "long_context_exact_step_amd/csrc/ra_device.h"]


def fwd_kernel_sha():
    h = hashlib.sha256()
    for p in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# The full-chunk merge step of the 128K share's double-buffer walk, on
# persistent blocks (the step kernel of the static schedule is
# fwd_step_kernel<128, false, true>).
COUNTER_KERNEL = "fwd_queue_kernel<128, true>"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def ingest_counters(fetch_dir, write_dir, cmd_fetch, cmd_write, out_path=PROFILE_COUNTERS):
    """Turn two rocprofv3 counter passes over the default forward walk (one
    with FETCH_SIZE, one with WRITE_SIZE, in KiB per dispatch) into the HBM
    bytes per full-chunk launch that `roofline.traffic` reports.  Each counter
    is scaled by what it reads for the 256 MiB key/value staging copies of the
    same run (a plain copy of known size), then stamped with the forward
    kernel's source hash so that a later change to the kernel voids it."""
    import csv
    import glob
    from long_context_exact_step_amd.workloads import WORKLOADS

    def values(d, counter):
        out = {"kernel": [], "copy": []}
        paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for path in paths:
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") != counter:
                        continue
                    name = r.get("Kernel_Name", "")
                    if COUNTER_KERNEL in name:
                        out["kernel"].append(float(r["Counter_Value"]))
                    elif COPY_KERNEL in name:
                        out["copy"].append(float(r["Counter_Value"]))
        if not out["kernel"] or not out["copy"]:
            raise SystemExit(f"{d}: no {counter} rows for {COUNTER_KERNEL} and the staging copies")
        return out

    w = WORKLOADS[2]
    chunk_kib = w.B * w.H * w.C * w.d * 2 / 1024  # one K or V chunk, bf16
    mean = lambda v: sum(v) / len(v)
    # The largest copies of the run are the chunk staging copies.
    big = lambda v: [x for x in v if x >= 0.95 * max(v)]
    fe, wr = values(fetch_dir, "FETCH_SIZE"), values(write_dir, "WRITE_SIZE")
    ff, wf = chunk_kib / mean(big(fe["copy"])), chunk_kib / mean(big(wr["copy"]))
    fetch_b = mean(fe["kernel"]) * ff * 1024
    write_b = mean(wr["kernel"]) * wf * 1024
    rec = {
        "kernel": COUNTER_KERNEL, "workload_id": w.id,
        "workload": w.name + " (full-chunk merge step)", "source_sha": fwd_kernel_sha(),
        "dispatches": {"fetch": len(fe["kernel"]), "write": len(wr["kernel"])},
        "fetch_kib_per_dispatch_raw": mean(fe["kernel"]), "write_kib_per_dispatch_raw": mean(wr["kernel"]),
        "copy_calibration": {"kernel": COPY_KERNEL + " (256 MiB chunk staging copy, same runs)",
                             "fetch_kib_raw": mean(big(fe["copy"])), "write_kib_raw": mean(big(wr["copy"])),
                             "fetch_factor": ff, "write_factor": wf},
        "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "command_fetch": cmd_fetch, "command_write": cmd_write,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))
    return rec


class HipEvents:
    """Timing-enabled hipEvent_t handles made through the HIP runtime."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.start, self.end = [], []
        for lst in (self.start, self.end):
            for _ in range(n):
                e = ctypes.c_void_p()
                rc = self.hip.hipEventCreate(ctypes.byref(e))
                if rc != 0:
                    raise RuntimeError(f"hipEventCreate failed ({rc})")
                lst.append(e.value)

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.end[i])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for e in self.start + self.end:
            self.hip.hipEventDestroy(e)


def pairs_of_kind(kind, w):
    """Visible (query, key) pairs one traced launch processes."""
    C, BH = w.C, w.B * w.H
    if kind in ("fwd_diag", "bwd_dq_diag", "bwd_dkdv_diag"):
        return BH * C * (C + 1) // 2
    if kind in ("fwd_full", "bwd_dq_full", "bwd_dkdv_full"):
        return BH * C * C
    return 0


class StepClock:
    """Events on the current stream at every step boundary of the timed loop
    (recorded between steps, with no synchronisation): the per-step times
    whose median the bench lines report beside the mean."""

    def __init__(self, steps):
        import torch
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        self.n = 0

    def mark(self):
        self.ev[self.n].record()
        self.n += 1

    def median_ms(self):
        d = sorted(self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(self.n - 1))
        if not d:
            return None
        m = len(d) // 2
        return d[m] if len(d) % 2 else 0.5 * (d[m - 1] + d[m])


class ClockSampler:
    """The GPU's current engine clock as its driver reports it (the level
    marked '*' in pp_dpm_sclk), read by a thread every `period` seconds
    between start() and stop(): the clock the timed steps ran at, for the
    fraction of the peak at that clock.  The file is that of cuda:0's PCI
    device (or the only one present); samples stay empty where it cannot be
    read."""

    def __init__(self, period=0.01):
        import glob
        import threading
        import torch
        self.path = None
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        try:
            p = torch.cuda.get_device_properties(0)
            bus = "%04x:%02x:%02x" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
            mine = [x for x in paths if os.path.basename(os.path.realpath(os.path.dirname(x))).startswith(bus)]
        except (AttributeError, RuntimeError, AssertionError):
            mine = []
        if len(mine) == 1:
            self.path = mine[0]
        elif len(paths) == 1:
            self.path = paths[0]
        self.period, self.samples = period, []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def parse(text):
        """MHz of the level marked '*' in pp_dpm_sclk text ("1: 1650Mhz *"), or None."""
        for line in text.splitlines():
            line = line.strip()
            if line.endswith("*"):
                try:
                    return float(line.split(":")[1].rstrip("*").strip().lower().rstrip("mhz"))
                except (IndexError, ValueError):
                    return None
        return None

    def _read(self):
        try:
            with open(self.path) as f:
                return self.parse(f.read())
        except OSError:
            return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def start(self):
        if self.path:
            self._thread.start()

    def stop(self):
        if self.path:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"mean_mhz": round(sum(v) / len(v), 1), "median_mhz": v[len(v) // 2], "min_mhz": v[0],
                "max_mhz": v[-1], "samples": len(v), "source": self.path}


def timed_steps(step_fn, n_launch_per_step, steps, warmup, clock=None, sampler=None):
    """Runs warmup, then exactly `steps` timed steps with per-launch tracing
    (and step-boundary events into `clock`, the engine clock into `sampler`,
    if given).  Returns (seconds, [(kind, ms), ...])."""
    import torch
    import long_context_exact_step_amd as ra

    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    cap = steps * n_launch_per_step
    ev = HipEvents(cap)
    kinds = (ctypes.c_int * cap)()
    keep = ra.trace_begin(ev.start, ev.end, kinds)
    torch.cuda.synchronize()
    if sampler:
        sampler.start()
    t0 = time.perf_counter()
    if clock:
        clock.mark()
    for _ in range(steps):
        step_fn()
        if clock:
            clock.mark()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if sampler:
        sampler.stop()
    n = ra.trace_end()
    del keep
    rec = [(ra.TRACE_KINDS[kinds[i]], ev.elapsed_ms(i)) for i in range(min(n, cap))]
    ev.close()
    return t1 - t0, rec


def kernel_stats(rec, w, kind_flops):
    """Per kind: launches, average ms, algorithmic TFLOP/s."""
    out = {}
    for kind in sorted({k for k, _ in rec}):
        ms = [m for k, m in rec if k == kind]
        avg = sum(ms) / len(ms)
        fl = kind_flops(kind) * pairs_of_kind(kind, w)
        out[kind] = {"launches": len(ms), "avg_ms": round(avg, 4),
                     "tflops": round(fl / (avg * 1e-3) / 1e12, 2) if fl else None}
    return out


def walk_stats(rec, flops, steps):
    """Fused walk: one launch per rank walks every visible chunk; its work is
    the walk's whole forward."""
    ms = sum(m for _, m in rec) / steps
    return {"fwd_walk": {"launches": len(rec), "ms_per_step": round(ms, 4),
                         "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}}


def untraced_steps(step_fn, steps, warmup, clock=None):
    """Runs warmup, then exactly `steps` timed steps with no per-launch
    events (for walks of many short launches, where bracketing every launch
    adds a gap of its own); step-boundary events into `clock`, if given.
    Returns seconds."""
    import torch

    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if clock:
        clock.mark()
    for _ in range(steps):
        step_fn()
        if clock:
            clock.mark()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def run_fwd(w, steps, warmup, ring_mode, H_kv=None, trace=True, concurrent=False, sampler=None):
    """The forward walk of workload w; H_kv < H runs it with grouped-query
    key/value chunks of H_kv heads.  trace=False times the steps without
    per-launch events (no per-kernel figures then).  concurrent=True walks
    every rank on a stream of its own, with its own staging slots, as the
    ranks of a real ring run at once (untraced)."""
    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd import inputs
    from long_context_exact_step_amd.workloads import fused_walk_applies, fwd_flops, step_kinds

    dev = torch.device("cuda", 0)
    B, H, C, d, P = w.B, w.H, w.C, w.d, w.P
    Hk = H if H_kv is None else H_kv
    qs = {r: inputs.chunk(w.id, inputs.Q, r, B, H, C, d).to(dev) for r in w.ranks}
    ks = [inputs.chunk(w.id, inputs.K, j, B, Hk, C, d).to(dev) for j in range(P)]
    vs = [inputs.chunk(w.id, inputs.V, j, B, Hk, C, d).to(dev) for j in range(P)]
    o = {r: torch.empty(B, H, C, d, device=dev) for r in w.ranks}
    lse = {r: torch.empty(B, H, C, device=dev) for r in w.ranks}
    # "double_buffer_in_kernel": the double-buffer walk with no copy stream,
    # each step kernel staging the next chunk itself.
    in_kernel = ring_mode == "double_buffer_in_kernel"
    if in_kernel:
        ring_mode = "double_buffer"
    nws = len(w.ranks) if concurrent else 1
    wss = [torch.empty(max(1, ra.workspace_bytes(P, B, H, C, d, ring_mode, H_kv=Hk)), dtype=torch.uint8,
                       device=dev) for _ in range(nws)]
    ws = wss[0]
    copy_stream = torch.cuda.Stream(dev) if ring_mode == "double_buffer" and not in_kernel else None
    if concurrent and copy_stream is not None:
        raise SystemExit("concurrent ranks: in-kernel staging or resident walks only (one copy stream per call)")
    streams = [torch.cuda.Stream(dev) for _ in w.ranks] if concurrent else None
    # The fused mode walks a rank's chunks in one launch where the library's
    # rule allows it, else per step; the launch count and the kernel stats
    # follow what runs.
    walks = [ring_mode == "fused" and fused_walk_applies(w, r) for r in w.ranks]
    if any(walks) and not all(walks):
        raise SystemExit(f"{w.name}: fused walk applies to some ranks only; time it per rank")
    fused = all(walks)
    n_launch = len(w.ranks) if fused else sum(sum(k != "skip" for *_, k in step_kinds(r, P, w.causal))
                                              for r in w.ranks)

    def step():
        for r in w.ranks:
            ra.ring_fwd(qs[r], ks, vs, o[r], lse[r], r, w.causal, w.scale, ring_mode=ring_mode,
                        workspace=ws, copy_stream=copy_stream)

    def step_concurrent():
        # Each rank's walk on its own stream, after the work queued so far.
        cur = torch.cuda.current_stream(dev)
        for n, r in enumerate(w.ranks):
            streams[n].wait_stream(cur)
            ra.ring_fwd(qs[r], ks, vs, o[r], lse[r], r, w.causal, w.scale, ring_mode=ring_mode,
                        workspace=wss[n], stream=streams[n], copy_stream=None)
        for st in streams:
            cur.wait_stream(st)

    clock = StepClock(steps)
    if concurrent:
        secs, rec = untraced_steps(step_concurrent, steps, warmup, clock), []
        trace = False
    elif trace:
        secs, rec = timed_steps(step, n_launch, steps, warmup, clock, sampler)
    else:
        secs, rec = untraced_steps(step, steps, warmup, clock), []
    flops = fwd_flops(w)
    res = {
        "secs": secs, "ms_per_step": secs / steps * 1e3, "ms_per_step_median": clock.median_ms(),
        "tflops": flops * steps / secs / 1e12,
        "tokens_per_s": B * C * len(w.ranks) * steps / secs,
        "launches_per_step": n_launch,
        "kernels": ({} if not trace else
                    walk_stats(rec, flops, steps) if fused else kernel_stats(rec, w, lambda k: 4 * d)),
        "kv_bytes_per_ring_step": 2 * B * Hk * C * d * 2,
        "rec": rec,
    }
    return res, (qs, ks, vs, o, lse)


def config_line(w, steps, warmup, ring_mode, concurrent=False):
    """The forward walk of workload w (every rank it lists) as a bench line:
    ms per step, algorithmic TFLOP/s, tokens/s and the fraction of the bf16
    peak.  Tokens are the local query tokens of every walked rank.  Timed
    without per-launch events."""
    import torch
    from long_context_exact_step_amd.workloads import fwd_flops
    r, tensors = run_fwd(w, steps, warmup, ring_mode, trace=False, concurrent=concurrent)
    del tensors
    torch.cuda.empty_cache()
    return {
        "workload": w.name, "ring_mode": ring_mode, "ranks": list(w.ranks), "steps": steps, "warmup": warmup,
        "ranks_walked": "concurrently, one stream each" if concurrent else "one after another, one stream",
        "ms_per_step": round(r["ms_per_step"], 4), "tflops": round(r["tflops"], 2),
        "ms_per_step_median": round(r["ms_per_step_median"], 4),
        "tflops_at_median": round(fwd_flops(w) / (r["ms_per_step_median"] * 1e-3) / 1e12, 2),
        "tokens_per_s": round(r["tokens_per_s"], 1),
        "frac_bf16_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
        "frac_derived_peak": round(r["tflops"] / DERIVED_PEAK_BF16_TFLOPS, 4),
        "launches_per_step": r["launches_per_step"],
        "timing": "wall clock over the timed steps, no per-launch events",
    }


def run_train(w, steps, warmup, H_kv=None):
    """Forward + backward walk of workload w; H_kv < H runs it with
    grouped-query key/value chunks of H_kv heads."""
    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd import inputs
    from long_context_exact_step_amd.workloads import bwd_flops, fwd_flops, step_kinds

    dev = torch.device("cuda", 0)
    B, H, C, d, P = w.B, w.H, w.C, w.d, w.P
    Hk = H if H_kv is None else H_kv
    r = w.ranks[0]
    q = inputs.chunk(w.id, inputs.Q, r, B, H, C, d).to(dev)
    do = inputs.chunk(w.id, inputs.DO, r, B, H, C, d).to(dev)
    ks = [inputs.chunk(w.id, inputs.K, j, B, Hk, C, d).to(dev) for j in range(P)]
    vs = [inputs.chunk(w.id, inputs.V, j, B, Hk, C, d).to(dev) for j in range(P)]
    o = torch.empty(B, H, C, d, device=dev)
    lse = torch.empty(B, H, C, device=dev)
    dq = torch.empty(B, H, C, d, device=dev)
    dk = [torch.zeros(B, Hk, C, d, device=dev) for _ in range(P)]
    dv = [torch.zeros(B, Hk, C, d, device=dev) for _ in range(P)]
    ws_f = torch.empty(ra.workspace_bytes(P, B, H, C, d, "double_buffer", H_kv=Hk), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(ra.workspace_bytes(P, B, H, C, d, "resident", bwd=True, H_kv=Hk), dtype=torch.uint8,
                       device=dev)
    copy_stream = torch.cuda.Stream(dev)
    nvis = sum(k != "skip" for *_, k in step_kinds(r, P, w.causal))
    n_launch = nvis + 2 + 2 * nvis

    def step():
        for t in dk + dv:
            t.zero_()
        ra.ring_fwd(q, ks, vs, o, lse, r, w.causal, w.scale, ring_mode="double_buffer", workspace=ws_f,
                    copy_stream=copy_stream)
        ra.ring_bwd(q, ks, vs, o, lse, do, dq, dk, dv, r, w.causal, w.scale, workspace=ws_b)

    clock = StepClock(steps)
    sampler = ClockSampler()
    secs, rec = timed_steps(step, n_launch, steps, warmup, clock, sampler)
    sclk = sampler.summary()
    cus, _ = ra.device_info()
    fl_f, fl_b = fwd_flops(w), bwd_flops(w)
    kf = {"fwd_diag": 4 * d, "fwd_full": 4 * d, "bwd_dq_diag": 6 * d, "bwd_dq_full": 6 * d,
          "bwd_dkdv_diag": 8 * d, "bwd_dkdv_full": 8 * d}
    ks_ = kernel_stats(rec, w, lambda k: kf.get(k, 0))
    fwd_ms = sum(m for k, m in rec if k.startswith("fwd")) / steps
    bwd_ms = sum(m for k, m in rec if k.startswith("bwd")) / steps
    bwd_mm_ms = sum(m for k, m in rec if k.startswith(("bwd_dq", "bwd_dkdv"))) / steps
    return {
        "workload": w.name, "steps": steps, "ms_per_step": secs / steps * 1e3,
        "ms_per_step_median": round(clock.median_ms(), 4),
        "tflops_fwd_bwd": (fl_f + fl_b) * steps / secs / 1e12,
        "tokens_per_s": B * C * steps / secs,
        "fwd_kernels_ms_per_step": round(fwd_ms, 3), "bwd_kernels_ms_per_step": round(bwd_ms, 3),
        "fwd_tflops_kernels": round(fl_f / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops_kernels_algorithmic": round(fl_b / (bwd_ms * 1e-3) / 1e12, 1),
        # The dQ and dK/dV kernels execute 14 d flop per pair (6 d + 8 d) for
        # the 10 d of the gradient: their executed rate, and that rate over the
        # peak at the engine clock the driver reported during the timed steps
        # (forward and backward together).
        "bwd_tflops_matmul_kernels_executed": round(1.4 * fl_b / (bwd_mm_ms * 1e-3) / 1e12, 1),
        "engine_clock_sampled": sclk,
        "bwd_executed_frac_of_peak_at_sampled_clock": (
            None if not sclk else
            round(1.4 * fl_b / (bwd_mm_ms * 1e-3) / (cus * 4096 * sclk["median_mhz"] * 1e6), 4)),
        "kernels": ks_,
    }


def run_ulysses(w, steps, warmup, rank=0):
    """One rank's share of head-partitioned (Ulysses) sequence parallelism on
    workload w's sequence: regroup its H/P heads of every chunk (the copies
    that stand in for the all-to-all), then attention over all P*C tokens."""
    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd import inputs

    dev = torch.device("cuda", 0)
    B, H, C, d, P = w.B, w.H, w.C, w.d, w.P
    S, Hs = P * C, H // P
    qc = [inputs.chunk(w.id, inputs.Q, j, B, H, C, d).to(dev) for j in range(P)]
    kc = [inputs.chunk(w.id, inputs.K, j, B, H, C, d).to(dev) for j in range(P)]
    vc = [inputs.chunk(w.id, inputs.V, j, B, H, C, d).to(dev) for j in range(P)]
    o = torch.empty(B, Hs, S, d, device=dev)
    lse = torch.empty(B, Hs, S, device=dev)
    ws = torch.empty(ra.ulysses_workspace_bytes(P, B, H, C, d), dtype=torch.uint8, device=dev)

    def step():
        ra.ulysses_fwd(qc, kc, vc, o, lse, rank, w.causal, w.scale, workspace=ws)

    secs, rec = timed_steps(step, 1, steps, warmup)
    pairs = B * Hs * (S * (S + 1) // 2 if w.causal else S * S)
    flops = 4 * d * pairs
    k_ms = sum(m for _, m in rec) / max(1, len(rec))
    out = {
        "rank": rank, "heads": Hs, "tokens": S, "ms_per_step": round(secs / steps * 1e3, 4),
        "tflops": round(flops * steps / secs / 1e12, 2),
        "attention_kernel_ms": round(k_ms, 4), "attention_kernel_tflops": round(flops / (k_ms * 1e-3) / 1e12, 2),
        "regroup_bytes_per_step": 2 * 3 * B * Hs * S * d * 2,
    }
    # Training step of the share: forward + backward (10*d flop per pair backward).
    dc = [inputs.chunk(w.id, inputs.DO, j, B, H, C, d).to(dev) for j in range(P)]
    dq, dk, dv = (torch.empty(B, Hs, S, d, device=dev) for _ in range(3))
    ws_b = torch.empty(ra.ulysses_workspace_bytes(P, B, H, C, d, bwd=True), dtype=torch.uint8, device=dev)

    def train_step():
        ra.ulysses_fwd(qc, kc, vc, o, lse, rank, w.causal, w.scale, workspace=ws)
        ra.ulysses_bwd(qc, kc, vc, dc, o, lse, dq, dk, dv, rank, w.causal, w.scale, workspace=ws_b)

    n_launch = 1 + 1 + 3 + 2
    t_secs, t_rec = timed_steps(train_step, n_launch, max(2, steps // 2), 1)
    t_steps = max(2, steps // 2)
    bwd_ms = sum(m for k_, m in t_rec if k_.startswith("bwd")) / t_steps
    out["train_ms_per_step"] = round(t_secs / t_steps * 1e3, 4)
    out["train_tflops_fwd_bwd"] = round(14 * d * pairs * t_steps / t_secs / 1e12, 2)
    out["bwd_kernels_ms"] = round(bwd_ms, 4)
    out["bwd_tflops_kernels_algorithmic"] = round(10 * d * pairs / (bwd_ms * 1e-3) / 1e12, 1)
    return out


def run_allgather(w, steps, warmup, wt):
    """One rank's share of all-gather sequence parallelism: copy the P key/value
    chunks into one gathered sequence (the copies stand in for the all-gather),
    then one attention pass of the rank's queries over it at a causal offset.
    Forward on workload w's rank, training step (forward + backward) on
    workload wt's rank."""
    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd import inputs
    from long_context_exact_step_amd.workloads import bwd_flops, fwd_flops

    dev = torch.device("cuda", 0)

    def tensors(x, with_do):
        B, H, C, d, P = x.B, x.H, x.C, x.d, x.P
        r = x.ranks[0]
        q = inputs.chunk(x.id, inputs.Q, r, B, H, C, d).to(dev)
        ks = [inputs.chunk(x.id, inputs.K, j, B, H, C, d).to(dev) for j in range(P)]
        vs = [inputs.chunk(x.id, inputs.V, j, B, H, C, d).to(dev) for j in range(P)]
        do = inputs.chunk(x.id, inputs.DO, r, B, H, C, d).to(dev) if with_do else None
        return r, q, ks, vs, do, torch.empty(B, H, C, d, device=dev), torch.empty(B, H, C, device=dev)

    r, q, ks, vs, _, o, lse = tensors(w, False)
    ws = torch.empty(ra.allgather_workspace_bytes(w.P, w.B, w.H, w.C, w.d), dtype=torch.uint8, device=dev)

    def step():
        ra.allgather_fwd(q, ks, vs, o, lse, r, w.causal, w.scale, workspace=ws)

    secs, rec = timed_steps(step, 1, steps, warmup)
    flops = fwd_flops(w, [r])
    k_ms = sum(m for _, m in rec) / max(1, len(rec))
    out = {
        "rank": r, "ms_per_step": round(secs / steps * 1e3, 4), "tflops": round(flops * steps / secs / 1e12, 2),
        "tokens_per_s": round(w.B * w.C * steps / secs, 1),
        "attention_kernel_ms": round(k_ms, 4), "attention_kernel_tflops": round(flops / (k_ms * 1e-3) / 1e12, 2),
        "gather_bytes_per_step": 2 * 2 * w.B * w.H * w.P * w.C * w.d * 2,
    }
    del q, ks, vs, o, lse, ws
    torch.cuda.empty_cache()

    r, q, ks, vs, do, o, lse = tensors(wt, True)
    S = wt.P * wt.C
    dq = torch.empty(wt.B, wt.H, wt.C, wt.d, device=dev)
    dk, dv = (torch.empty(wt.B, wt.H, S, wt.d, device=dev) for _ in range(2))
    ws_f = torch.empty(ra.allgather_workspace_bytes(wt.P, wt.B, wt.H, wt.C, wt.d), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(ra.allgather_workspace_bytes(wt.P, wt.B, wt.H, wt.C, wt.d, bwd=True), dtype=torch.uint8,
                       device=dev)

    def train_step():
        ra.allgather_fwd(q, ks, vs, o, lse, r, wt.causal, wt.scale, workspace=ws_f)
        ra.allgather_bwd(q, ks, vs, o, lse, do, dq, dk, dv, r, wt.causal, wt.scale, workspace=ws_b)

    t_steps = max(2, steps)
    # Launches per step: attention; rowdot, three fills, the dq kernel, the dk/dv pair.
    t_secs, t_rec = timed_steps(train_step, 7, t_steps, 1)
    fl_f, fl_b = fwd_flops(wt, [r]), bwd_flops(wt, [r])
    fwd_ms = sum(m for k_, m in t_rec if k_.startswith("fwd")) / t_steps
    bwd_ms = sum(m for k_, m in t_rec if k_.startswith("bwd")) / t_steps
    out["train"] = {
        "workload": wt.name, "rank": r, "steps": t_steps, "ms_per_step": round(t_secs / t_steps * 1e3, 4),
        "tflops_fwd_bwd": round((fl_f + fl_b) * t_steps / t_secs / 1e12, 2),
        "tokens_per_s": round(wt.B * wt.C * t_steps / t_secs, 1),
        "fwd_kernels_ms_per_step": round(fwd_ms, 3), "bwd_kernels_ms_per_step": round(bwd_ms, 3),
        "bwd_tflops_kernels_algorithmic": round(fl_b / (bwd_ms * 1e-3) / 1e12, 1),
    }
    del q, ks, vs, do, o, lse, dq, dk, dv, ws_f, ws_b
    torch.cuda.empty_cache()
    return out


def mfma_ceiling(iters=200000):
    """What the bf16 matrix cores deliver on this device: the peak derived from
    the CU count and maximum engine clock (4096 flop per CU per clock), and the
    throughput of a probe kernel (two waves per SIMD issuing back-to-back
    independent 32x32x16 bf16 MFMAs) on random N(0,1) operands and on zeros.
    The chip is power-limited and MFMA power depends on the data, so the
    random-operand figure is the ceiling that attention on N(0,1) inputs
    meets."""
    import torch
    import long_context_exact_step_amd as ra

    dev = torch.device("cuda", 0)
    cus, clk_khz = ra.device_info()
    out = {"cus": cus, "max_clock_mhz": clk_khz / 1e3,
           "derived_peak_tflops": round(cus * 4096 * clk_khz * 1e3 / 1e12, 1)}
    gen = torch.Generator().manual_seed(20261202)
    operands = {"random": torch.randn(8192, generator=gen).to(torch.bfloat16).to(dev),
                "zero": torch.zeros(8192, dtype=torch.bfloat16, device=dev)}
    sink = torch.empty(cus * 512, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    flops = cus * 8 * iters * 16 * 32768
    for name, ops in operands.items():
        ra.mfma_probe(ops, sink, clocks, cus, max(1, iters // 10))  # warm-up
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        ra.mfma_probe(ops, sink, clocks, cus, iters)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        cyc, ref = clocks.tolist()
        out[name] = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3),
                     "clock_ghz": round(cyc / (ref / 100e6) / 1e9, 3) if ref > 0 else None}
    return out


LADDER_LEVELS = {
    0: "dense probe: independent accumulators, register operands",
    1: "+ the kernel's accumulator pattern (4 P V outputs, 2 score chains restarting per tile)",
    2: "+ A operands read from LDS (ds_read_b64_tr_b16 pairs, ds_read_b128), 3 MFMAs ahead",
    3: "+ online softmax of the previous tile in the MFMA slots (scale, exp2, row sum, bf16 pack)",
    4: "+ one workgroup barrier per 64-key tile",
    5: "+ direct-to-LDS tile loads two tiles ahead, waited for before the barrier",
    6: "level 2 with one wave per SIMD holding 64 rows (each LDS operand read feeds two MFMAs)",
    7: "level 5 with one wave per SIMD holding 64 rows",
    8: "level 6 + the softmax only",
    9: "level 8 + one barrier per tile",
    10: "level 7 with the barrier every second tile",
}


def fwd_ladder(iters=20000):
    """The forward kernel's instruction stream rebuilt from the MFMA probe
    one feature per level (ra_fwd_ladder_probe), each on random N(0,1) and
    on all-zero data: TFLOP/s and the clock the cores ran at.  Random data
    show what each feature costs under the power limit; zeros show what it
    costs in the schedule at the unthrottled clock."""
    import torch
    import long_context_exact_step_amd as ra

    dev = torch.device("cuda", 0)
    cus, _ = ra.device_info()
    gen = torch.Generator().manual_seed(20261203)
    data = {"random": (torch.randn(10240, generator=gen).to(torch.bfloat16).to(dev),
                       torch.randn(524288, generator=gen).to(torch.bfloat16).to(dev)),
            "zero": (torch.zeros(10240, dtype=torch.bfloat16, device=dev),
                     torch.zeros(524288, dtype=torch.bfloat16, device=dev))}
    sink = torch.empty(cus * 512, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    flops = cus * 8 * iters * 4194304
    c = 1.0 / math.sqrt(128) * 1.4426950408889634
    out = {}
    for level, what in LADDER_LEVELS.items():
        row = {"adds": what}
        for name, (ops, tiles) in data.items():
            ra.fwd_ladder_probe(level, ops, tiles, sink, clocks, cus, max(1, iters // 20), c)  # warm-up
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            ra.fwd_ladder_probe(level, ops, tiles, sink, clocks, cus, iters, c)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            cyc, ref = clocks.tolist()
            tf = flops / (ms * 1e-3) / 1e12
            ghz = cyc / (ref / 100e6) / 1e9 if ref > 0 else None
            row[name] = {"tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "clock_ghz": round(ghz, 3) if ghz else None,
                         # Cycles per tile on one SIMD (two waves' 32 MFMAs, or one
                         # wave's 64: the floor is 64 x 32 = 2048), from the launch
                         # time and the clock.
                         "cycles_per_tile": round(ghz * 1e9 * ms * 1e-3 / (iters * 4), 1) if ghz else None,
                         # The same from wave 0 of block 0's own loop: without a
                         # barrier (levels 0-3) that wave can run ahead of its SIMD
                         # partner, and then reads less than the SIMD's figure.
                         "wave0_cycles_per_tile": round(cyc / (iters * 4), 1)}
        out[f"level{level}"] = row
    return out


def step_on_zeros(w, launches=5):
    """One full-chunk forward step (ra_step_fwd, no mask) at the workload's
    chunk shape on its seeded N(0,1) inputs and on all-zero inputs.  The
    instructions are the same; only the data, and so the matrix cores' power
    and the clock the chip holds, differ.  The zero-input rate shows what the
    kernel's schedule reaches at the unthrottled clock."""
    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd import inputs

    dev = torch.device("cuda", 0)
    B, H, C, d = w.B, w.H, w.C, w.d
    flops = 4 * d * B * H * C * C
    q = inputs.chunk(w.id, inputs.Q, w.ranks[-1], B, H, C, d).to(dev)
    k = inputs.chunk(w.id, inputs.K, 0, B, H, C, d).to(dev)
    v = inputs.chunk(w.id, inputs.V, 0, B, H, C, d).to(dev)
    o = torch.empty(B, H, C, d, device=dev)
    lse = torch.empty(B, H, C, device=dev)
    out = {"kernel": "fwd_step_kernel, full chunk, no merge", "C": C, "H": H}
    for name, (qq, kk, vv) in {"random": (q, k, v), "zero": tuple(torch.zeros_like(t) for t in (q, k, v))}.items():
        ra.step_fwd(qq, kk, vv, o, lse, 1, False, w.scale)  # warm-up
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(launches):
            ra.step_fwd(qq, kk, vv, o, lse, 1, False, w.scale)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / launches
        out[name] = {"ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def cpu_baseline(w, tensors, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample: 256 seeded query
    rows per head of the measured rank, heads taken in order until the time
    budget is spent.  Returns the baseline record and the GPU-vs-oracle error
    on those rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from long_context_exact_step_amd import inputs

    qs, ks, vs, o, lse = tensors
    r = w.ranks[-1]
    C, d, P = w.C, w.d, w.P
    f64 = lambda t: t.float().cpu().double().numpy()
    q_cpu = qs[r].cpu()
    secs = 0.0
    pairs = 0
    rows_done = 0
    heads = 0
    err_o = err_l = 0.0
    conv_secs = 0.0
    for h in range(w.H):
        rows = inputs.query_row_sample(w.id, h, C)
        tc = time.perf_counter()
        kh = np.concatenate([f64(ks[j][:, h:h + 1]) for j in range(P)], axis=2)
        vh = np.concatenate([f64(vs[j][:, h:h + 1]) for j in range(P)], axis=2)
        qh = f64(q_cpu[:, h:h + 1, rows])
        conv_secs += time.perf_counter() - tc
        pos = r * C + rows
        t0 = time.perf_counter()
        ro, rl = oracle.attention_fwd(qh, kh, vh, w.scale, w.causal, q_pos=pos)
        secs += time.perf_counter() - t0
        pairs += int((pos + 1).sum()) if w.causal else len(rows) * P * C
        rows_done += len(rows)
        heads += 1
        go = f64(o[r][:, h:h + 1, rows])
        gl = f64(lse[r][:, h:h + 1, rows])
        err_o = max(err_o, float(np.abs(go - ro).max()))
        err_l = max(err_l, float(np.abs(gl - rl).max()))
        if secs >= budget_s:
            break
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max((i.get("num_threads", 1) for i in blas), default=1)
    flops = 4 * d * pairs
    rate = flops / secs  # fp64 flop/s of the oracle on this sample
    from long_context_exact_step_amd.workloads import WORKLOADS, Workload, fwd_flops, queue_steps_apply
    # Whole-config times at the sample's rate: the sampled rows are uniform
    # over each head's rows, so the visible-pair ratio scales them without
    # bias.  Extrapolated, not measured.
    extrap = {"label": "extrapolated",
              "method": "sample seconds x (visible pairs of the full forward / visible pairs of the sample)"}
    for wid in sorted(WORKLOADS):
        x = WORKLOADS[wid]
        extrap[f"{x.name} full forward"] = {"tflop_fp64": round(fwd_flops(x) / 1e12, 3),
                                           "seconds": round(fwd_flops(x) / rate, 1)}
    return {
        "value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{rows_done} query rows ({heads} heads x 256 seeded rows) of rank {r}, each against its "
                  f"{'visible' if w.causal else 'whole'} key range of the unchunked sequence; fp64 NumPy",
        "blas": ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or None,
        "seconds": round(secs, 2),
        # Outside `seconds`: copying the sampled heads' bf16 inputs from the
        # GPU and widening them to fp64.
        "conversion_seconds": round(conv_secs, 2),
        # A token is one query position over all heads: the sample's rows
        # divided by the head count, per second.
        "tokens_per_s": round(rows_done / w.H / secs, 3),
        "host_cpus": len(os.sched_getaffinity(0)),
        "extrapolated": extrap,
    }, {"max_abs_err_o": err_o, "max_abs_err_lse": err_l, "rows": rows_done}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--ring-mode", default="double_buffer",
                    choices=["double_buffer", "double_buffer_in_kernel", "resident", "fused"])
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gqa", action="store_true", help="skip the grouped-query (H_kv = H/4) measurements")
    ap.add_argument("--no-ulysses", action="store_true", help="skip the head-partitioned (Ulysses) share")
    ap.add_argument("--no-allgather", action="store_true", help="skip the all-gather sequence-parallel share")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA throughput probe")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' forward lines (tiny ring, 32K full ring, 1M share)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CMD_FETCH", "CMD_WRITE"),
                    help="write the forward kernel's HBM traffic from two rocprofv3 counter passes (no GPU used)")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the ring on a single MI355X; multi-GPU runs "
              "(--gpus > 1) are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_exact_step_amd as ra
    from long_context_exact_step_amd.workloads import WORKLOADS, Workload, fwd_flops, queue_steps_apply

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    sampler = ClockSampler()
    fwd, tensors = run_fwd(w, args.steps, args.warmup, args.ring_mode, sampler=sampler)
    sclk = sampler.summary()
    print(f"[bench] fwd {w.name}: {fwd['ms_per_step']:.3f} ms/step, {fwd['tflops']:.1f} TFLOP/s", file=sys.stderr,
          flush=True)

    if "fwd_walk" in fwd["kernels"]:  # fused walk: the launches are the whole forward
        dom = "fwd_walk"
        dk = fwd["kernels"][dom]
        dk = {"launches": dk["launches"], "avg_ms": dk["ms_per_step"]}
        dom_flops = fwd_flops(w)
    else:
        dom = "fwd_full" if "fwd_full" in fwd["kernels"] else "fwd_diag"
        dk = fwd["kernels"][dom]
        dom_flops = 4 * w.d * pairs_of_kind(dom, w)
    # The kernel those launches ran: full-chunk steps of a double-buffer walk
    # large enough for persistent blocks run fwd_queue_kernel.
    cus, _ = ra.device_info()
    queued = args.ring_mode.startswith("double_buffer") and queue_steps_apply(w, "double_buffer", cus)
    full_kernel = "fwd_queue_kernel" if dom == "fwd_full" and queued else "fwd_step_kernel"
    achieved = dom_flops / (dk["avg_ms"] * 1e-3) / 1e12
    traffic = None
    try:
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
        # The counters cover one kernel of one workload (not the fused walk).
        if (prof.get("source_sha") == fwd_kernel_sha() and prof.get("workload_id") == w.id and dom != "fwd_walk"
                and prof.get("kernel", "").startswith(full_kernel)):
            traffic = prof.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
        # HBM bytes per launch (counters) over the live launch time: achieved HBM bandwidth.
        "traffic_gbps": None if traffic is None else round(traffic / (dk["avg_ms"] * 1e-3) / 1e9, 1),
        "kernel": (f"fwd_walk_kernel (fused walk), {dk['launches']} launches, {dk['avg_ms']} ms per step"
                   if dom == "fwd_walk" else f"{full_kernel} ({dom}), {dk['launches']} launches, avg {dk['avg_ms']} ms"),
        "flops_per_launch": dom_flops,  # fused walk: per step (all its launches)
        # The engine clock the driver reported during the timed steps, and
        # `achieved` over the peak at that clock (CUs x 4096 flop per clock;
        # the median sample, which the full-chunk launches dominate).
        "engine_clock_sampled": sclk,
        "frac_of_peak_at_sampled_clock": (None if not sclk else
                                          round(achieved / (cus * 4096 * sclk["median_mhz"] * 1e6 / 1e12), 4)),
    }

    out = {
        "metric": METRIC, "value": round(fwd["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(fwd["ms_per_step"], 4),
        # Median over the timed steps (step-boundary events on the compute
        # stream) beside the mean that `value` is computed from.
        "ms_per_step_median": round(fwd["ms_per_step_median"], 4),
        "tflops_at_median": round(fwd_flops(w) / (fwd["ms_per_step_median"] * 1e-3) / 1e12, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "C": w.C, "P": w.P, "rank": list(w.ranks), "d": w.d,
                   "causal": w.causal, "ring_mode": args.ring_mode},
        "tokens_per_s": round(fwd["tokens_per_s"], 1),
        "pct_bf16_dense_peak": round(100 * fwd["tflops"] / PEAK_BF16_TFLOPS, 2),
        "pct_derived_bf16_peak": round(100 * fwd["tflops"] / DERIVED_PEAK_BF16_TFLOPS, 2),
        "kernels": fwd["kernels"],
        "roofline": roofline,
    }
    if not args.no_ceiling:
        ce = mfma_ceiling()
        ce["kernel_frac_of_random_ceiling"] = round(achieved / ce["random"]["tflops"], 4)
        ce["step_kernel_by_input_data"] = step_on_zeros(w)
        ce["fwd_ladder"] = fwd_ladder()
        for lv, row in ce["fwd_ladder"].items():
            print(f"[bench] ladder {lv}: random {row['random']['tflops']} TFLOP/s at {row['random']['clock_ghz']} GHz"
                  f" ({row['random']['cycles_per_tile']} cyc/tile), zero {row['zero']['tflops']} at "
                  f"{row['zero']['clock_ghz']} GHz ({row['zero']['cycles_per_tile']} cyc/tile)", file=sys.stderr,
                  flush=True)
        out["mfma_ceiling"] = ce
        print(f"[bench] MFMA probe: random {ce['random']['tflops']} TFLOP/s at {ce['random']['clock_ghz']} GHz, "
              f"zero {ce['zero']['tflops']} TFLOP/s at {ce['zero']['clock_ghz']} GHz; derived peak "
              f"{ce['derived_peak_tflops']}", file=sys.stderr, flush=True)
        sz = ce["step_kernel_by_input_data"]
        print(f"[bench] full-chunk step kernel: random inputs {sz['random']['tflops']} TFLOP/s, zero inputs "
              f"{sz['zero']['tflops']} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_cpu:
        cb, par = cpu_baseline(w, tensors, args.cpu_seconds)
        cb["pct_derived_bf16_peak_of_gpu_line"] = out["pct_derived_bf16_peak"]
        out["cpu_baseline"] = cb
        out["parity_on_baseline_rows"] = par
    del tensors
    torch.cuda.empty_cache()
    if not args.no_configs:
        # Every other forward workload in the same run: the tiny ring and the
        # 32K full ring over all ranks, the 1M share; the full ring in both the
        # double-buffer walk (the ring's emulation) and the fused walk.
        cfgs = {}
        # The 128K share at head size 64 (H = 64: the same flops and bytes).
        d64 = dataclasses.replace(WORKLOADS[2], H=64, d=64,
                                  name="128K/CP=4 local share, rank 3, H=64, d=64, causal fwd")
        for key, wid, mode, st, conc in (
                ("tiny_ring", 1, "double_buffer", args.steps, False),
                ("share_128k_cp4_d64", d64, "double_buffer", args.steps, False),
                ("share_128k_cp4_double_buffer_in_kernel", 2, "double_buffer_in_kernel", args.steps, False),
                ("full_ring_32k_double_buffer", 3, "double_buffer", args.steps, False),
                ("full_ring_32k_double_buffer_in_kernel", 3, "double_buffer_in_kernel", args.steps, False),
                ("full_ring_32k_double_buffer_in_kernel_ranks_concurrent", 3, "double_buffer_in_kernel",
                 args.steps, True),
                ("full_ring_32k_resident", 3, "resident", args.steps, False),
                ("full_ring_32k_fused", 3, "fused", args.steps, False),
                ("share_1m_cp8", 4, "double_buffer", 5, False)):
            wl = wid if isinstance(wid, Workload) else WORKLOADS[wid]
            if wl == w and mode == args.ring_mode and not conc:
                continue
            c = config_line(wl, st, min(2, args.warmup), mode, concurrent=conc)
            cfgs[key] = c
            print(f"[bench] {key}: {c['ms_per_step']:.3f} ms/step, {c['tflops']:.1f} TFLOP/s "
                  f"({c['frac_bf16_peak']:.3f} of peak), {c['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
        out["configs"] = cfgs
    if not args.no_train and w.id != 5:
        tr = run_train(WORKLOADS[5], max(3, args.steps // 2), max(1, args.warmup))
        out["train"] = tr
        print(f"[bench] train: {tr['ms_per_step']:.3f} ms/step, {tr['tflops_fwd_bwd']:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
        # The training share at head size 64 (H = 64).
        w64 = dataclasses.replace(WORKLOADS[5], H=64, d=64,
                                  name="training share C=16K, P=4, rank 3, H=64, d=64, causal fwd+bwd")
        t64 = run_train(w64, max(3, args.steps // 2), max(1, args.warmup))
        out["train_d64"] = t64
        print(f"[bench] train d=64: {t64['ms_per_step']:.3f} ms/step, {t64['tflops_fwd_bwd']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    if not args.no_gqa and w.H % 4 == 0:
        # Grouped-query attention, 4 query heads per key/value head: the same
        # attention flops, a quarter of the key/value bytes each ring step moves.
        Hk = w.H // 4
        g, _ = run_fwd(w, args.steps, args.warmup, args.ring_mode, H_kv=Hk)
        out["gqa"] = {
            "H": w.H, "H_kv": Hk, "fwd_ms_per_step": round(g["ms_per_step"], 4),
            "fwd_tflops": round(g["tflops"], 2), "kernels": g["kernels"],
            "kv_bytes_per_ring_step": g["kv_bytes_per_ring_step"],
            "kv_bytes_per_ring_step_mha": fwd["kv_bytes_per_ring_step"],
        }
        print(f"[bench] gqa fwd H_kv={Hk}: {g['ms_per_step']:.3f} ms/step, {g['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        wt = WORKLOADS[5]
        if not args.no_train and wt.H % 4 == 0:
            gt = run_train(wt, max(3, args.steps // 2), max(1, args.warmup), H_kv=wt.H // 4)
            out["gqa"]["train"] = gt
            print(f"[bench] gqa train H_kv={wt.H // 4}: {gt['ms_per_step']:.3f} ms/step, "
                  f"{gt['tflops_fwd_bwd']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_ulysses and w.H % w.P == 0:
        torch.cuda.empty_cache()
        u = run_ulysses(w, max(3, args.steps // 2), max(1, args.warmup))
        u["ring_rank_ms_per_step"] = out["ms_per_step"]
        out["ulysses"] = u
        print(f"[bench] ulysses share ({u['heads']} heads x {u['tokens']} tokens): {u['ms_per_step']:.3f} ms/step, "
              f"{u['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_allgather:
        torch.cuda.empty_cache()
        a = run_allgather(w, args.steps, args.warmup, WORKLOADS[5])
        a["ring_rank_ms_per_step"] = out["ms_per_step"]
        out["allgather"] = a
        print(f"[bench] all-gather share rank {a['rank']}: {a['ms_per_step']:.3f} ms/step, {a['tflops']:.1f} TFLOP/s; "
              f"train {a['train']['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
