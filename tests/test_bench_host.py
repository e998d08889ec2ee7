"""bench.py's host logic on the CPU: the multi-GPU refusal and the counter
ingestion that turns two rocprofv3 counter passes into the forward kernel's
HBM bytes per launch (copy-calibrated)."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

KERNEL = "void ra::(anonymous namespace)::fwd_queue_kernel<128, true>(unsigned short const*, float*)"
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr


def _write_pass(d, counter, kernel_values, copy_values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        n = 0
        for name, vals in ((KERNEL, kernel_values), (COPY, copy_values)):
            for v in vals:
                n += 1
                w.writerow({"Dispatch_Id": n, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_counter_ingestion(tmp_path):
    """The staging copies move one 256 MiB chunk (262144 KiB); a copy that
    reads FETCH_SIZE 131072 KiB gives a factor of 2.  Small copies (not the
    chunk staging) are ignored for the calibration."""
    _write_pass(tmp_path / "f", "FETCH_SIZE", [1000.0, 1200.0], [131072.0, 131072.0, 64.0])
    _write_pass(tmp_path / "w", "WRITE_SIZE", [500.0, 700.0], [262144.0, 262144.0, 8.0])
    out = tmp_path / "counters.json"
    rec = bench.ingest_counters(str(tmp_path / "f"), str(tmp_path / "w"), "cmd f", "cmd w", out_path=str(out))
    assert rec["copy_calibration"]["fetch_factor"] == 2.0
    assert rec["copy_calibration"]["write_factor"] == 1.0
    assert rec["hbm_fetch_bytes_per_launch"] == 1100.0 * 2 * 1024
    assert rec["hbm_write_bytes_per_launch"] == 600.0 * 1024
    assert rec["hbm_bytes_per_launch"] == (2200.0 + 600.0) * 1024
    assert rec["source_sha"] == bench.fwd_kernel_sha()
    assert json.loads(out.read_text()) == rec


def test_engine_clock_parse():
    """The sampled engine clock is the level marked '*' in pp_dpm_sclk."""
    assert bench.ClockSampler.parse("0: 500Mhz\n1: 1652Mhz *\n2: 2400Mhz\n") == 1652.0
    assert bench.ClockSampler.parse("0: 500Mhz *\n1: 2400Mhz\n") == 500.0
    assert bench.ClockSampler.parse("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.ClockSampler.parse("") is None


def test_queue_rule():
    """bench.py names the kernel of the full-chunk launches by the library's
    rule for persistent steps: the double-buffer walk with at least four
    units of 256 query rows per compute unit."""
    from dataclasses import replace

    from long_context_exact_step_amd.workloads import WORKLOADS, queue_steps_apply

    assert queue_steps_apply(WORKLOADS[2], "double_buffer", 256)      # 32 heads x 128 query tiles
    assert queue_steps_apply(WORKLOADS[5], "double_buffer", 256)      # 32 x 64
    assert not queue_steps_apply(WORKLOADS[3], "double_buffer", 256)  # 32 x 16: 2 per CU
    assert not queue_steps_apply(WORKLOADS[2], "resident", 256)
    assert not queue_steps_apply(WORKLOADS[2], "fused", 256)
    w = replace(WORKLOADS[3], C=8192)
    assert queue_steps_apply(w, "double_buffer", 256)                 # 32 x 32 = 4 per CU
    assert not queue_steps_apply(replace(w, C=8192 - 256), "double_buffer", 256)


def test_fused_walk_rule_mirrors_the_library():
    """bench.py sizes a fused-mode run by the library's rule for when one
    launch walks a rank's chunks (C % 64 == 0, at most 16 visible chunks,
    visible chunks * C < 2^30); otherwise the call runs per step."""
    from dataclasses import replace

    from long_context_exact_step_amd.workloads import WORKLOADS, fused_walk_applies

    for wid in (2, 3, 4, 5):
        w = WORKLOADS[wid]
        assert all(fused_walk_applies(w, r) for r in w.ranks)
    w = WORKLOADS[3]
    assert not fused_walk_applies(replace(w, C=4000), 7)            # C not a multiple of 64
    assert not fused_walk_applies(replace(w, P=17, causal=False), 0)  # 17 visible chunks
    assert fused_walk_applies(replace(w, P=17), 15)                 # causal rank 15: 16 visible
    assert not fused_walk_applies(replace(w, C=2 ** 27), 7)         # 8 chunks * 2^27 = 2^30
    assert fused_walk_applies(replace(w, C=2 ** 27 - 64), 7)
    assert fused_walk_applies(replace(w, C=2 ** 27), 6)             # 7 chunks
