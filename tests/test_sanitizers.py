"""Host sanitizers on the C-ABI library: the host code (argument validation,
the ring schedule and walk set-up, workspace sizing, tracing state) built
with AddressSanitizer and UndefinedBehaviorSanitizer, and the host-side ABI
tests run against that build with the sanitizer runtime preloaded.  Any
report fails the run (halt on error, no recovery).  No GPU is used: every
call the host tests make returns before enqueueing work."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from long_context_exact_step_amd import build as rabuild  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def runtime():
    rt = rabuild.asan_runtime()
    if rt is None or shutil.which(rabuild.hipcc()) is None and not os.path.exists(rabuild.hipcc()):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    return rt


def _env(rt, **extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = rt
    env.update(extra)
    return env


@pytest.mark.parametrize("fault,report", [("heap", "AddressSanitizer: heap-buffer-overflow"),
                                          ("signed", "runtime error: signed integer overflow")])
def test_harness_reports_planted_faults(runtime, tmp_path, fault, report):
    """The harness itself: a shared library with a planted heap overflow and
    a planted signed overflow, built with the same host flags and loaded by
    Python the same way, must be stopped with the sanitizer's report (so a
    clean run below means something)."""
    src = tmp_path / "faults.hip"
    src.write_text("#include <climits>\n#include <cstdlib>\n"
                   "extern \"C\" int heap(int i) { int* p = (int*)std::malloc(4 * sizeof(int));\n"
                   "  p[i + 3] = 1; int r = p[0]; std::free(p); return r; }\n"
                   "extern \"C\" int signed_add(int i) { return INT_MAX - 1 + i; }\n")
    lib = tmp_path / "libfaults.so"
    subprocess.run([rabuild.hipcc(), *rabuild.common_flags(("-g", *rabuild.SANITIZE_HOST), "-O1"), "-shared",
                    str(src), "-o", str(lib)], check=True, capture_output=True)
    call = "heap(1)" if fault == "heap" else "signed_add(2)"
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(lib)!r}).{call}"],
                       env=_env(runtime), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert report in r.stderr, r.stderr[-2000:]


def test_host_abi_tests_clean_under_asan_and_ubsan(runtime, tmp_path):
    lib = rabuild.build_sanitized(str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=_env(runtime, RA_LIB_PATH=lib),
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
