"""Builds libra.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m long_context_exact_step_amd.build

Each HIP source is compiled to an object under <repo>/_build/ in parallel and
linked into long_context_exact_step_amd/libra.so; the plain-C client
(csrc/ra_client.c) is then built beside it as ra_client.  Always rebuilds.

build_sanitized() builds the same library with the host code instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual); the
CPU tests load it with the sanitizer runtime preloaded and run the host-side
validation and ring-walk logic against it.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libra.so")
CLIENT = os.path.join(PKG, "ra_client")
SOURCES = ["ra_api.hip", "ra_fwd.hip", "ra_merge.hip", "ra_bwd.hip", "ra_ceiling.hip", "ra_ladder.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


# Host-only sanitizers: -Xarch_host keeps them off the device code.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """The clang ASan runtime (with the UBSan handlers) that a process must
    preload to load the sanitized library; None if absent."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def common_flags(extra=(), opt="-O3"):
    return [
        f"--offload-arch={ARCH}", opt, "-std=c++17", "-fPIC",
        # No packed-fp32 VALU instructions in any kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE, "-I" + CSRC, *extra,
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False, extra_flags=(), out=LIB, build_dir=BUILD, opt="-O3"):
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc(), *common_flags(extra_flags, opt), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    if out == LIB:
        client = build_client()
        if verbose:
            print(f"built {client}", file=sys.stderr)
    return out


def build_sanitized(out_dir, verbose=False):
    """libra_san.so under out_dir: host code with ASan + UBSan (-O1 -g),
    device code unchanged.  Returns its path."""
    return build(verbose=verbose, extra_flags=("-g", *SANITIZE_HOST), out=os.path.join(out_dir, "libra_san.so"),
                 build_dir=os.path.join(out_dir, "obj"), opt="-O1")


def build_client():
    """ra_client: a plain-C program that drives the library through
    include/ra.h alone (C11, host code, linked against libra.so and the HIP
    runtime)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = CLIENT + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I" + INCLUDE, "-I" + os.path.join(rocm, "include"), os.path.join(CSRC, "ra_client.c"),
          "-L" + PKG, "-lra", "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp])
    os.replace(tmp, CLIENT)
    return CLIENT


if __name__ == "__main__":
    build(verbose=True)
