"""The C-ABI library on the CPU: it loads, exports every function include/ra.h
declares, and rejects bad arguments with the documented status codes before
touching the GPU (validation is pure host code; no call here launches work).
"""

import ctypes
import os
import re

import pytest

import long_context_exact_step_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")

RA_OK, RA_ERR_NULL, RA_ERR_SHAPE, RA_ERR_ALIGN, RA_ERR_UNSUPPORTED, RA_ERR_RANK, RA_ERR_WORKSPACE = range(7)

FAKE = 0x10000  # an aligned, never-dereferenced address
MIS = 0x10008   # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return ra.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"ra_step_fwd", "ra_lse_merge", "ra_ring_fwd", "ra_ring_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in ra.h but not exported"


def test_version_and_status_strings(L):
    # 2: grouped-query (*_gqa) entry points; 3: ra_ulysses_fwd, ra_ulysses_bwd;
    # 4: ra_allgather_fwd, ra_allgather_bwd; 5: ra_ring_bwd_noalloc; 6: ra_fwd_ladder_probe
    assert L.ra_version() == 6
    assert L.ra_status_string(RA_OK) == b"RA_OK"
    assert L.ra_status_string(RA_ERR_WORKSPACE) == b"RA_ERR_WORKSPACE"
    assert L.ra_status_string(12345) == b"RA_ERR_UNKNOWN"


def vp(x):
    return ctypes.c_void_p(x)


def step(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Sq=64, Sk=64, d=128, step=1, causal=0):
    return L.ra_step_fwd(vp(q), vp(k), vp(v), vp(o), vp(lse), B, H, Sq, Sk, d, 0.125, step, causal, None)


def test_step_fwd_validation(L):
    assert step(L, q=0) == RA_ERR_NULL
    assert step(L, lse=0) == RA_ERR_NULL
    assert step(L, d=96) == RA_ERR_UNSUPPORTED
    assert step(L, d=256) == RA_ERR_UNSUPPORTED
    assert step(L, B=0) == RA_ERR_SHAPE
    assert step(L, Sk=0) == RA_ERR_SHAPE
    assert step(L, step=-1) == RA_ERR_SHAPE
    assert step(L, step=0, causal=1, Sq=64, Sk=65) == RA_ERR_SHAPE
    assert step(L, v=MIS) == RA_ERR_ALIGN
    assert step(L, B=1 << 16, H=1 << 16, Sq=1) == RA_ERR_SHAPE  # rows overflow 32 bits
    assert b"d=96" in (step(L, d=96), L.ra_last_error())[1]


def test_lse_merge_validation(L):
    m = lambda o=FAKE, lse=FAKE, op=FAKE + 4096, lp=FAKE + 8192, d=64: L.ra_lse_merge(
        vp(o), vp(lse), vp(op), vp(lp), 1, 1, 8, d, None)
    assert m(o=0) == RA_ERR_NULL
    assert m(d=32) == RA_ERR_UNSUPPORTED
    assert m(lse=MIS) == RA_ERR_ALIGN
    assert m(op=FAKE) == RA_ERR_SHAPE  # output aliases the partial


def ring_fwd(L, P=4, rank=3, mode=1, ws=FAKE, ws_bytes=None, chunks=None, d=128, C=64):
    arr = (ctypes.c_void_p * P)(*([FAKE] * P if chunks is None else chunks))
    need = L.ra_ring_workspace_bytes(P, 1, 2, C, d, mode, 0)
    wsb = need if ws_bytes is None else ws_bytes
    return L.ra_ring_fwd(vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), rank, 1, 0.1, 1, 2, C, d, mode,
                         vp(ws), wsb, None, None)


def test_ring_fwd_validation(L):
    assert ring_fwd(L, rank=4) == RA_ERR_RANK
    assert ring_fwd(L, rank=-1) == RA_ERR_RANK
    assert ring_fwd(L, mode=7) == RA_ERR_UNSUPPORTED
    assert ring_fwd(L, mode=2, rank=4) == RA_ERR_RANK  # the fused walk validates like the others
    assert ring_fwd(L, mode=2, chunks=[FAKE, MIS, FAKE, FAKE]) == RA_ERR_ALIGN
    assert ring_fwd(L, chunks=[FAKE, 0, FAKE, FAKE]) == RA_ERR_NULL
    assert ring_fwd(L, chunks=[FAKE, MIS, FAKE, FAKE]) == RA_ERR_ALIGN
    assert ring_fwd(L, ws=0) == RA_ERR_WORKSPACE
    need = L.ra_ring_workspace_bytes(4, 1, 2, 64, 128, 1, 0)
    assert ring_fwd(L, ws_bytes=need - 1) == RA_ERR_WORKSPACE
    assert ring_fwd(L, d=80) == RA_ERR_UNSUPPORTED
    assert ring_fwd(L, P=0, rank=0) == RA_ERR_SHAPE


def test_ring_bwd_validation(L):
    P, C, d = 4, 64, 128
    arr = (ctypes.c_void_p * P)(*([FAKE] * P))
    need = L.ra_ring_workspace_bytes(P, 1, 2, C, d, 0, 1)
    args = lambda rank=3, ws=FAKE, wsb=need: L.ra_ring_bwd(
        vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), arr, arr, rank, 1, 0.1,
        1, 2, C, d, vp(ws), wsb, None)
    assert args(rank=5) == RA_ERR_RANK
    assert args(ws=0) == RA_ERR_WORKSPACE
    assert args(wsb=need - 4) == RA_ERR_WORKSPACE
    assert L.ra_ring_bwd(None, arr, arr, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), arr, arr, 0, 1, 0.1,
                         1, 2, C, d, vp(FAKE), need, None) == RA_ERR_NULL


def test_ring_bwd_noalloc_validation(L):
    """The no-allocation backward validates like ra_ring_bwd_gqa (before the
    scratch lookup, which is the first device call) and rejects more query
    rows than its static scratch holds."""
    P, C, d = 4, 64, 128
    arr = (ctypes.c_void_p * P)(*([FAKE] * P))
    call = lambda q=FAKE, rank=3, B=1, H=2, Hk=2, C=C, d=d, chunks=arr: L.ra_ring_bwd_noalloc(
        vp(q), chunks, chunks, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), chunks, chunks, rank, 1, 0.1,
        B, H, Hk, C, d, None)
    assert call(q=0) == RA_ERR_NULL
    assert call(q=MIS) == RA_ERR_ALIGN
    assert call(rank=4) == RA_ERR_RANK
    assert call(d=96) == RA_ERR_UNSUPPORTED
    assert call(H=6, Hk=4) == RA_ERR_SHAPE
    assert call(chunks=(ctypes.c_void_p * P)(FAKE, 0, FAKE, FAKE)) == RA_ERR_NULL
    max_rows = 1 << 21
    assert call(B=1, H=32, C=max_rows // 32 + 1) == RA_ERR_WORKSPACE
    assert b"scratch" in L.ra_last_error()
    assert call(B=2, H=32, Hk=8, C=max_rows // 64 + 64) == RA_ERR_WORKSPACE


def test_workspace_sizes(L):
    # Double buffer: 2 slots x (K + V) x B*H*C*d bf16, then 2 x 512 bytes of queue counters.
    assert L.ra_ring_workspace_bytes(4, 1, 32, 32768, 128, 1, 0) == 2 * 2 * 32 * 32768 * 128 * 2 + 1024
    assert L.ra_ring_workspace_bytes(4, 1, 32, 32768, 128, 0, 0) == 0
    assert L.ra_ring_workspace_bytes(4, 1, 32, 32768, 128, 2, 0) == 0  # fused walk: no staging
    assert L.ra_ring_workspace_bytes(4, 1, 32, 16384, 128, 0, 1) == 2 * 32 * 16384 * 4
    assert L.ra_ring_workspace_bytes(4, 1, 32, 16384, 96, 0, 1) == 0


def test_gqa_workspace_sizes(L):
    # Double buffer holds H_kv-head chunks; the backward's per-row values keep H heads.
    assert L.ra_ring_workspace_bytes_gqa(4, 1, 32, 8, 32768, 128, 1, 0) == 2 * 2 * 8 * 32768 * 128 * 2 + 1024
    assert L.ra_ring_workspace_bytes_gqa(4, 1, 32, 8, 16384, 128, 0, 1) == 2 * 32 * 16384 * 4
    assert L.ra_ring_workspace_bytes_gqa(4, 1, 32, 32, 32768, 128, 1, 0) == L.ra_ring_workspace_bytes(
        4, 1, 32, 32768, 128, 1, 0)
    assert L.ra_ring_workspace_bytes_gqa(4, 1, 32, 5, 32768, 128, 1, 0) == 0  # 5 does not divide 32
    assert L.ra_ring_workspace_bytes_gqa(4, 1, 32, 0, 32768, 128, 1, 0) == 0


def test_gqa_validation(L):
    P, C, d = 4, 64, 128
    arr = (ctypes.c_void_p * P)(*([FAKE] * P))
    for H, Hk in ((6, 4), (4, 0), (3, 6)):
        assert L.ra_step_fwd_gqa(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, H, Hk, 64, 64, d, 0.1,
                                 1, 1, None) == RA_ERR_SHAPE
        assert L.ra_ring_fwd_gqa(vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), 3, 1, 0.1, 1, H, Hk, C, d, 0,
                                 None, 0, None, None) == RA_ERR_SHAPE
        assert L.ra_ring_bwd_gqa(vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), arr, arr, 3, 1,
                                 0.1, 1, H, Hk, C, d, vp(FAKE), 1 << 20, None) == RA_ERR_SHAPE
    # A valid grouping gets past the head check to the next one (here: the rank).
    assert L.ra_ring_fwd_gqa(vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), 9, 1, 0.1, 1, 8, 2, C, d, 0,
                             None, 0, None, None) == RA_ERR_RANK


def test_ulysses_workspace_and_validation(L):
    assert L.ra_ulysses_workspace_bytes(4, 1, 32, 32768, 128, 0) == 3 * 8 * 131072 * 128 * 2
    assert L.ra_ulysses_workspace_bytes(4, 1, 32, 32768, 128, 1) == 4 * 8 * 131072 * 128 * 2 + 2 * 8 * 131072 * 4
    assert L.ra_ulysses_workspace_bytes(3, 1, 32, 64, 128, 0) == 0  # 32 heads do not split over 3
    P, C, d = 4, 64, 128
    arr = (ctypes.c_void_p * P)(*([FAKE] * P))
    need = L.ra_ulysses_workspace_bytes(P, 1, 8, C, d, 0)
    call = lambda H=8, rank=1, ws=FAKE, wsb=need, chunks=arr: L.ra_ulysses_fwd(
        chunks, chunks, chunks, P, vp(FAKE), vp(FAKE), rank, 1, 0.1, 1, H, C, d, vp(ws), wsb, None)
    assert call(H=6) == RA_ERR_SHAPE
    assert call(rank=4) == RA_ERR_RANK
    assert call(ws=0) == RA_ERR_WORKSPACE
    assert call(wsb=need - 16) == RA_ERR_WORKSPACE
    assert call(chunks=(ctypes.c_void_p * P)(FAKE, FAKE, 0, FAKE)) == RA_ERR_NULL
    assert call(chunks=(ctypes.c_void_p * P)(FAKE, MIS, FAKE, FAKE)) == RA_ERR_ALIGN
    need_b = L.ra_ulysses_workspace_bytes(P, 1, 8, C, d, 1)
    bwd = lambda H=8, rank=1, wsb=need_b, dO=arr: L.ra_ulysses_bwd(
        arr, arr, arr, dO, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), rank, 1, 0.1, 1, H, C, d,
        vp(FAKE), wsb, None)
    assert bwd(H=6) == RA_ERR_SHAPE
    assert bwd(rank=-1) == RA_ERR_RANK
    assert bwd(wsb=need_b - 16) == RA_ERR_WORKSPACE
    assert bwd(dO=(ctypes.c_void_p * P)(FAKE, FAKE, FAKE, 0)) == RA_ERR_NULL


def test_allgather_workspace_and_validation(L):
    kv = 2 * 8 * 131072 * 128 * 2  # gathered K and V, H_kv = 8, S = 4 * 32768
    assert L.ra_allgather_workspace_bytes(4, 1, 32, 8, 32768, 128, 0) == kv
    assert L.ra_allgather_workspace_bytes(4, 1, 32, 8, 32768, 128, 1) == kv + 2 * 32 * 32768 * 4
    assert L.ra_allgather_workspace_bytes(4, 1, 32, 6, 64, 128, 0) == 0  # 32 heads over 6 groups
    assert L.ra_allgather_workspace_bytes(4, 1, 32, 32, 64, 96, 0) == 0  # unsupported d
    P, C, d = 4, 64, 128
    arr = (ctypes.c_void_p * P)(*([FAKE] * P))
    need = L.ra_allgather_workspace_bytes(P, 1, 8, 2, C, d, 0)
    call = lambda H=8, Hk=2, rank=1, ws=FAKE, wsb=need, k=arr, q=FAKE, d=d: L.ra_allgather_fwd(
        vp(q), k, arr, P, vp(FAKE), vp(FAKE), rank, 1, 0.1, 1, H, Hk, C, d, vp(ws), wsb, None)
    assert call(Hk=3) == RA_ERR_SHAPE
    assert call(d=96) == RA_ERR_UNSUPPORTED
    assert call(rank=4) == RA_ERR_RANK
    assert call(rank=-1) == RA_ERR_RANK
    assert call(ws=0) == RA_ERR_WORKSPACE
    assert call(wsb=need - 16) == RA_ERR_WORKSPACE
    assert call(q=0) == RA_ERR_NULL
    assert call(q=MIS) == RA_ERR_ALIGN
    assert call(k=(ctypes.c_void_p * P)(FAKE, FAKE, FAKE, 0)) == RA_ERR_NULL  # every chunk is gathered
    assert call(k=(ctypes.c_void_p * P)(FAKE, MIS, FAKE, FAKE)) == RA_ERR_ALIGN
    need_b = L.ra_allgather_workspace_bytes(P, 1, 8, 2, C, d, 1)
    assert need_b == need + 2 * 8 * C * 4
    bwd = lambda Hk=2, rank=1, wsb=need_b, dk=FAKE: L.ra_allgather_bwd(
        vp(FAKE), arr, arr, P, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(dk), vp(FAKE), rank, 1, 0.1, 1, 8, Hk,
        C, d, vp(FAKE), wsb, None)
    assert bwd(Hk=5) == RA_ERR_SHAPE
    assert bwd(rank=4) == RA_ERR_RANK
    assert bwd(wsb=need_b - 16) == RA_ERR_WORKSPACE
    assert bwd(dk=0) == RA_ERR_NULL
    assert bwd(dk=MIS) == RA_ERR_ALIGN


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    o = torch.zeros(1, 1, 8, 64)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        ra.step_fwd(q, q, q, o, lse, 1, False)


def test_python_binding_rejects_mis_shaped_tensors():
    """Shapes are checked from tensor metadata before anything reaches the
    library, so a mis-sized output cannot be written past its end."""
    import torch
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.zeros(*s)
    B, H, C, d, P = 1, 2, 8, 64, 3
    q, kc = bf(B, H, C, d), [bf(B, H, C, d) for _ in range(P)]
    o, lse = f32(B, H, C, d), f32(B, H, C)
    cases = [
        lambda: ra.step_fwd(q, q, q, f32(B, H, C + 1, d), lse, 1, False),
        lambda: ra.step_fwd(q, bf(B, H, C, d), bf(B, H, C + 1, d), o, lse, 1, False),
        lambda: ra.lse_merge(o, f32(B, H, C - 1), o, lse),
        lambda: ra.ring_fwd(q, kc, kc[:2], o, lse, 1, True),
        lambda: ra.ring_fwd(q, kc, kc, o, f32(B, H, 2 * C), 1, True),
        lambda: ra.ring_fwd(q, kc + [bf(B, H, C + 1, d)], kc + [bf(B, H, C, d)], o, lse, 1, True),
        lambda: ra.ring_bwd(q, kc, kc, o, lse, q, o, [f32(B, H, C, d)] * P, [f32(B, H, C, 2 * d)] * P, 1, True),
        # Ulysses over 2 ranks: outputs hold H/2 = 1 head of the 2*C tokens.
        lambda: ra.ulysses_fwd(kc[:2], kc[:2], kc[:2], f32(B, H, 2 * C, d), f32(B, H, 2 * C), 0, True),
        lambda: ra.ulysses_bwd(kc[:2], kc[:2], kc[:2], kc[:2], f32(B, 1, 2 * C, d), f32(B, 1, 2 * C),
                               *([f32(B, 1, C, d)] * 3), 0, True),
        lambda: ra.allgather_fwd(q, kc, kc, f32(B, H, C, d + 1), lse, 1, True),
        lambda: ra.allgather_bwd(q, kc, kc, o, lse, q, o, f32(B, H, C, d), f32(B, H, P * C, d), 1, True),
        lambda: ra.allgather_fwd(bf(H, C, d), kc, kc, o, lse, 1, True),
    ]
    for n, call in enumerate(cases):
        with pytest.raises(ValueError, match="expected"):
            call()


def test_probe_helpers_validation(L):
    """The MFMA probe rejects NULL buffers and empty launches on the host."""
    assert L.ra_device_info(None, None) == RA_ERR_NULL
    assert L.ra_mfma_probe(vp(0), vp(FAKE), vp(FAKE), 1, 1, None) == RA_ERR_NULL
    assert L.ra_mfma_probe(vp(FAKE), vp(FAKE), vp(FAKE), 0, 1, None) == RA_ERR_SHAPE
    assert L.ra_mfma_probe(vp(FAKE), vp(FAKE), vp(FAKE), 4, 0, None) == RA_ERR_SHAPE
    L.ra_fwd_ladder_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
    assert L.ra_fwd_ladder_probe(0, None, vp(FAKE), vp(FAKE), vp(FAKE), 1, 1, 0.1, None) == RA_ERR_NULL
    assert L.ra_fwd_ladder_probe(11, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, 1, 0.1, None) == RA_ERR_SHAPE
    assert L.ra_fwd_ladder_probe(-1, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1, 1, 0.1, None) == RA_ERR_SHAPE
    assert L.ra_fwd_ladder_probe(2, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, 1, 0.1, None) == RA_ERR_SHAPE



def test_c_client_links_and_reports_usage():
    """ra_client (csrc/ra_client.c) is plain C11 against include/ra.h: it
    links against libra.so and the HIP runtime, and without arguments prints
    its usage and exits with status 2 before touching the GPU."""
    import subprocess
    client = os.path.join(ROOT, "long_context_exact_step_amd", "ra_client")
    if not os.path.exists(client):
        pytest.skip("ra_client is not built (__graft_entry__.build() builds it)")
    r = subprocess.run([client], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "usage: ra_client IN OUT" in r.stderr
