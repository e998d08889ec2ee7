"""One GPU's share of Ring Attention on MI355X (gfx950): Python binding.

Thin ctypes marshalling over libra.so (include/ra.h).  Every step of the
path runs in the library's HIP kernels; this module only turns torch tensors
into device pointers and streams.  There is no fallback: if libra.so is
missing, every call raises.

    import long_context_exact_step_amd as ra
    ra.ring_fwd(q, k_chunks, v_chunks, o, lse, rank=3, causal=True)
"""

import ctypes
import math
import os

__all__ = [
    "RAError", "lib", "version", "step_fwd", "lse_merge", "ring_fwd", "ring_bwd",
    "workspace_bytes", "ring_bwd_noalloc", "NOALLOC_MAX_ROWS", "RING_RESIDENT", "RING_DOUBLE_BUFFER", "LIB_PATH", "trace_begin", "trace_end",
    "ulysses_fwd", "ulysses_bwd", "ulysses_workspace_bytes",
    "allgather_fwd", "allgather_bwd", "allgather_workspace_bytes",
    "TRACE_KINDS", "device_info", "mfma_probe", "fwd_ladder_probe",
]

# ra_trace_kind values (include/ra.h).
TRACE_KINDS = {1: "fwd_diag", 2: "fwd_full", 3: "merge", 4: "bwd_rowdot", 5: "bwd_zero",
               6: "bwd_dq_diag", 7: "bwd_dq_full", 8: "bwd_dkdv_diag", 9: "bwd_dkdv_full"}

# RA_LIB_PATH may name another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libra.so.
LIB_PATH = os.environ.get("RA_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")
RING_RESIDENT = 0
NOALLOC_MAX_ROWS = 1 << 21  # RA_NOALLOC_MAX_ROWS (include/ra.h)
RING_DOUBLE_BUFFER = 1
RING_FUSED = 2
_MODES = {"resident": RING_RESIDENT, "double_buffer": RING_DOUBLE_BUFFER, "fused": RING_FUSED,
          RING_RESIDENT: RING_RESIDENT, RING_DOUBLE_BUFFER: RING_DOUBLE_BUFFER, RING_FUSED: RING_FUSED}

_lib = None


class RAError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{detail} (status {status})")
        self.status = status
        self.detail = detail


def lib():
    """The loaded libra.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m long_context_exact_step_amd.build` "
                "(or __graft_entry__.build()) first. There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        vpp = ctypes.POINTER(ctypes.c_void_p)
        L.ra_version.restype = i
        L.ra_version.argtypes = []
        L.ra_status_string.restype = ctypes.c_char_p
        L.ra_status_string.argtypes = [i]
        L.ra_last_error.restype = ctypes.c_char_p
        L.ra_last_error.argtypes = []
        L.ra_step_fwd.restype = i
        L.ra_step_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.ra_lse_merge.restype = i
        L.ra_lse_merge.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.ra_ring_workspace_bytes.restype = sz
        L.ra_ring_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.ra_ring_fwd.restype = i
        L.ra_ring_fwd.argtypes = [vp, vpp, vpp, i, vp, vp, i, i, f, i, i, i, i, i, vp, sz, vp, vp]
        L.ra_ring_bwd.restype = i
        L.ra_ring_bwd.argtypes = [vp, vpp, vpp, i, vp, vp, vp, vp, vpp, vpp, i, i, f, i, i, i, i, vp, sz, vp]
        L.ra_step_fwd_gqa.restype = i
        L.ra_step_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.ra_ring_workspace_bytes_gqa.restype = sz
        L.ra_ring_workspace_bytes_gqa.argtypes = [i, i, i, i, i, i, i, i]
        L.ra_ring_fwd_gqa.restype = i
        L.ra_ring_fwd_gqa.argtypes = [vp, vpp, vpp, i, vp, vp, i, i, f, i, i, i, i, i, i, vp, sz, vp, vp]
        L.ra_ring_bwd_gqa.restype = i
        L.ra_ring_bwd_gqa.argtypes = [vp, vpp, vpp, i, vp, vp, vp, vp, vpp, vpp, i, i, f, i, i, i, i, i, vp, sz, vp]
        L.ra_ring_bwd_noalloc.restype = i
        L.ra_ring_bwd_noalloc.argtypes = [vp, vpp, vpp, i, vp, vp, vp, vp, vpp, vpp, i, i, f, i, i, i, i, i, vp]
        L.ra_ulysses_workspace_bytes.restype = sz
        L.ra_ulysses_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.ra_ulysses_bwd.restype = i
        L.ra_ulysses_bwd.argtypes = [vpp, vpp, vpp, vpp, i, vp, vp, vp, vp, vp, i, i, f, i, i, i, i, vp, sz, vp]
        L.ra_ulysses_fwd.restype = i
        L.ra_allgather_workspace_bytes.restype = sz
        L.ra_allgather_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.ra_allgather_fwd.restype = i
        L.ra_allgather_fwd.argtypes = [vp, vpp, vpp, i, vp, vp, i, i, f, i, i, i, i, i, vp, sz, vp]
        L.ra_allgather_bwd.restype = i
        L.ra_allgather_bwd.argtypes = [vp, vpp, vpp, i, vp, vp, vp, vp, vp, vp, i, i, f, i, i, i, i, i, vp, sz, vp]
        L.ra_ulysses_fwd.argtypes = [vpp, vpp, vpp, i, vp, vp, i, i, f, i, i, i, i, vp, sz, vp]
        L.ra_trace_begin.restype = i
        L.ra_trace_begin.argtypes = [vpp, vpp, ctypes.POINTER(ctypes.c_int), i]
        L.ra_trace_end.restype = i
        L.ra_trace_end.argtypes = []
        L.ra_device_info.restype = i
        L.ra_device_info.argtypes = [ctypes.POINTER(i), ctypes.POINTER(i)]
        L.ra_mfma_probe.restype = i
        L.ra_mfma_probe.argtypes = [vp, vp, vp, i, i, vp]
        L.ra_fwd_ladder_probe.restype = i
        L.ra_fwd_ladder_probe.argtypes = [i, vp, vp, vp, vp, i, i, f, vp]
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        L = lib()
        raise RAError(status, f"{L.ra_status_string(status).decode()}: {L.ra_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for n, t in enumerate(ts):
        arr[n] = None if t is None else t.data_ptr()
    return arr


def _stream(stream, like):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _bhsd(t, name):
    """(B, H, S, d) of a 4-d tensor."""
    if t.dim() != 4:
        raise ValueError(f"{name}: expected a [B, H, S, d] tensor, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _chunks(ts, shape, name):
    """Every chunk of a list has `shape`; returns the count."""
    if len(ts) < 1:
        raise ValueError(f"{name}: no chunks")
    for n, t in enumerate(ts):
        if t is not None:
            _shape(t, shape, f"{name}[{n}]")
    return len(ts)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dim() != (3 if name.startswith("lse") else 4):
        raise ValueError(f"{name}: wrong rank {t.dim()}")


def version():
    return lib().ra_version()


def step_fwd(q, k, v, o_partial, lse_partial, step, causal, scale=None, stream=None):
    """ra_step_fwd: one ring step's normalised partial and its lse.  k and v
    may carry fewer heads than q (grouped-query attention, ra_step_fwd_gqa)."""
    import torch
    B, H, Sq, d = _bhsd(q, "q")
    _, Hk, Sk, _ = _bhsd(k, "k")
    _shape(k, (B, Hk, Sk, d), "k"); _shape(v, (B, Hk, Sk, d), "v")
    _shape(o_partial, (B, H, Sq, d), "o_partial"); _shape(lse_partial, (B, H, Sq), "lse_partial")
    _need(q, torch.bfloat16, "q"); _need(k, torch.bfloat16, "k"); _need(v, torch.bfloat16, "v")
    _need(o_partial, torch.float32, "o_partial"); _need(lse_partial, torch.float32, "lse_partial")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (int(step), int(bool(causal)), _stream(stream, q))
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(o_partial), _ptr(lse_partial))
    if Hk == H:
        _check(lib().ra_step_fwd(*ptrs, B, H, Sq, Sk, d, scale, *args))
    else:
        _check(lib().ra_step_fwd_gqa(*ptrs, B, H, Hk, Sq, Sk, d, scale, *args))


def lse_merge(o, lse, o_partial, lse_partial, stream=None):
    """ra_lse_merge: fold (o_partial, lse_partial) into (o, lse) in place."""
    import torch
    B, H, S, d = _bhsd(o, "o")
    _shape(o_partial, (B, H, S, d), "o_partial")
    _shape(lse, (B, H, S), "lse"); _shape(lse_partial, (B, H, S), "lse_partial")
    for t, n in ((o, "o"), (o_partial, "o_partial")):
        _need(t, torch.float32, n)
    for t, n in ((lse, "lse"), (lse_partial, "lse_partial")):
        _need(t, torch.float32, n)
    _check(lib().ra_lse_merge(_ptr(o), _ptr(lse), _ptr(o_partial), _ptr(lse_partial),
                              B, H, S, d, _stream(stream, o)))


def workspace_bytes(P, B, H, C, d, ring_mode="double_buffer", bwd=False, H_kv=None):
    """ra_ring_workspace_bytes (ra_ring_workspace_bytes_gqa when H_kv differs from H)."""
    if H_kv is None or H_kv == H:
        return int(lib().ra_ring_workspace_bytes(P, B, H, C, d, _MODES[ring_mode], int(bool(bwd))))
    return int(lib().ra_ring_workspace_bytes_gqa(P, B, H, H_kv, C, d, _MODES[ring_mode], int(bool(bwd))))


def ring_fwd(q, k_chunks, v_chunks, o, lse, rank, causal, scale=None, ring_mode="double_buffer",
             workspace=None, stream=None, copy_stream=None):
    """ra_ring_fwd: rank's whole ring walk; overwrites (o, lse).  The chunks
    may carry fewer heads than q (grouped-query attention, ra_ring_fwd_gqa).

    workspace: a uint8 GPU tensor of at least workspace_bytes(...) bytes (only
    for ring_mode "double_buffer"); allocated here if not given.
    """
    import torch
    B, H, C, d = _bhsd(q, "q")
    Hk = _bhsd(k_chunks[0], "k_chunks[0]")[1]
    P = _chunks(k_chunks, (B, Hk, C, d), "k_chunks")
    if _chunks(v_chunks, (B, Hk, C, d), "v_chunks") != P:
        raise ValueError(f"v_chunks: {len(v_chunks)} chunks, expected {P} like k_chunks")
    _shape(o, (B, H, C, d), "o"); _shape(lse, (B, H, C), "lse")
    _need(q, torch.bfloat16, "q")
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    for n, t in enumerate(list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    mode = _MODES[ring_mode]
    need = workspace_bytes(P, B, H, C, d, mode, False, H_kv=Hk)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ka, va = _ptr_array(k_chunks), _ptr_array(v_chunks)
    cs = None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    head = (_ptr(q), ka, va, P, _ptr(o), _ptr(lse), int(rank), int(bool(causal)), scale, B, H)
    tail = (C, d, mode, _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream, q), cs)
    if Hk == H:
        _check(lib().ra_ring_fwd(*head, *tail))
    else:
        _check(lib().ra_ring_fwd_gqa(*head, Hk, *tail))
    return workspace


def ring_bwd(q, k_chunks, v_chunks, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, scale=None,
             workspace=None, stream=None):
    """ra_ring_bwd: rank's backward walk; dq overwritten, dk/dv chunks += .
    The chunks and their gradients may carry fewer heads than q (grouped-query
    attention, ra_ring_bwd_gqa)."""
    import torch
    B, H, C, d = _bhsd(q, "q")
    Hk = _bhsd(k_chunks[0], "k_chunks[0]")[1]
    P = _chunks(k_chunks, (B, Hk, C, d), "k_chunks")
    for ts, n in ((v_chunks, "v_chunks"), (dk_chunks, "dk_chunks"), (dv_chunks, "dv_chunks")):
        if _chunks(ts, (B, Hk, C, d), n) != P:
            raise ValueError(f"{n}: {len(ts)} chunks, expected {P}")
    for t, n in ((o, "o"), (dO, "dO"), (dq, "dq")):
        _shape(t, (B, H, C, d), n)
    _shape(lse, (B, H, C), "lse")
    _need(q, torch.bfloat16, "q"); _need(dO, torch.bfloat16, "dO")
    _need(o, torch.float32, "o"); _need(lse, torch.float32, "lse"); _need(dq, torch.float32, "dq")
    for n, t in enumerate(list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    for n, t in enumerate(list(dk_chunks) + list(dv_chunks)):
        if t is not None:
            _need(t, torch.float32, f"grad_chunk{n}")
    need = workspace_bytes(P, B, H, C, d, "resident", True, H_kv=Hk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    head = (_ptr(q), _ptr_array(k_chunks), _ptr_array(v_chunks), P, _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
            _ptr_array(dk_chunks), _ptr_array(dv_chunks), int(rank), int(bool(causal)), scale, B, H)
    tail = (C, d, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q))
    if Hk == H:
        _check(lib().ra_ring_bwd(*head, *tail))
    else:
        _check(lib().ra_ring_bwd_gqa(*head, Hk, *tail))
    return workspace


def ring_bwd_noalloc(q, k_chunks, v_chunks, o, lse, dO, dq, dk_chunks, dv_chunks, rank, causal, scale=None,
                     stream=None):
    """ra_ring_bwd_noalloc: ring_bwd without a workspace (the library's
    static device scratch holds the row terms; B*H*C <= NOALLOC_MAX_ROWS).
    Calls that overlap on one device race on that scratch."""
    import torch
    B, H, C, d = _bhsd(q, "q")
    Hk = _bhsd(k_chunks[0], "k_chunks[0]")[1]
    P = _chunks(k_chunks, (B, Hk, C, d), "k_chunks")
    for ts, n in ((v_chunks, "v_chunks"), (dk_chunks, "dk_chunks"), (dv_chunks, "dv_chunks")):
        if _chunks(ts, (B, Hk, C, d), n) != P:
            raise ValueError(f"{n}: {len(ts)} chunks, expected {P}")
    for t, n in ((o, "o"), (dO, "dO"), (dq, "dq")):
        _shape(t, (B, H, C, d), n)
    _shape(lse, (B, H, C), "lse")
    _need(q, torch.bfloat16, "q"); _need(dO, torch.bfloat16, "dO")
    _need(o, torch.float32, "o"); _need(lse, torch.float32, "lse"); _need(dq, torch.float32, "dq")
    for n, t in enumerate(list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    for n, t in enumerate(list(dk_chunks) + list(dv_chunks)):
        if t is not None:
            _need(t, torch.float32, f"grad_chunk{n}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().ra_ring_bwd_noalloc(_ptr(q), _ptr_array(k_chunks), _ptr_array(v_chunks), P, _ptr(o), _ptr(lse),
                                     _ptr(dO), _ptr(dq), _ptr_array(dk_chunks), _ptr_array(dv_chunks), int(rank),
                                     int(bool(causal)), scale, B, H, Hk, C, d, _stream(stream, q)))


def ulysses_workspace_bytes(P, B, H, C, d, bwd=False):
    return int(lib().ra_ulysses_workspace_bytes(P, B, H, C, d, int(bool(bwd))))


def ulysses_fwd(q_chunks, k_chunks, v_chunks, o, lse, rank, causal, scale=None, workspace=None, stream=None):
    """ra_ulysses_fwd: one rank's share of head-partitioned (Ulysses) sequence
    parallelism.  q/k/v_chunks: P tensors [B,H,C,d] bf16 (the sequence split in
    chunks); o [B,H/P,P*C,d], lse [B,H/P,P*C] fp32 receive attention of the
    rank's heads over the whole sequence."""
    import torch
    B, H, C, d = _bhsd(q_chunks[0], "q_chunks[0]")
    P = _chunks(q_chunks, (B, H, C, d), "q_chunks")
    for ts, n in ((k_chunks, "k_chunks"), (v_chunks, "v_chunks")):
        if _chunks(ts, (B, H, C, d), n) != P:
            raise ValueError(f"{n}: {len(ts)} chunks, expected {P}")
    if H % P:
        raise ValueError(f"H={H} heads do not split over P={P} ranks")
    _shape(o, (B, H // P, P * C, d), "o"); _shape(lse, (B, H // P, P * C), "lse")
    for n, t in enumerate(list(q_chunks) + list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    need = ulysses_workspace_bytes(P, B, H, C, d)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=o.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().ra_ulysses_fwd(_ptr_array(q_chunks), _ptr_array(k_chunks), _ptr_array(v_chunks), P, _ptr(o),
                                _ptr(lse), int(rank), int(bool(causal)), scale, B, H, C, d, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream, o)))
    return workspace


def ulysses_bwd(q_chunks, k_chunks, v_chunks, dO_chunks, o, lse, dq, dk, dv, rank, causal, scale=None,
                workspace=None, stream=None):
    """ra_ulysses_bwd: the Ulysses share's backward.  dO_chunks split by
    sequence like q_chunks; o, lse from ulysses_fwd; dq, dk, dv [B,H/P,P*C,d]
    fp32 are overwritten."""
    import torch
    B, H, C, d = _bhsd(q_chunks[0], "q_chunks[0]")
    P = _chunks(q_chunks, (B, H, C, d), "q_chunks")
    for ts, n in ((k_chunks, "k_chunks"), (v_chunks, "v_chunks"), (dO_chunks, "dO_chunks")):
        if _chunks(ts, (B, H, C, d), n) != P:
            raise ValueError(f"{n}: {len(ts)} chunks, expected {P}")
    if H % P:
        raise ValueError(f"H={H} heads do not split over P={P} ranks")
    for t, n in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _shape(t, (B, H // P, P * C, d), n)
    _shape(lse, (B, H // P, P * C), "lse")
    for n, t in enumerate(list(q_chunks) + list(k_chunks) + list(v_chunks) + list(dO_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    for t, n in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.float32, n)
    _need(lse, torch.float32, "lse")
    need = ulysses_workspace_bytes(P, B, H, C, d, bwd=True)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=o.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().ra_ulysses_bwd(_ptr_array(q_chunks), _ptr_array(k_chunks), _ptr_array(v_chunks),
                                _ptr_array(dO_chunks), P, _ptr(o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                int(rank), int(bool(causal)), scale, B, H, C, d, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream, o)))
    return workspace


def allgather_workspace_bytes(P, B, H, C, d, H_kv=None, bwd=False):
    return int(lib().ra_allgather_workspace_bytes(P, B, H, H if H_kv is None else H_kv, C, d, int(bool(bwd))))


def allgather_fwd(q, k_chunks, v_chunks, o, lse, rank, causal, scale=None, workspace=None, stream=None):
    """ra_allgather_fwd: one rank's share of all-gather sequence parallelism.
    q [B,H,C,d] bf16 (the rank's chunk); k/v_chunks: P tensors [B,H_kv,C,d]
    bf16; o [B,H,C,d], lse [B,H,C] fp32 receive attention over the gathered
    sequence."""
    import torch
    B, H, C, d = _bhsd(q, "q")
    Hk = _bhsd(k_chunks[0], "k_chunks[0]")[1]
    P = _chunks(k_chunks, (B, Hk, C, d), "k_chunks")
    if _chunks(v_chunks, (B, Hk, C, d), "v_chunks") != P:
        raise ValueError(f"v_chunks: {len(v_chunks)} chunks, expected {P} like k_chunks")
    _shape(o, (B, H, C, d), "o"); _shape(lse, (B, H, C), "lse")
    _need(q, torch.bfloat16, "q")
    for n, t in enumerate(list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    need = allgather_workspace_bytes(P, B, H, C, d, H_kv=Hk)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().ra_allgather_fwd(_ptr(q), _ptr_array(k_chunks), _ptr_array(v_chunks), P, _ptr(o), _ptr(lse),
                                  int(rank), int(bool(causal)), scale, B, H, Hk, C, d, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream, q)))
    return workspace


def allgather_bwd(q, k_chunks, v_chunks, o, lse, dO, dq, dk, dv, rank, causal, scale=None, workspace=None,
                  stream=None):
    """ra_allgather_bwd: the all-gather share's backward.  o, lse from
    allgather_fwd; dq [B,H,C,d] and dk, dv [B,H_kv,P*C,d] fp32 are
    overwritten (dk, dv: the gathered sequence's gradient from this rank)."""
    import torch
    B, H, C, d = _bhsd(q, "q")
    Hk = _bhsd(k_chunks[0], "k_chunks[0]")[1]
    P = _chunks(k_chunks, (B, Hk, C, d), "k_chunks")
    if _chunks(v_chunks, (B, Hk, C, d), "v_chunks") != P:
        raise ValueError(f"v_chunks: {len(v_chunks)} chunks, expected {P} like k_chunks")
    for t, n in ((o, "o"), (dO, "dO"), (dq, "dq")):
        _shape(t, (B, H, C, d), n)
    _shape(lse, (B, H, C), "lse")
    for t, n in ((dk, "dk"), (dv, "dv")):
        _shape(t, (B, Hk, P * C, d), n)
    _need(q, torch.bfloat16, "q"); _need(dO, torch.bfloat16, "dO")
    for n, t in enumerate(list(k_chunks) + list(v_chunks)):
        _need(t, torch.bfloat16, f"chunk{n}")
    for t, n in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.float32, n)
    need = allgather_workspace_bytes(P, B, H, C, d, H_kv=Hk, bwd=True)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().ra_allgather_bwd(_ptr(q), _ptr_array(k_chunks), _ptr_array(v_chunks), P, _ptr(o), _ptr(lse),
                                  _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), int(rank), int(bool(causal)), scale,
                                  B, H, Hk, C, d, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream, q)))
    return workspace


def trace_begin(start_events, end_events, kinds):
    """ra_trace_begin: start_events/end_events are raw hipEvent_t handles
    (ints, timing enabled); kinds is a ctypes c_int array of the same length.
    The arrays must stay alive until trace_end()."""
    n = len(start_events)
    sa = (ctypes.c_void_p * n)(*start_events)
    ea = (ctypes.c_void_p * n)(*end_events)
    _check(lib().ra_trace_begin(sa, ea, kinds, n))
    return sa, ea


def trace_end():
    """ra_trace_end: number of launches made while tracing was armed."""
    return int(lib().ra_trace_end())


def device_info():
    """ra_device_info: (compute units, maximum engine clock in kHz) of the
    current device."""
    cu, clk = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().ra_device_info(ctypes.byref(cu), ctypes.byref(clk)))
    return cu.value, clk.value


def mfma_probe(operands, sink, clocks, blocks, iters, stream=None):
    """ra_mfma_probe: dense bf16 MFMA throughput probe.  operands: >= 16384
    bytes of bf16 data; sink: float32, >= blocks * 512 values; clocks: int64,
    >= 2 values (shader cycles, 100 MHz reference ticks of wave 0's loop)."""
    import torch
    if operands.dtype != torch.bfloat16 or operands.numel() * 2 < 16384:
        raise ValueError("operands: expected >= 8192 bf16 values")
    if sink.dtype != torch.float32 or sink.numel() < blocks * 512:
        raise ValueError(f"sink: expected >= {blocks * 512} float32 values")
    if clocks.dtype != torch.int64 or clocks.numel() < 2:
        raise ValueError("clocks: expected >= 2 int64 values")
    for t, n in ((operands, "operands"), (sink, "sink"), (clocks, "clocks")):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{n}: must be a contiguous GPU tensor")
    _check(lib().ra_mfma_probe(_ptr(operands), _ptr(sink), _ptr(clocks), int(blocks), int(iters),
                               _stream(stream, sink)))



def fwd_ladder_probe(level, operands, tiles, sink, clocks, blocks, iters, c, stream=None):
    """ra_fwd_ladder_probe: the forward kernel's instruction stream rebuilt
    on synthetic data up to `level` (0..5: two waves per SIMD, 32 rows each;
    6..10: one wave per SIMD with 64 rows).  operands: >= 10240 bf16 values;
    tiles: >= 524288 bf16 values; sink: float32, >= blocks * 512; clocks:
    int64, >= 2.  The same matrix work at every level: 4194304 * iters flop
    per 32 query rows (8 such row groups per block)."""
    import torch
    if operands.dtype != torch.bfloat16 or operands.numel() * 2 < 20480:
        raise ValueError("operands: expected >= 10240 bf16 values")
    if tiles.dtype != torch.bfloat16 or tiles.numel() * 2 < (1 << 20):
        raise ValueError("tiles: expected >= 524288 bf16 values")
    if sink.dtype != torch.float32 or sink.numel() < blocks * 512:
        raise ValueError(f"sink: expected >= {blocks * 512} float32 values")
    if clocks.dtype != torch.int64 or clocks.numel() < 2:
        raise ValueError("clocks: expected >= 2 int64 values")
    for t, n in ((operands, "operands"), (tiles, "tiles"), (sink, "sink"), (clocks, "clocks")):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{n}: must be a contiguous GPU tensor")
    _check(lib().ra_fwd_ladder_probe(int(level), _ptr(operands), _ptr(tiles), _ptr(sink), _ptr(clocks), int(blocks),
                                     int(iters), float(c), _stream(stream, sink)))
