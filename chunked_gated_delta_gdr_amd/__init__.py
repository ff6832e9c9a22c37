"""Python binding of libgdr.so: the MI355X chunkwise gated delta-rule backward.

Argument marshalling only: every step of the backward runs in the HIP kernels
behind the C ABI (include/gdr.h). torch supplies device memory and the current
stream. There is no fallback: if the library is missing or the tensors are not
on a ROCm device, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["bwd", "bwd_after_fwd", "bwd_from_states", "bwd_fused", "bwd_static", "fwd", "workspace_bytes", "workspace_offsets",
           "library_path", "Desc", "GATE_PER_CHANNEL", "GATE_SCALAR", "GdrError", "STATIC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lib = None

GATE_PER_CHANNEL, GATE_SCALAR = 0, 1
STATIC_SCRATCH_BYTES = 64 << 20   # GDR_STATIC_SCRATCH_BYTES of include/gdr.h
_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
WS_NAMES = ("ctab", "seq_off", "sAqkT", "A", "AT", "w", "wT", "kt", "ktT", "uT", "qsT",
            "glast", "h", "X", "dh", "T")


class GdrError(RuntimeError):
    pass


class Desc(ctypes.Structure):
    """Mirror of gdr_bwd_desc_t."""
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64),
                ("H", ctypes.c_int32), ("Hg", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("sub_chunk", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("state_v_first", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise GdrError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(python -m chunked_gated_delta_gdr_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(Desc)
        lib.gdr_bwd_check.restype = ctypes.c_int
        lib.gdr_bwd_check.argtypes = [D]
        lib.gdr_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_bwd_workspace_bytes.argtypes = [D]
        lib.gdr_bwd_workspace_offsets.restype = ctypes.c_int
        lib.gdr_bwd_workspace_offsets.argtypes = [D, ctypes.POINTER(ctypes.c_size_t), ctypes.c_int]
        lib.gdr_bwd.restype = ctypes.c_int
        lib.gdr_bwd.argtypes = [D] + [P] * 15 + [P, ctypes.c_size_t, P]
        lib.gdr_bwd_with_events.restype = ctypes.c_int
        lib.gdr_bwd_with_events.argtypes = [D] + [P] * 15 + [P, ctypes.c_size_t, P,
                                                              ctypes.POINTER(ctypes.c_void_p)]
        lib.gdr_fwd.restype = ctypes.c_int
        lib.gdr_fwd.argtypes = [D] + [P] * 9 + [P, ctypes.c_size_t, P]
        lib.gdr_bwd_after_fwd.restype = ctypes.c_int
        lib.gdr_bwd_after_fwd.argtypes = [D] + [P] * 14 + [P, ctypes.c_size_t, P]
        lib.gdr_bwd_from_states.restype = ctypes.c_int
        lib.gdr_bwd_from_states.argtypes = [D] + [P] * 9 + [ctypes.c_int64] + [P] * 6 + [P, ctypes.c_size_t, P]
        lib.gdr_bwd_fused.restype = ctypes.c_int
        lib.gdr_bwd_fused.argtypes = [D] + [P] * 15 + [P, ctypes.c_size_t, P]
        lib.gdr_bwd_fused_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_bwd_fused_workspace_bytes.argtypes = [D]
        lib.gdr_bwd_static.restype = ctypes.c_int
        lib.gdr_bwd_static.argtypes = [D] + [P] * 15 + [P]
        lib.gdr_strerror.restype = ctypes.c_char_p
        lib.gdr_strerror.argtypes = [ctypes.c_int]
        lib.gdr_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _err(rc: int) -> GdrError:
    return GdrError(f"gdr error {rc}: {_load().gdr_strerror(rc).decode()}")


def make_desc(B, T, H, Hg, K, V, chunk=64, n_seqs=0, gate=GATE_PER_CHANNEL,
              io_dtype=torch.bfloat16, scale=0.0, sub_chunk=16, state_v_first=False) -> Desc:
    return Desc(B=B, T=T, H=H, Hg=Hg, K=K, V=V, chunk=chunk, sub_chunk=sub_chunk,
                n_seqs=n_seqs, gate=gate, io_dtype=_DTYPES.get(io_dtype, -1)
                if isinstance(io_dtype, torch.dtype) else int(io_dtype), scale=scale,
                state_v_first=int(bool(state_v_first)))


def check(desc: Desc) -> int:
    return int(_load().gdr_bwd_check(ctypes.byref(desc)))


def workspace_bytes(desc: Desc) -> int:
    n = int(_load().gdr_bwd_workspace_bytes(ctypes.byref(desc)))
    if n == 0:
        raise _err(check(desc))
    return n


def workspace_offsets(desc: Desc) -> dict:
    arr = (ctypes.c_size_t * (len(WS_NAMES) + 1))()
    rc = _load().gdr_bwd_workspace_offsets(ctypes.byref(desc), arr, len(WS_NAMES) + 1)
    if rc != 0:
        raise _err(rc)
    out = {n: int(arr[i]) for i, n in enumerate(WS_NAMES)}
    out["total"] = int(arr[len(WS_NAMES)])
    return out


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise GdrError(f"{name} must be on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise GdrError(f"{name} is on {t.device}, the inputs on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


STAGES = ("chunk_table", "prep", "sweep", "chunk_bwd")


def _workspace(desc: Desc, workspace: Optional[torch.Tensor], device) -> torch.Tensor:
    """The caller's workspace after checks, or a new one of the required size."""
    nbytes = workspace_bytes(desc)
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 torch tensor")
    if workspace.device != device:
        raise GdrError(f"workspace is on {workspace.device}, the inputs on {device}")
    if not workspace.is_contiguous() or workspace.numel() < nbytes:
        raise ValueError(f"workspace must be contiguous with >= {nbytes} bytes")
    return workspace


def _grad_outputs(q, k, v, g, beta, N, H, K, V, out):
    """(dq, dk, dv, dg, db, dh0): new tensors, or the caller's after checks."""
    if out is None:
        return (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
                torch.empty_like(beta), torch.empty((N, H, K, V), dtype=torch.float32, device=q.device))
    if len(out) != 6:
        raise ValueError("out: (dq, dk, dv, dg, db, dh0)")
    for name, t, ref in zip(("dq", "dk", "dv", "dg", "db"), out[:5], (q, k, v, g, beta)):
        _need(t, f"out {name}", ref.dtype, ref.shape, q.device)
    _need(out[5], "out dh0", torch.float32, (N, H, K, V), q.device)
    return tuple(out)


def _bwd_desc(q, k, v, g, beta, do, h0, dht, cu_seqlens, scale, chunk_size, state_v_first=False):
    """Checks the backward's inputs; returns (descriptor, N, H, K, V)."""
    io = q.dtype
    if io not in _DTYPES:
        raise TypeError(f"unsupported io dtype {io}")
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    gate = GATE_PER_CHANNEL if g.dim() == 4 else GATE_SCALAR
    n_seqs = 0
    N = B
    dev = q.device
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.shape[0],), dev)
        n_seqs = cu_seqlens.shape[0] - 1
        N = n_seqs
    _need(q, "q", io, (B, T, Hg, K))
    _need(k, "k", io, (B, T, Hg, K), dev)
    _need(v, "v", io, (B, T, H, V), dev)
    _need(do, "do", io, (B, T, H, V), dev)
    _need(beta, "beta", io, (B, T, H), dev)
    _need(g, "g", torch.float32, (B, T, H, K) if gate == GATE_PER_CHANNEL else (B, T, H), dev)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, H, K, V), dev)
    if dht is not None:
        _need(dht, "dht", torch.float32, (N, H, K, V), dev)
    desc = make_desc(B, T, H, Hg, K, V, chunk=chunk_size, n_seqs=n_seqs, gate=gate,
                     io_dtype=io, scale=float(scale) if scale is not None else 0.0,
                     state_v_first=state_v_first)
    rc = check(desc)
    if rc != 0:
        raise _err(rc)
    return desc, N, H, K, V


def bwd(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None,
        chunk_size: int = 64, workspace: Optional[torch.Tensor] = None, out=None,
        stage_events=None, after_fwd: bool = False, state_v_first: bool = False):
    """Backward of the gated delta rule (see include/gdr.h for the definition).

    q, k [B,T,Hg,K]; v, do [B,T,H,V]; beta [B,T,H] (all in one io dtype:
    float32, bfloat16 or float16); g fp32 [B,T,H,K] (per-channel gate) or
    [B,T,H] (scalar gate), raw per-token log2 gate; h0, dht fp32 [N,H,K,V] or
    None; cu_seqlens int32 [N+1] on the device (varlen, B == 1) or None.
    Returns (dq, dk, dv, dg, db, dh0). ``workspace`` (uint8, at least
    workspace_bytes) may be passed to avoid an allocation per call; ``out``
    may hold preallocated outputs in the same order. ``stage_events``: five
    torch.cuda.Event(enable_timing=True), already recorded once, recorded at
    the kernel boundaries (see gdr_bwd_with_events). ``after_fwd``: see
    :func:`bwd_after_fwd`. ``state_v_first``: h0, dht and dh0 hold each state
    transposed, [N,H,V,K] (the same shape, since K == V).
    """
    lib = _load()
    if after_fwd and (h0 is not None or workspace is None or stage_events is not None):
        raise ValueError("after_fwd: pass the forward's workspace, and no h0 or stage_events")
    desc, N, H, K, V = _bwd_desc(q, k, v, g, beta, do, h0, dht, cu_seqlens, scale, chunk_size,
                                 state_v_first)
    workspace = _workspace(desc, workspace, q.device)
    dq, dk, dv, dg, db, dh0 = _grad_outputs(q, k, v, g, beta, N, H, K, V, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(h0), _ptr(do), _ptr(dht), _ptr(cu_seqlens),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0),
            _ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if after_fwd:
        rc = lib.gdr_bwd_after_fwd(*(args[:6] + args[7:]))   # no h0
    elif stage_events is None:
        rc = lib.gdr_bwd(*args)
    else:
        if len(stage_events) != 5 or any(e.cuda_event == 0 for e in stage_events):
            raise ValueError("stage_events: five created (recorded once) timing events")
        evs = (ctypes.c_void_p * 5)(*[e.cuda_event for e in stage_events])
        rc = lib.gdr_bwd_with_events(*args, evs)
    if rc != 0:
        raise _err(rc)
    return dq, dk, dv, dg, db, dh0


def bwd_from_states(q, k, v, g, beta, do, h, dht=None, cu_seqlens=None, scale=None,
                    chunk_size: int = 64, state_v_first: bool = False,
                    workspace: Optional[torch.Tensor] = None, out=None):
    """Backward from the per-chunk states the forward pass saved
    (gdr_bwd_from_states): the forward state sweep is not run.

    ``h`` holds the state before every chunk in the io dtype: [B, NT, H, K, V]
    (fixed length, NT = ceil(T / chunk_size)) or [n_chunks, H, K, V] (chunks of
    all sequences in order; varlen); with ``state_v_first`` the last two axes
    are (V, K), as are dht's and dh0's. Returns what :func:`bwd` returns."""
    lib = _load()
    desc, N, H, K, V = _bwd_desc(q, k, v, g, beta, do, None, dht, cu_seqlens, scale, chunk_size,
                                 state_v_first)
    if not isinstance(h, torch.Tensor):
        raise TypeError("h must be a torch tensor")
    n_h = h.shape[0] * h.shape[1] if h.dim() == 5 else h.shape[0]
    _need(h, "h", q.dtype, (h.shape[0], h.shape[1], H, K, V) if h.dim() == 5 else (n_h, H, K, V), q.device)
    if cu_seqlens is None:
        nt = (q.shape[1] + chunk_size - 1) // chunk_size
        if n_h != q.shape[0] * nt or (h.dim() == 5 and h.shape[:2] != (q.shape[0], nt)):
            raise ValueError(f"h: expected [{q.shape[0]}, {nt}, H, K, V] per-chunk states")
    workspace = _workspace(desc, workspace, q.device)
    dq, dk, dv, dg, db, dh0 = _grad_outputs(q, k, v, g, beta, N, H, K, V, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.gdr_bwd_from_states(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(do), _ptr(dht), _ptr(cu_seqlens), _ptr(h), ctypes.c_int64(n_h),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0),
                                 _ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if rc != 0:
        raise _err(rc)
    return dq, dk, dv, dg, db, dh0


def bwd_fused(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None,
              chunk_size: int = 32, workspace: Optional[torch.Tensor] = None, out=None,
              state_v_first: bool = False):
    """:func:`bwd` through gdr_bwd_fused: one fused reverse kernel per
    (sequence, value head) with the state gradient on chip (chunk 32 only).
    ``workspace`` (uint8) needs gdr_bwd_fused_workspace_bytes bytes."""
    lib = _load()
    desc, N, H, K, V = _bwd_desc(q, k, v, g, beta, do, h0, dht, cu_seqlens, scale, chunk_size,
                                 state_v_first)
    nbytes = int(lib.gdr_bwd_fused_workspace_bytes(ctypes.byref(desc)))
    if nbytes == 0:
        raise GdrError(f"gdr_bwd_fused: unsupported descriptor (chunk {chunk_size}; built for 32)")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or
          workspace.device != q.device or not workspace.is_contiguous() or workspace.numel() < nbytes):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {q.device} with >= {nbytes} bytes")
    dq, dk, dv, dg, db, dh0 = _grad_outputs(q, k, v, g, beta, N, H, K, V, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.gdr_bwd_fused(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(h0), _ptr(do), _ptr(dht), _ptr(cu_seqlens),
                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0),
                           _ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if rc != 0:
        raise _err(rc)
    return dq, dk, dv, dg, db, dh0


def bwd_static(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None,
               chunk_size: int = 64, out=None, state_v_first: bool = False):
    """:func:`bwd` through gdr_bwd_static: no workspace argument, the library's
    fixed per-GPU scratch (STATIC_SCRATCH_BYTES) instead. The C call allocates
    nothing; pass ``out`` (dq, dk, dv, dg, db, dh0) to keep this binding from
    allocating the outputs. Calls that may overlap on one GPU race on the
    scratch (see gdr_bwd_static in include/gdr.h)."""
    lib = _load()
    desc, N, H, K, V = _bwd_desc(q, k, v, g, beta, do, h0, dht, cu_seqlens, scale, chunk_size,
                                 state_v_first)
    dq, dk, dv, dg, db, dh0 = _grad_outputs(q, k, v, g, beta, N, H, K, V, out)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.gdr_bwd_static(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(h0), _ptr(do), _ptr(dht), _ptr(cu_seqlens),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0),
                            ctypes.c_void_p(stream))
    if rc != 0:
        raise _err(rc)
    return dq, dk, dv, dg, db, dh0


def bwd_after_fwd(q, k, v, g, beta, do, workspace: torch.Tensor, dht=None, cu_seqlens=None,
                  scale=None, chunk_size: int = 64, out=None, state_v_first: bool = False):
    """Backward after :func:`fwd`, from the per-chunk states it saved.

    ``workspace`` must be the one a :func:`fwd` call filled, with the same
    q, k, v, g, beta, h0, cu_seqlens, scale and chunk size, unchanged since
    (gdr_bwd_after_fwd in include/gdr.h): only the reverse sweep and the
    gradient kernel run. Returns what :func:`bwd` returns for those inputs.
    """
    return bwd(q, k, v, g, beta, do, dht=dht, cu_seqlens=cu_seqlens, scale=scale,
               chunk_size=chunk_size, workspace=workspace, out=out, after_fwd=True,
               state_v_first=state_v_first)


def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, chunk_size: int = 64,
        workspace: Optional[torch.Tensor] = None, out=None, final_state: bool = True,
        state_v_first: bool = False):
    """Forward of the gated delta rule: returns (o, ht).

    Same inputs as :func:`bwd` (without do, dht). o [B,T,H,V] in the io dtype;
    ht fp32 [N,H,K,V] (None when ``final_state`` is False). ``workspace`` and
    ``out`` (o, ht) may be preallocated.
    """
    lib = _load()
    io = q.dtype
    if io not in _DTYPES:
        raise TypeError(f"unsupported io dtype {io}")
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    gate = GATE_PER_CHANNEL if g.dim() == 4 else GATE_SCALAR
    n_seqs, N = 0, B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.shape[0],), q.device)
        n_seqs = N = cu_seqlens.shape[0] - 1
    _need(q, "q", io, (B, T, Hg, K))
    _need(k, "k", io, (B, T, Hg, K), q.device)
    _need(v, "v", io, (B, T, H, V), q.device)
    _need(beta, "beta", io, (B, T, H), q.device)
    _need(g, "g", torch.float32, (B, T, H, K) if gate == GATE_PER_CHANNEL else (B, T, H), q.device)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, H, K, V), q.device)
    desc = make_desc(B, T, H, Hg, K, V, chunk=chunk_size, n_seqs=n_seqs, gate=gate,
                     io_dtype=io, scale=float(scale) if scale is not None else 0.0,
                     state_v_first=state_v_first)
    rc = check(desc)
    if rc != 0:
        raise _err(rc)
    workspace = _workspace(desc, workspace, q.device)
    if out is None:
        o = torch.empty_like(v)
        ht = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device) if final_state else None
    else:
        if len(out) != 2:
            raise ValueError("out: (o, ht)")
        o, ht = out
        _need(o, "out o", v.dtype, v.shape, q.device)
        if ht is not None:
            _need(ht, "out ht", torch.float32, (N, H, K, V), q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.gdr_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                     _ptr(cu_seqlens), _ptr(o), _ptr(ht), _ptr(workspace),
                     ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if rc != 0:
        raise _err(rc)
    return o, ht
