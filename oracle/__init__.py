"""fp64 CPU oracle for the gated delta-rule backward -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package. It shares no code with the HIP path (chunked_gated_delta_gdr_amd) and
never imports it. The arithmetic lives in gdr_oracle.c (token-by-token
recurrence and its hand-derived reverse); this file only builds that library,
converts arrays to fp64 and calls it through ctypes.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(central finite differences, an independent chunked WY forward, closed forms at
beta = 0, the scalar-gate / per-channel-gate equivalence, GQA and varlen
decompositions, linearity in (do, dht)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdr_oracle.c into libgdr_oracle.so (plain gcc, OpenMP)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.gdr_oracle_run.restype = ctypes.c_int
        lib.gdr_oracle_run.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
            P, ctypes.c_int32,
            P, P, P, P, P, P, P, P,
            P, P, P, P, P, P, P, P,
            ctypes.c_int32, P, P]
        lib.gdr_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle will use (OMP_NUM_THREADS or all cores)."""
    return int(_load().gdr_oracle_threads())


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast the already-rounded values
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run(q, k, v, g, beta, do=None, h0=None, dht=None, cu_seqlens=None, scale=None,
        gate: str = "kda", backward: bool = True, forward_out: bool = False,
        chunk: int = 0) -> dict:
    """Run the oracle on (already io-rounded) inputs; everything is upcast to fp64.

    Shapes: q, k [B,T,Hg,K]; v, do [B,T,H,V]; g [B,T,H,K] ("kda") or [B,T,H]
    ("gdn"), raw log2 gate per token; beta [B,T,H]; h0, dht [N,H,K,V] or None
    (zero); cu_seqlens [N+1] int (varlen, B == 1) or None.
    Returns fp64 numpy arrays: dq, dk (q/k shape, summed over GQA groups), dv,
    dg, db, dh0 when ``backward``; o [B,T,H,V] and ht [N,H,K,V] when
    ``forward_out``; h_chunks / dh_chunks [chunks,H,K,V] when ``chunk`` > 0.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    do, h0, dht = _f64(do), _f64(h0), _f64(dht)
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    scalar = {"kda": 0, "gdn": 1}[gate]
    expect_g = (B, T, H) if scalar else (B, T, H, K)
    if g.shape != expect_g:
        raise ValueError(f"g shape {g.shape} != {expect_g}")
    if scale is None:
        scale = K ** -0.5
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int32))
        N = len(cu) - 1
        if B != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("bad cu_seqlens")
    out = {}
    if backward:
        if do is None:
            raise ValueError("backward needs do")
        out["dq"] = np.zeros_like(q)
        out["dk"] = np.zeros_like(q)
        out["dv"] = np.zeros((B, T, H, V))
        out["dg"] = np.zeros_like(g)
        out["db"] = np.zeros((B, T, H))
        out["dh0"] = np.zeros((N, H, K, V))
    if forward_out:
        out["o"] = np.zeros((B, T, H, V))
        out["ht"] = np.zeros((N, H, K, V))
    if chunk > 0:
        lens = np.diff(cu) if cu is not None else np.full(B, T)
        nch = int(sum((int(L) + chunk - 1) // chunk for L in lens))
        out["h_chunks"] = np.zeros((nch, H, K, V))
        if backward:
            out["dh_chunks"] = np.zeros((nch, H, K, V))
    if do is None:
        do = np.zeros((B, T, H, V))
    rc = _load().gdr_oracle_run(
        B, T, H, Hg, K, V, scalar, float(scale), _ptr(cu), N,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht),
        _ptr(out.get("dq")), _ptr(out.get("dk")), _ptr(out.get("dv")),
        _ptr(out.get("dg")), _ptr(out.get("db")), _ptr(out.get("dh0")),
        _ptr(out.get("o")), _ptr(out.get("ht")),
        int(chunk), _ptr(out.get("h_chunks")), _ptr(out.get("dh_chunks")))
    if rc != 0:
        raise RuntimeError("oracle failed (bad arguments or out of memory)")
    return out


def loss(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None,
         gate: str = "kda") -> float:
    """The objective L = sum_t <do_t, o_t> + <dht, S_T> from the oracle's forward."""
    f = run(q, k, v, g, beta, None, h0, None, cu_seqlens, scale, gate,
            backward=False, forward_out=True)
    total = float(np.sum(f["o"] * _f64(do)))
    if dht is not None:
        total += float(np.sum(f["ht"] * _f64(dht)))
    return total
