"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare per tensor with
max|gpu - ref| / max|ref| (the tolerance metric of the method's description:
1e-4 for fp32 io, 2e-2 for bf16 / fp16 io)."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from gdr_workloads import WORKLOADS, Workload, head_subset, make_inputs, scaled  # noqa: F401

OUTS = ("dq", "dk", "dv", "dg", "db", "dh0")


def tolerance(w: Workload) -> float:
    return 1e-4 if w.io_dtype == torch.float32 else 2e-2


def run_gpu(inp: dict, with_h0=True, with_dht=True, workspace=None):
    import chunked_gated_delta_gdr_amd as gdr
    dev = "cuda"
    w = inp["workload"]
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"],
                  h0=t["h0"] if with_h0 else None, dht=t["dht"] if with_dht else None,
                  cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk,
                  workspace=workspace)
    torch.cuda.synchronize()
    return dict(zip(OUTS, [o.detach().cpu() for o in out]))


def run_oracle(inp: dict, with_h0=True, with_dht=True, chunk=0):
    w = inp["workload"]
    return oracle.run(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"],
                      inp["h0"] if with_h0 else None, inp["dht"] if with_dht else None,
                      inp["cu_seqlens"], inp["scale"], w.gate, chunk=chunk)


def real_token_mask(inp: dict) -> np.ndarray:
    """[B, T] bool: tokens that belong to a sequence (all, unless varlen)."""
    w = inp["workload"]
    m = np.ones((w.B, w.T), dtype=bool)
    cu = inp["cu_seqlens"]
    if cu is not None:
        m[:] = False
        c = cu.cpu().numpy()
        m[0, c[0]:c[-1]] = True
    return m


def rel_errors(gpu: dict, ref: dict, mask: np.ndarray | None = None, hks=None, hv=None) -> dict:
    errs = {}
    for name in OUTS:
        g = gpu[name].double().numpy()
        r = ref[name]
        if hks is not None:
            g = g[:, :, hks] if name in ("dq", "dk") else (g[:, hv] if name == "dh0" else g[:, :, hv])
        if mask is not None and name != "dh0":
            g = g[mask]
            r = r[mask]
        denom = np.abs(r).max()
        errs[name] = float(np.abs(g - r).max() / denom) if denom > 0 else float(np.abs(g).max())
        if not np.all(np.isfinite(g)):
            errs[name] = float("inf")
    return errs


def parity(w: Workload, hks=None, with_h0=True, with_dht=True):
    """Relative error per output of the HIP path vs the oracle for workload w
    (optionally only q/k heads ``hks`` and their value heads)."""
    inp = make_inputs(w)
    gpu = run_gpu(inp, with_h0, with_dht)
    if hks is None:
        ref = run_oracle(inp, with_h0, with_dht)
        return rel_errors(gpu, ref, real_token_mask(inp))
    sub, hv = head_subset(inp, hks)
    ref = run_oracle(sub, with_h0, with_dht)
    return rel_errors(gpu, ref, real_token_mask(inp), hks=hks, hv=hv)


def varlen_with_empty_sequences() -> dict:
    """Packed T = 128 with sequence lengths [0, 37, 0, 0, 90, 1, 0] (K = V = 64,
    bf16, per-channel gate); h0 and dht drawn per sequence (seed 41)."""
    w = scaled(WORKLOADS["kda_fixed_h16"], B=1, T=128, H=2, Hg=2, K=64, V=64, seed=41)
    inp = make_inputs(w)
    gen = torch.Generator().manual_seed(41)
    inp["cu_seqlens"] = torch.tensor([0, 0, 37, 37, 37, 127, 128, 128], dtype=torch.int32)
    inp["h0"] = torch.randn(7, 2, 64, 64, generator=gen) * 0.1
    inp["dht"] = torch.randn(7, 2, 64, 64, generator=gen) * 0.1
    return inp


def report(label: str, errs: dict, tol: float) -> None:
    """Print the observed max relative error per output (and, when the
    environment names a file in GDR_PARITY_LOG, append it there as a JSON line),
    so that every parity margin against its bar is on record."""
    line = f"parity {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (bar {tol:g})"
    print(line, flush=True)
    path = os.environ.get("GDR_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, "tol": tol, "errs": errs}) + "\n")


def one_reference_split(w: Workload, guard: float) -> tuple[int, int]:
    """(chunk, head) items on each side of the preparation kernel's
    one-reference bound: max over rows r and channels of |G_r - G_last / 2|,
    with G the chunk-local cumsum of the raw gate, at most `guard` or not.
    Computed from the seeded inputs on the host (fixed-length workloads)."""
    g = make_inputs(w)["g"].double()
    if g.dim() == 3:
        g = g.unsqueeze(-1)
    fast = slow = 0
    for b in range(g.shape[0]):
        for c0 in range(0, g.shape[1], w.chunk):
            G = g[b, c0:c0 + w.chunk].cumsum(0)
            dev = (G - 0.5 * G[-1:]).abs().amax(dim=(0, 2))
            fast += int((dev <= guard).sum())
            slow += int((dev > guard).sum())
    return fast, slow
