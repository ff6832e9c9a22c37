"""Seeded synthetic inputs for the gated delta-rule backward.

This module holds no arithmetic of the method itself: it only draws random
tensors, applies the input preparation the workloads describe (L2
normalisation of q/k rows, sigmoid for beta, -softplus for the log2 gate) and
casts to the io dtype. Both the HIP path's tests/bench and the CPU oracle's
tests take their inputs from here; neither side imports the other.

Draw order is fixed: [varlen lengths], q, k, v, g, beta, h0, do, dht, all from
one torch CPU generator seeded with the workload's seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "varlen_lengths", "scaled", "head_subset"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int              # per-sequence length (fixed) or packed total (varlen)
    H: int              # value heads
    Hg: int             # q/k heads (H % Hg == 0)
    K: int
    V: int
    chunk: int
    gate: str           # "kda" (per-channel) or "gdn" (scalar per head)
    io_dtype: torch.dtype
    gate_mult: float    # g = -softplus(N(0,1)) * gate_mult
    h0_std: float       # 0 -> h0 = 0 (zeros are passed, not NULL)
    dht_std: float      # 0 -> dht = 0
    n_seqs: int = 0     # > 0 -> varlen packed, B must be 1
    seed: int = 0
    sub_chunk: int = 16

    @property
    def varlen(self) -> bool:
        return self.n_seqs > 0

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads of the method's benchmark description. Seeds are 0 for all.
WORKLOADS = {
    "tiny_kda_fp32": Workload("tiny_kda_fp32", B=1, T=256, H=2, Hg=2, K=64, V=64,
                              chunk=64, gate="kda", io_dtype=torch.float32,
                              gate_mult=0.5, h0_std=0.0, dht_std=0.0),
    "kda_fixed_h16": Workload("kda_fixed_h16", B=2, T=4096, H=16, Hg=16, K=128, V=128,
                              chunk=64, gate="kda", io_dtype=torch.bfloat16,
                              gate_mult=0.5, h0_std=0.1, dht_std=0.0),
    "gdn_gqa_fp16": Workload("gdn_gqa_fp16", B=4, T=8192, H=32, Hg=16, K=128, V=128,
                             chunk=32, gate="gdn", io_dtype=torch.float16,
                             gate_mult=0.1, h0_std=0.0, dht_std=0.1),
    "kda_varlen": Workload("kda_varlen", B=1, T=32768, H=16, Hg=16, K=128, V=128,
                           chunk=64, gate="kda", io_dtype=torch.bfloat16,
                           gate_mult=0.5, h0_std=0.1, dht_std=0.0, n_seqs=24),
    "kda_long": Workload("kda_long", B=1, T=65536, H=32, Hg=32, K=128, V=128,
                         chunk=64, gate="kda", io_dtype=torch.bfloat16,
                         gate_mult=0.5, h0_std=0.1, dht_std=0.1),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of workload ``w`` with some fields replaced (smaller test shapes)."""
    return dataclasses.replace(w, **kw)


def varlen_lengths(gen: torch.Generator, n: int, total: int, lo: int = 17,
                   hi: int = 8192, mu: float = math.log(1024.0),
                   sigma: float = 1.0) -> list[int]:
    """Sequence lengths ~ lognormal(mu, sigma), clipped to [lo, hi], then rescaled
    to sum exactly to ``total`` (largest-remainder rounding, re-clipped, repeated).
    """
    if n * lo > total or n * hi < total:
        raise ValueError("cannot fit lengths")
    z = torch.randn(n, generator=gen, dtype=torch.float64)
    L = torch.exp(mu + sigma * z).clamp(lo, hi)
    for _ in range(64):
        x = L * (total / float(L.sum()))
        f = torch.floor(x)
        rem = int(total - f.sum().item())
        frac = x - f
        order = torch.argsort(-frac, stable=True)
        if rem > 0:
            f[order[:rem]] += 1
        elif rem < 0:
            f[order[rem:]] -= 1
        f = f.clamp(lo, hi)
        if int(f.sum().item()) == total:
            return [int(v) for v in f.tolist()]
        L = f
    raise RuntimeError("length rescaling did not converge")


def _l2norm_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)


def make_inputs(w: Workload, device: Optional[str] = None) -> dict:
    """Seeded inputs for workload ``w`` (CPU tensors unless ``device`` given).

    Returns dict with q, k [B,T,Hg,K] (io); v, do [B,T,H,V] (io);
    g fp32 [B,T,H,K] (kda) or [B,T,H] (gdn), raw per-token log2 gate (not
    cumulated); beta [B,T,H] (io); h0, dht fp32 [N,H,K,V] (zeros when the std
    is 0); cu_seqlens int32 [N+1] or None; scale = K**-0.5; the workload.
    """
    gen = torch.Generator().manual_seed(w.seed)
    B, T, H, Hg, K, V = w.B, w.T, w.H, w.Hg, w.K, w.V
    cu = None
    N = B
    if w.varlen:
        if B != 1:
            raise ValueError("varlen workloads are packed with B == 1")
        lens = varlen_lengths(gen, w.n_seqs, T)
        cu = torch.zeros(w.n_seqs + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
        N = w.n_seqs
    f32 = torch.float32
    q = _l2norm_rows(torch.randn(B, T, Hg, K, generator=gen, dtype=f32))
    k = _l2norm_rows(torch.randn(B, T, Hg, K, generator=gen, dtype=f32))
    v = torch.randn(B, T, H, V, generator=gen, dtype=f32)
    gshape = (B, T, H, K) if w.gate == "kda" else (B, T, H)
    g = -torch.nn.functional.softplus(torch.randn(*gshape, generator=gen, dtype=f32)) * w.gate_mult
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen, dtype=f32))
    h0 = torch.randn(N, H, K, V, generator=gen, dtype=f32) * w.h0_std
    do = torch.randn(B, T, H, V, generator=gen, dtype=f32)
    dht = torch.randn(N, H, K, V, generator=gen, dtype=f32) * w.dht_std
    io = w.io_dtype
    out = dict(q=q.to(io), k=k.to(io), v=v.to(io), g=g, beta=beta.to(io), h0=h0,
               do=do.to(io), dht=dht, cu_seqlens=cu, scale=K ** -0.5, workload=w)
    if device is not None:
        for key in ("q", "k", "v", "g", "beta", "h0", "do", "dht", "cu_seqlens"):
            if out[key] is not None:
                out[key] = out[key].to(device)
    return out


def head_subset(inp: dict, hks: list) -> tuple:
    """Inputs restricted to q/k heads ``hks`` and the value heads of their GQA
    groups (head h reads q/k head h // (H / Hg)). Returns (inputs, value heads).
    Every (sequence, head) is independent, so this is an exact sub-problem."""
    w = inp["workload"]
    G = w.H // w.Hg
    hv = [hk * G + j for hk in hks for j in range(G)]
    out = dict(inp)
    out["q"] = inp["q"][:, :, hks]
    out["k"] = inp["k"][:, :, hks]
    for key in ("v", "do", "beta", "g"):
        out[key] = inp[key][:, :, hv]
    out["h0"] = inp["h0"][:, hv]
    out["dht"] = inp["dht"][:, hv]
    return out, hv
