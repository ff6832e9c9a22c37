"""GPU parity of the forward pass (gdr_fwd through the C ABI) against the fp64
oracle's forward: o for every real token and the final states ht.

Bar: per output tensor, max|gpu - ref| / max|ref| <= 1e-4 for fp32 io and
<= 2e-2 for bf16 / fp16 io (the backward's bar, same arithmetic types).
"""
import numpy as np
import pytest
import torch

import oracle
from gdr_workloads import WORKLOADS, head_subset, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")

KDA16 = WORKLOADS["kda_fixed_h16"]
GDN = WORKLOADS["gdn_gqa_fp16"]
VARLEN = WORKLOADS["kda_varlen"]
TINY = WORKLOADS["tiny_kda_fp32"]


def run_fwd(inp, with_h0=True):
    import chunked_gated_delta_gdr_amd as gdr
    w = inp["workload"]
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, ht = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"] if with_h0 else None,
                    cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk)
    torch.cuda.synchronize()
    return o.detach().cpu().double().numpy(), ht.detach().cpu().double().numpy()


def ref_fwd(inp, with_h0=True):
    w = inp["workload"]
    r = oracle.run(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None,
                   inp["h0"] if with_h0 else None, None, inp["cu_seqlens"], inp["scale"], w.gate,
                   backward=False, forward_out=True)
    return r["o"], r["ht"]


def errs(o, ht, ro, rht, mask):
    out = {}
    for name, g, r in (("o", o[mask], ro[mask]), ("ht", ht, rht)):
        out[name] = float(np.abs(g - r).max() / np.abs(r).max()) if np.all(np.isfinite(g)) else float("inf")
    return out


def check(w, hks=None, with_h0=True):
    inp = make_inputs(w)
    o, ht = run_fwd(inp, with_h0)
    mask = tu.real_token_mask(inp)
    if hks is None:
        ro, rht = ref_fwd(inp, with_h0)
    else:
        sub, hv = head_subset(inp, hks)
        ro, rht = ref_fwd(sub, with_h0)
        o, ht = o[:, :, hv], ht[:, hv]
    e = errs(o, ht, ro, rht, mask)
    tol = tu.tolerance(w)
    tu.report(f"fwd {w.name} T={w.T} H={w.H}", e, tol)
    assert all(v <= tol for v in e.values()), f"{w.name}: {e} (tolerance {tol})"


SMALL = {
    "tiny_kda_fp32": TINY,
    "fp32_gdn_c32_h0": scaled(TINY, T=150, gate="gdn", chunk=32, h0_std=0.1),
    "bf16_kda_ragged_h0": scaled(KDA16, B=2, T=200, H=2, Hg=2),
    "bf16_kda_gqa": scaled(KDA16, B=1, T=130, H=4, Hg=1, seed=1),
    "f16_gdn_gqa_c32": scaled(GDN, B=2, T=100, H=4, Hg=2, h0_std=0.1),
    "bf16_varlen": scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5),
    "bf16_gates_x16": scaled(KDA16, B=1, T=150, H=2, Hg=2, gate_mult=8.0, seed=3),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_small(name):
    check(SMALL[name])


@pytest.mark.parametrize("T", [1, 17, 64, 65])
def test_fwd_short_sequences(T):
    check(scaled(KDA16, B=2, T=T, H=2, Hg=2, seed=T))


def test_fwd_without_h0():
    check(scaled(KDA16, B=1, T=140, H=2, Hg=2, seed=11), with_h0=False)


def test_fwd_full_kda_fixed_h16():
    check(KDA16, hks=[0, 9])


def test_fwd_full_gdn_gqa_fp16():
    check(GDN, hks=[5])


def test_fwd_full_kda_varlen():
    check(VARLEN, hks=[3])


def test_fwd_full_kda_long():
    check(WORKLOADS["kda_long"], hks=[7, 30])


def test_fwd_varlen_more_sequences_than_one_table_pass():
    """The forward pass over 300 packed sequences (the chunk table's multi-pass path)."""
    gen = torch.Generator().manual_seed(62)
    lens = torch.randint(1, 24, (300,), generator=gen)
    cu = torch.zeros(301, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    w = scaled(VARLEN, T=int(cu[-1]), H=2, Hg=2, K=64, V=64, n_seqs=1, seed=62)
    inp = make_inputs(w)
    inp["cu_seqlens"] = cu
    inp["h0"] = torch.randn(300, w.H, w.K, w.V, generator=gen) * 0.1
    o, ht = run_fwd(inp)
    ro, rht = ref_fwd(inp)
    e = errs(o, ht, ro, rht, tu.real_token_mask(inp))
    tu.report("fwd varlen 300 sequences", e, 2e-2)
    assert all(v <= 2e-2 for v in e.values()), e


def test_fwd_empty_input():
    """T = 0: o is empty and ht is h0 passed through."""
    import chunked_gated_delta_gdr_amd as gdr
    w = scaled(KDA16, B=2, T=0, H=2, Hg=2, K=64, V=64, h0_std=0.1)
    inp = make_inputs(w)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, ht = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], scale=inp["scale"])
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(ht.cpu(), inp["h0"])


def test_fwd_varlen_with_empty_sequences():
    inp = tu.varlen_with_empty_sequences()
    o, ht = run_fwd(inp)
    ro, rht = ref_fwd(inp)
    e = errs(o, ht, ro, rht, tu.real_token_mask(inp))
    assert all(v <= 2e-2 for v in e.values()), e
