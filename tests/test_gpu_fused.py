"""The fused reverse backward (gdr_bwd_fused: one kernel per (sequence, value
head) walks the chunks from the last to the first with the state gradient dh on
chip) against the fp64 oracle, at the bar of the full backward (1e-4 fp32,
2e-2 bf16 / fp16, max|gpu - ref| / max|ref| per output). Built for chunk 32:
the GDN GQA workload's configuration first, plus the per-channel gate, fp32
io, K = 64, varlen, GQA group sizes 1, 2 and 4, and the edge cases.
"""
import pytest
import torch

from gdr_workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")
gdr = pytest.importorskip("chunked_gated_delta_gdr_amd")

GDN = WORKLOADS["gdn_gqa_fp16"]
KDA16 = WORKLOADS["kda_fixed_h16"]
VARLEN = WORKLOADS["kda_varlen"]
TINY = WORKLOADS["tiny_kda_fp32"]

CASES = {
    "f16_gdn_gqa2": scaled(GDN, B=2, T=150, H=4, Hg=2, dht_std=0.1, h0_std=0.1, seed=71),
    "f16_gdn_gqa4_varlen": scaled(GDN, B=1, T=333, H=4, Hg=1, n_seqs=6, seed=72),
    "f16_gdn_nogqa": scaled(GDN, B=1, T=97, H=2, Hg=2, seed=73),
    "bf16_kda_c32": scaled(KDA16, B=1, T=130, H=2, Hg=2, chunk=32, dht_std=0.1, seed=74),
    "bf16_kda_c32_gqa_d64": scaled(KDA16, B=1, T=100, H=4, Hg=2, K=64, V=64, chunk=32, seed=75),
    "fp32_kda_c32": scaled(TINY, T=150, chunk=32, h0_std=0.1, dht_std=0.1, seed=76),
    "fp32_gdn_c32_gqa": scaled(TINY, T=90, H=4, Hg=2, gate="gdn", chunk=32, dht_std=0.1, seed=77),
    "bf16_varlen_c32": scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5, chunk=32, seed=78),
}


def run_fused(inp, v_first=False, with_h0=True, with_dht=True):
    w = inp["workload"]
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    h0 = t["h0"] if with_h0 else None
    dht = t["dht"] if with_dht else None
    if v_first:
        h0 = None if h0 is None else h0.transpose(-1, -2).contiguous()
        dht = None if dht is None else dht.transpose(-1, -2).contiguous()
    out = gdr.bwd_fused(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=h0, dht=dht,
                        cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk,
                        state_v_first=v_first)
    torch.cuda.synchronize()
    res = dict(zip(tu.OUTS, [o.detach().cpu() for o in out]))
    if v_first:
        res["dh0"] = res["dh0"].transpose(-1, -2).contiguous()
    return res


def _check(errs, tol, label):
    tu.report(label, errs, tol)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad}"


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_oracle(name):
    w = CASES[name]
    inp = make_inputs(w)
    errs = tu.rel_errors(run_fused(inp), tu.run_oracle(inp), tu.real_token_mask(inp))
    _check(errs, tu.tolerance(w), f"fused {name}")


@pytest.mark.parametrize("with_h0,with_dht,v_first", [(False, False, False), (True, True, True)])
def test_fused_states_and_layout(with_h0, with_dht, v_first):
    w = scaled(GDN, B=1, T=120, H=4, Hg=2, h0_std=0.2, dht_std=0.2, seed=79)
    inp = make_inputs(w)
    gpu = run_fused(inp, v_first=v_first, with_h0=with_h0, with_dht=with_dht)
    ref = tu.run_oracle(inp, with_h0, with_dht)
    _check(tu.rel_errors(gpu, ref), tu.tolerance(w), f"fused h0={with_h0} dht={with_dht} v_first={v_first}")


@pytest.mark.parametrize("T", [1, 31, 32, 33])
def test_fused_short_sequences(T):
    w = scaled(GDN, B=2, T=T, H=4, Hg=2, dht_std=0.1, seed=80 + T)
    inp = make_inputs(w)
    _check(tu.rel_errors(run_fused(inp), tu.run_oracle(inp)), tu.tolerance(w), f"fused T={T}")


def test_fused_empty_and_ragged_varlen():
    """Empty sequences pass dht through to dh0; tokens outside every sequence stay untouched."""
    inp = tu.varlen_with_empty_sequences()
    inp["workload"] = scaled(inp["workload"], chunk=32)
    got = run_fused(inp)
    _check(tu.rel_errors(got, tu.run_oracle(inp), tu.real_token_mask(inp)), 2e-2, "fused empty sequences")
    for n in (0, 2, 3, 6):
        assert torch.equal(got["dh0"][n], inp["dht"][n]), n


def test_fused_full_gdn_gqa_workload():
    """The full-size GDN GQA workload (B=4, T=8192, H=32, Hg=16, C=32, fp16),
    every head computed, q/k head 5 and its value heads compared."""
    inp = make_inputs(GDN)
    gpu = run_fused(inp)
    sub, hv = tu.head_subset(inp, [5])
    ref = tu.run_oracle(sub)
    _check(tu.rel_errors(gpu, ref, tu.real_token_mask(inp), hks=[5], hv=hv), 2e-2, "fused full gdn_gqa_fp16")


def test_fused_only_chunk_32():
    w = scaled(KDA16, B=1, T=64, H=2, Hg=2)
    inp = make_inputs(w)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    with pytest.raises(gdr.GdrError):
        gdr.bwd_fused(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], chunk_size=64)
