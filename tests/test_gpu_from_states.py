"""The backward from caller-supplied per-chunk states (gdr_bwd_from_states)
against the fp64 oracle: the states fed in are the oracle's own chunk-boundary
states h_c (the state before each chunk), rounded to the io dtype, in both
layouts ([chunks][H][K][V] and, with state_v_first, [chunks][H][V][K]; dht and
dh0 then transposed too). Bar: max|gpu - ref| / max|ref| per output, 1e-4 for
fp32 io, 2e-2 for bf16 / fp16 io, as for the full backward.
"""
import numpy as np
import pytest
import torch

from gdr_workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")
gdr = pytest.importorskip("chunked_gated_delta_gdr_amd")

KDA16 = WORKLOADS["kda_fixed_h16"]
GDN = WORKLOADS["gdn_gqa_fp16"]
VARLEN = WORKLOADS["kda_varlen"]
TINY = WORKLOADS["tiny_kda_fp32"]

CASES = {
    "bf16_kda_ragged": scaled(KDA16, B=2, T=200, H=2, Hg=2, dht_std=0.1, seed=51),
    "f16_gdn_gqa_varlen_c32": scaled(GDN, B=1, T=333, H=4, Hg=2, n_seqs=6, seed=52),
    "fp32_kda_d64": scaled(TINY, T=150, h0_std=0.1, dht_std=0.1, seed=53),
    "bf16_kda_d64_c32_gqa": scaled(KDA16, B=1, T=130, H=4, Hg=2, K=64, V=64, chunk=32, dht_std=0.1, seed=54),
    "bf16_varlen": scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5, seed=55),
}


def _transpose_states(x):
    return None if x is None else x.transpose(-1, -2).contiguous()


def _from_states(inp, ref_chunks, v_first: bool):
    w = inp["workload"]
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    h = torch.from_numpy(ref_chunks).to(w.io_dtype)            # [chunks, H, K, V], rounded once
    dht = t["dht"]
    if v_first:
        h, dht = _transpose_states(h), _transpose_states(dht)
    if not w.varlen:
        h = h.reshape(w.B, -1, *h.shape[1:])                     # [B, NT, H, K, V]
    out = gdr.bwd_from_states(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h.contiguous().cuda(),
                              dht=dht, cu_seqlens=t["cu_seqlens"], scale=inp["scale"],
                              chunk_size=w.chunk, state_v_first=v_first)
    torch.cuda.synchronize()
    res = dict(zip(tu.OUTS, [o.detach().cpu() for o in out]))
    if v_first:
        res["dh0"] = _transpose_states(res["dh0"])
    return res


@pytest.mark.parametrize("v_first", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_from_states_matches_oracle(name, v_first):
    w = CASES[name]
    inp = make_inputs(w)
    ref = tu.run_oracle(inp, chunk=w.chunk)
    gpu = _from_states(inp, ref["h_chunks"], v_first)
    errs = tu.rel_errors(gpu, ref, tu.real_token_mask(inp))
    print(f"from_states {name} v_first={v_first}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tu.tolerance(w)}
    assert not bad, f"{name}: {bad}"


def test_from_states_headline_workload():
    """The full-size headline workload (B=2, T=4096, H=16, K=V=128, bf16),
    every head, from the oracle's states in the value-first layout."""
    w = KDA16
    inp = make_inputs(w)
    ref = tu.run_oracle(inp, chunk=w.chunk)
    gpu = _from_states(inp, ref["h_chunks"], True)
    errs = tu.rel_errors(gpu, ref, tu.real_token_mask(inp))
    print("from_states headline: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= tu.tolerance(w) for v in errs.values()), errs


def test_state_v_first_full_backward():
    """gdr_bwd with state_v_first: h0, dht in and dh0 out transposed give the
    transposed results of the default layout, bit for bit."""
    w = scaled(KDA16, B=2, T=150, H=2, Hg=2, h0_std=0.1, dht_std=0.1, seed=56)
    inp = make_inputs(w)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"])
    a = gdr.bwd(*args, h0=t["h0"], dht=t["dht"], scale=inp["scale"])
    b = gdr.bwd(*args, h0=_transpose_states(t["h0"]), dht=_transpose_states(t["dht"]), scale=inp["scale"],
                state_v_first=True)
    torch.cuda.synchronize()
    for name, x, y in zip(tu.OUTS, a, b):
        if name == "dh0":
            y = _transpose_states(y)
        assert torch.equal(x, y), name
    o1, ht1 = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], scale=inp["scale"])
    o2, ht2 = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=_transpose_states(t["h0"]),
                      scale=inp["scale"], state_v_first=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, _transpose_states(ht2))
