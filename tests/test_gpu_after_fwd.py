"""The backward after the forward pass (gdr_bwd_after_fwd through the C ABI):
gdr_fwd fills the workspace, then only the reverse sweep and the gradient
kernel run on it.

Checks: the six gradients against the fp64 oracle (the backward's bar:
max|gpu - ref| / max|ref| <= 1e-4 for fp32 io, <= 2e-2 for bf16 / fp16), and
bitwise equality with gdr_bwd on the same inputs (same kernels, same saved
states), for small cases that span several chunks and a ragged tail, varlen,
GQA, both gate forms, every io dtype, and a full-size workload.
"""
import pytest
import torch

from gdr_workloads import WORKLOADS, head_subset, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")

KDA16 = WORKLOADS["kda_fixed_h16"]
GDN = WORKLOADS["gdn_gqa_fp16"]
VARLEN = WORKLOADS["kda_varlen"]
TINY = WORKLOADS["tiny_kda_fp32"]

CASES = {
    "fp32_kda_h0_dht": scaled(TINY, T=200, h0_std=0.1, dht_std=0.1),
    "fp32_gdn_c32_ragged": scaled(TINY, T=150, gate="gdn", chunk=32, h0_std=0.1, dht_std=0.1),
    "bf16_kda_ragged": scaled(KDA16, B=2, T=200, H=2, Hg=2, dht_std=0.1),
    "bf16_kda_gqa": scaled(KDA16, B=1, T=130, H=4, Hg=1, seed=1),
    "bf16_kda_d64": scaled(KDA16, B=1, T=190, H=3, Hg=3, K=64, V=64, seed=2),
    "f16_gdn_gqa_c32": scaled(GDN, B=2, T=100, H=4, Hg=2, h0_std=0.1),
    "bf16_varlen": scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5),
    "f16_gdn_varlen_c32": scaled(GDN, B=1, T=333, H=2, Hg=1, n_seqs=6, seed=9),
    # enough (sequence, head) pairs that even the one-direction sweeps take
    # 64-column tiles (N H D / 32 >= 2 x 256 CUs), which at C = 64 read the w^T
    # and k~^T the forward pass's preparation must then have stored
    "bf16_kda_wide_c64": scaled(KDA16, B=10, T=70, H=16, Hg=16, dht_std=0.1, seed=11),
}


def run_after_fwd(inp):
    """gdr_fwd, then gdr_bwd_after_fwd on the same workspace; returns the
    gradients and gdr_bwd's on the same inputs."""
    import chunked_gated_delta_gdr_amd as gdr
    w = inp["workload"]
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk,
                         n_seqs=0 if t["cu_seqlens"] is None else t["cu_seqlens"].numel() - 1,
                         gate=0 if w.gate == "kda" else 1, io_dtype=w.io_dtype)
    ws = torch.full((gdr.workspace_bytes(desc),), 255, dtype=torch.uint8, device="cuda")
    common = dict(cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk)
    gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], workspace=ws, **common)
    got = gdr.bwd_after_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], ws, dht=t["dht"], **common)
    full = gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=t["h0"], dht=t["dht"], **common)
    torch.cuda.synchronize()
    return (dict(zip(tu.OUTS, [o.detach().cpu() for o in got])),
            dict(zip(tu.OUTS, [o.detach().cpu() for o in full])))


@pytest.mark.parametrize("name", list(CASES))
def test_after_fwd_matches_oracle_and_bwd(name):
    w = CASES[name]
    inp = make_inputs(w)
    got, full = run_after_fwd(inp)
    mask = tu.real_token_mask(inp)
    errs = tu.rel_errors(got, tu.run_oracle(inp), mask)
    tol = tu.tolerance(w)
    assert all(v <= tol for v in errs.values()), f"{name}: {errs}"
    m = torch.from_numpy(mask)
    for n in tu.OUTS:
        a, b = (got[n], full[n]) if n == "dh0" else (got[n][m], full[n][m])
        assert torch.equal(a, b), f"{name}: {n} differs from gdr_bwd"


def test_after_fwd_full_kda_fixed_h16():
    inp = make_inputs(KDA16)
    got, full = run_after_fwd(inp)
    for n in tu.OUTS:
        assert torch.equal(got[n], full[n]), n
    hks = [4]
    sub, hv = head_subset(inp, hks)
    errs = tu.rel_errors(got, tu.run_oracle(sub), tu.real_token_mask(inp), hks=hks, hv=hv)
    assert all(v <= 2e-2 for v in errs.values()), errs


def test_after_fwd_argument_checks():
    import chunked_gated_delta_gdr_amd as gdr
    w = scaled(KDA16, B=1, T=64, H=2, Hg=2)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in make_inputs(w).items()}
    with pytest.raises(ValueError):   # the forward's workspace is required
        gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], after_fwd=True)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # h0 belongs to the forward call
        gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=t["h0"], workspace=ws,
                after_fwd=True)
