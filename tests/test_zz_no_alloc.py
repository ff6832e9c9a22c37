"""gdr_bwd_static, the backward without a workspace argument (its workspace is
the library's fixed per-GPU scratch), against gdr_bwd with a caller workspace
on the same inputs: two calls in a row, the second on a smaller problem, so
that the second call runs over scratch the first one left dirty.

Both entry points run the same kernels on the same inputs, so the outputs must
agree bit for bit (stricter than the oracle tolerance of the parity tests).
"""
import pytest
import torch

from gdr_workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

gdr = pytest.importorskip("chunked_gated_delta_gdr_amd")

OUTS = ("dq", "dk", "dv", "dg", "db", "dh0")
KDA16 = WORKLOADS["kda_fixed_h16"]
GDN = WORKLOADS["gdn_gqa_fp16"]


def _run(w, static: bool):
    inp = make_inputs(w)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"])
    kw = dict(h0=t["h0"], dht=t["dht"], cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk)
    out = gdr.bwd_static(*args, **kw) if static else gdr.bwd(*args, **kw)
    torch.cuda.synchronize()
    return [o.cpu() for o in out]


@pytest.mark.parametrize("first,second", [
    # bf16 KDA at K = V = 128, then a shorter and narrower one
    (scaled(KDA16, B=2, T=300, H=4, Hg=4, dht_std=0.1, seed=21), scaled(KDA16, B=1, T=70, H=2, Hg=2, seed=22)),
    # fp16 GDN with GQA at chunk 32 (varlen), then a smaller fixed-length one
    (scaled(GDN, B=1, T=400, H=4, Hg=2, n_seqs=5, seed=23), scaled(GDN, B=1, T=45, H=2, Hg=1, seed=24)),
])
def test_static_matches_workspace_entry(first, second):
    for w in (first, second):
        desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, n_seqs=w.n_seqs,
                             gate=0 if w.gate == "kda" else 1, io_dtype=w.io_dtype)
        assert gdr.workspace_bytes(desc) <= gdr.STATIC_SCRATCH_BYTES
        print(f"no-alloc case {w.name} B={w.B} T={w.T} H={w.H} Hg={w.Hg} C={w.chunk} n_seqs={w.n_seqs}",
              flush=True)
        a = _run(w, static=True)
        b = _run(w, static=False)
        for name, x, y in zip(OUTS, a, b):
            assert torch.equal(x, y), f"{w.name}: {name} differs between gdr_bwd_static and gdr_bwd"

