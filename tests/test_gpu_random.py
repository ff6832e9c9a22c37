"""Randomized GPU parity: small problems drawn from every supported axis (io
dtype, gate form, K = V in {64, 128}, chunk in {32, 64}, GQA ratio, length
mix, varlen with empty and length-1 sequences, h0 / dht present or not), each
compared element by element with the fp64 oracle at the method's bar
(max|gpu - ref| / max|ref| <= 1e-4 fp32 io, <= 2e-2 bf16 / fp16 io), the
backward through gdr_bwd and, on the same inputs, gdr_fwd's outputs.

The cases come from a fixed seed, so the set is the same on every run.
"""
import random

import numpy as np
import pytest
import torch

import oracle
from gdr_workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")

KDA16 = WORKLOADS["kda_fixed_h16"]


def draw_cases(n=24, seed=1234):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        io = rng.choice([torch.float32, torch.bfloat16, torch.float16])
        K = 64 if io == torch.float32 else rng.choice([64, 128])
        chunk = rng.choice([32, 64])
        gate = rng.choice(["kda", "gdn"])
        Hg = rng.choice([1, 2])
        H = Hg * rng.choice([1, 2, 3])
        varlen = rng.random() < 0.4
        if varlen:
            lens = [rng.choice([0, 1, rng.randint(2, 40), rng.randint(41, 150)]) for _ in range(rng.randint(2, 5))]
            if sum(lens) == 0:
                lens[0] = 5
            B, T = 1, sum(lens)
        else:
            lens = None
            B, T = rng.choice([1, 2]), rng.randint(1, 200)
        w = scaled(KDA16, B=B, T=T, H=H, Hg=Hg, K=K, V=K, chunk=chunk, gate=gate, io_dtype=io,
                   gate_mult=rng.choice([0.1, 0.5, 2.0]) if gate == "kda" else rng.choice([0.1, 0.5]),
                   h0_std=rng.choice([0.0, 0.1]), dht_std=rng.choice([0.0, 0.1]), seed=1000 + i)
        cases.append((f"case{i}_{str(io).split('.')[-1]}_{gate}_k{K}_c{chunk}_h{H}g{Hg}_t{T}"
                      + ("_varlen" if varlen else ""), w, lens))
    return cases


CASES = draw_cases()


def inputs(w, lens):
    inp = make_inputs(w)
    if lens is not None:
        gen = torch.Generator().manual_seed(w.seed)
        cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
        inp["cu_seqlens"] = cu
        inp["h0"] = torch.randn(len(lens), w.H, w.K, w.V, generator=gen) * w.h0_std
        inp["dht"] = torch.randn(len(lens), w.H, w.K, w.V, generator=gen) * w.dht_std
    return inp


@pytest.mark.parametrize("name,w,lens", CASES, ids=[c[0] for c in CASES])
def test_random_backward(name, w, lens):
    inp = inputs(w, lens)
    errs = tu.rel_errors(tu.run_gpu(inp), tu.run_oracle(inp), tu.real_token_mask(inp))
    tol = tu.tolerance(w)
    assert all(v <= tol for v in errs.values()), f"{name}: {errs}"


@pytest.mark.parametrize("name,w,lens", CASES[::2], ids=[c[0] for c in CASES[::2]])
def test_random_forward(name, w, lens):
    import chunked_gated_delta_gdr_amd as gdr
    inp = inputs(w, lens)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, ht = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                    scale=inp["scale"], chunk_size=w.chunk)
    torch.cuda.synchronize()
    r = oracle.run(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None, inp["h0"], None,
                   inp["cu_seqlens"], inp["scale"], w.gate, backward=False, forward_out=True)
    mask = tu.real_token_mask(inp)
    tol = tu.tolerance(w)
    for nm, g, ref in (("o", o.cpu().double().numpy()[mask], r["o"][mask]),
                       ("ht", ht.cpu().double().numpy(), r["ht"])):
        denom = np.abs(ref).max()
        err = np.abs(g - ref).max() / denom if denom > 0 else np.abs(g).max()
        assert err <= tol, f"{name}: {nm} {err}"
