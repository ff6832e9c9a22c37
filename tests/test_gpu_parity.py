"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar (from the method description): per output tensor, max|gpu - ref| /
max|ref| over real tokens <= 1e-4 for fp32 io and <= 2e-2 for bf16 / fp16 io.
Small cases compare every element; the full-size workloads run in the launch
configuration the benchmark times and compare sampled heads (the oracle is
per (sequence, head), so a head subset is an exact sub-problem).
"""
import numpy as np
import pytest
import torch

from gdr_workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

tu = pytest.importorskip("gdr_testutil")


def _check(errs, tol, label=""):
    import os
    tu.report(label or os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], errs, tol)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"{label} over tolerance {tol}: {bad} (all: {errs})"


KDA16 = WORKLOADS["kda_fixed_h16"]
GDN = WORKLOADS["gdn_gqa_fp16"]
VARLEN = WORKLOADS["kda_varlen"]
TINY = WORKLOADS["tiny_kda_fp32"]

SMALL = {
    # the tiny workload at its full size
    "tiny_kda_fp32": TINY,
    "tiny_fp32_h0_dht": scaled(TINY, T=200, h0_std=0.1, dht_std=0.1),
    "fp32_gdn_c32_ragged": scaled(TINY, T=150, gate="gdn", chunk=32, h0_std=0.1, dht_std=0.1),
    "fp32_kda_c32_gqa": scaled(TINY, T=97, H=4, Hg=2, chunk=32, dht_std=0.1, seed=3),
    # several chunks and a ragged tail at K = V = 128
    "bf16_kda_ragged": scaled(KDA16, B=2, T=200, H=2, Hg=2, dht_std=0.1),
    "bf16_kda_gqa": scaled(KDA16, B=1, T=130, H=4, Hg=1, seed=1),
    "bf16_kda_d64": scaled(KDA16, B=1, T=190, H=3, Hg=3, K=64, V=64, seed=2),
    "bf16_gdn_c64": scaled(GDN, B=1, T=160, H=2, Hg=1, chunk=64, io_dtype=torch.bfloat16),
    "f16_gdn_gqa_c32": scaled(GDN, B=2, T=100, H=4, Hg=2),
    "f16_kda_c32": scaled(KDA16, B=1, T=75, H=2, Hg=2, chunk=32, io_dtype=torch.float16, seed=5),
    "bf16_varlen": scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5),
    "bf16_varlen_many_short": scaled(VARLEN, T=700, H=2, Hg=2, n_seqs=30, seed=7),
    "f16_gdn_varlen_c32": scaled(GDN, B=1, T=333, H=2, Hg=1, n_seqs=6, seed=9),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_compare(name):
    w = SMALL[name]
    _check(tu.parity(w), tu.tolerance(w), name)


@pytest.mark.parametrize("with_h0,with_dht", [(False, False), (True, False), (False, True)])
def test_optional_states(with_h0, with_dht):
    """h0 / dht passed as NULL behave as zero; dh0 is always written."""
    w = scaled(KDA16, B=1, T=140, H=2, Hg=2, h0_std=0.2, dht_std=0.2, seed=11)
    _check(tu.parity(w, with_h0=with_h0, with_dht=with_dht), tu.tolerance(w))


@pytest.mark.parametrize("T", [1, 5, 16, 17, 63, 64, 65])
def test_short_sequences(T):
    """Shorter than one chunk, exactly one, one plus a single token."""
    w = scaled(KDA16, B=2, T=T, H=2, Hg=2, dht_std=0.1, seed=T)
    _check(tu.parity(w), tu.tolerance(w), f"T={T}")


def test_varlen_lengths_1_to_17():
    """17 packed sequences of lengths 1, 2, ..., 17 (every partial-chunk size)."""
    cu = np.cumsum([0] + list(range(1, 18)))
    w = scaled(VARLEN, T=int(cu[-1]), H=2, Hg=2, n_seqs=9, seed=13)  # 9 x 17 = 153 fits the draw
    inp = make_inputs(w)
    inp["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    gen = torch.Generator().manual_seed(14)
    inp["h0"] = torch.randn(17, w.H, w.K, w.V, generator=gen) * 0.1
    inp["dht"] = torch.randn(17, w.H, w.K, w.V, generator=gen) * 0.1
    gpu = tu.run_gpu(inp)
    ref = tu.run_oracle(inp)
    _check(tu.rel_errors(gpu, ref, tu.real_token_mask(inp)), tu.tolerance(w))


@pytest.mark.parametrize("beta_val", [0.0, 1.0])
def test_beta_extremes(beta_val):
    w = scaled(KDA16, B=1, T=150, H=2, Hg=2, dht_std=0.1, seed=17)
    inp = make_inputs(w)
    inp["beta"] = torch.full_like(inp["beta"], beta_val)
    gpu = tu.run_gpu(inp)
    ref = tu.run_oracle(inp)
    errs = tu.rel_errors(gpu, ref)
    if beta_val == 0.0:  # frozen state: dk = dv = 0 exactly
        assert gpu["dk"].abs().max() == 0 and gpu["dv"].abs().max() == 0
        errs.pop("dk"), errs.pop("dv")
    _check(errs, tu.tolerance(w))


def test_large_gates_x16():
    """Gates x16 (the exponent-law guard arm): decays underflow, nothing overflows."""
    w = scaled(KDA16, B=1, T=200, H=2, Hg=2, gate_mult=8.0, dht_std=0.1, seed=19)
    errs = tu.parity(w)
    _check(errs, tu.tolerance(w))


@pytest.mark.parametrize("gate_mult", [3.7, 32.0])
def test_diagonal_guard_paths(gate_mult):
    """In-block gate ranges around and far beyond the diagonal-block MFMA
    guard (2^64): at x7.4 the default gates, 19 of 52 (block, column half)
    pairs take the exact per-element path and the rest the MFMA path within
    the same chunks; at x64 every block takes the exact path. (x16 above is
    also all exact.)"""
    w = scaled(KDA16, B=1, T=200, H=2, Hg=2, gate_mult=gate_mult, dht_std=0.1, seed=37)
    _check(tu.parity(w), tu.tolerance(w))


def test_f16_diagonal_guard_mixed():
    """fp16 operands keep the MFMA diagonal only within 2^8: at the default KDA
    gates 44 of 52 (block, column half) pairs take the exact path, 8 the MFMA."""
    w = scaled(KDA16, B=1, T=200, H=2, Hg=2, io_dtype=torch.float16, dht_std=0.1, seed=47)
    _check(tu.parity(w), tu.tolerance(w))


ONE_REF_MIXED = {
    "bf16_c64": (scaled(KDA16, B=1, T=200, H=3, Hg=3, gate_mult=2.0, dht_std=0.1, seed=53), 64.0),
    "f16_c64": (scaled(KDA16, B=1, T=200, H=3, Hg=3, io_dtype=torch.float16, gate_mult=0.25, dht_std=0.1,
                       seed=53), 8.0),
    "f32_c64": (scaled(TINY, T=130, gate_mult=2.4, h0_std=0.1, dht_std=0.1, seed=57), 64.0),
    "bf16_c32": (scaled(KDA16, B=1, T=200, H=3, Hg=3, chunk=32, gate_mult=4.0, dht_std=0.1, seed=53), 64.0),
    "f16_c32": (scaled(KDA16, B=1, T=200, H=3, Hg=3, chunk=32, io_dtype=torch.float16, gate_mult=0.5,
                       dht_std=0.1, seed=53), 8.0),
    "f32_c32": (scaled(TINY, T=130, chunk=32, gate_mult=4.0, h0_std=0.1, dht_std=0.1, seed=57), 64.0),
}


@pytest.mark.parametrize("name", list(ONE_REF_MIXED))
def test_prep_one_reference_bound_mixed(name):
    """The preparation kernel forms Aqk / Akk through one reference G_last / 2
    per column when every |G_r - G_last / 2| is within the operand guard, else
    through the block boundaries. Gates chosen so that one launch holds
    (chunk, head) items of both kinds, at both chunk sizes."""
    w, guard = ONE_REF_MIXED[name]
    fast, slow = tu.one_reference_split(w, guard)
    assert fast > 0 and slow > 0, (fast, slow)
    _check(tu.parity(w), tu.tolerance(w))


def test_gdn_scalar_prep_across_the_operand_bound():
    """Scalar gate: the preparation kernel forms Aqk / Akk as plain products
    times the decay for every chunk, including chunks whose gate range is past
    the bound that sends per-channel chunks to the per-boundary route."""
    w = scaled(GDN, B=1, T=200, H=4, Hg=2, gate_mult=1.0, seed=59)
    fast, slow = tu.one_reference_split(w, 8.0)
    assert fast > 0 and slow > 0, (fast, slow)
    _check(tu.parity(w), tu.tolerance(w))


def test_gdn_gqa_huge_gates():
    """Scalar gate, GQA, C = 32, gates large enough for the exact diagonal path."""
    w = scaled(GDN, B=1, T=150, H=4, Hg=2, gate_mult=8.0, seed=43)
    _check(tu.parity(w), tu.tolerance(w))


def test_fp32_diagonal_guard_mixed():
    w = scaled(TINY, T=130, gate_mult=3.7, h0_std=0.1, dht_std=0.1, seed=41)
    _check(tu.parity(w), tu.tolerance(w))


def test_fp32_large_gates_x16():
    w = scaled(TINY, T=130, gate_mult=8.0, h0_std=0.1, dht_std=0.1, seed=23)
    _check(tu.parity(w), tu.tolerance(w))


def test_stage_states_match_oracle():
    """Per-chunk states h_c and state gradients dh_{c+1} in the workspace
    match the oracle's chunk-boundary states."""
    import chunked_gated_delta_gdr_amd as gdr
    w = scaled(VARLEN, T=300, H=2, Hg=2, n_seqs=5, dht_std=0.1)
    inp = make_inputs(w)
    desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, n_seqs=w.n_seqs,
                         io_dtype=w.io_dtype)
    offs = gdr.workspace_offsets(desc)
    ws = torch.zeros(offs["total"], dtype=torch.uint8, device="cuda")
    tu.run_gpu(inp, workspace=ws)
    ref = tu.run_oracle(inp, chunk=w.chunk)
    nch, D = ref["h_chunks"].shape[0], w.K
    for name, key in (("h", "h_chunks"), ("dh", "dh_chunks")):
        raw = ws[offs[name]: offs[name] + nch * w.H * D * D * 2].cpu()
        # stored in tiles of 32 state columns: [nch][H][D/32][D][32]
        got = (raw.view(torch.bfloat16).double().numpy().reshape(nch, w.H, D // 32, D, 32)
               .transpose(0, 1, 3, 2, 4).reshape(nch, w.H, D, D))
        err = np.abs(got - ref[key]).max() / np.abs(ref[key]).max()
        assert err < 2e-2, f"{name}: {err}"


def test_deterministic_and_workspace_reuse():
    w = scaled(GDN, B=1, T=300, H=4, Hg=2, seed=29)
    inp = make_inputs(w)
    import chunked_gated_delta_gdr_amd as gdr
    desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, gate=1, io_dtype=w.io_dtype)
    ws = torch.full((gdr.workspace_bytes(desc),), 255, dtype=torch.uint8, device="cuda")
    a = tu.run_gpu(inp, workspace=ws)
    b = tu.run_gpu(inp, workspace=ws)
    for n in tu.OUTS:
        assert torch.equal(a[n], b[n]), n


def test_linear_in_output_gradients():
    """All six gradients are jointly linear in (do, dht): an oracle-free check."""
    w = scaled(TINY, T=160, h0_std=0.1, dht_std=0.1, seed=31)
    i1, i2 = make_inputs(w), make_inputs(scaled(w, seed=32))
    i3 = dict(i1)
    i3["do"] = 0.5 * i1["do"] - 2.0 * i2["do"]
    i3["dht"] = 0.5 * i1["dht"] - 2.0 * i2["dht"]
    i2 = dict(i1, do=i2["do"], dht=i2["dht"])
    r1, r2, r3 = tu.run_gpu(i1), tu.run_gpu(i2), tu.run_gpu(i3)
    for n in tu.OUTS:
        comb = 0.5 * r1[n].double() - 2.0 * r2[n].double()
        assert (r3[n].double() - comb).abs().max() <= 1e-4 * comb.abs().max(), n


# Enough (sequence, head) pairs that the sweep takes 64-column V tiles (when
# 2 N H D / 32 >= 2 x 256 CUs), at every (io, K, chunk) form; every element
# compared, backward and forward.
WIDE = {
    "fp32_d64_c64": scaled(TINY, B=10, T=90, H=16, Hg=16, h0_std=0.1, dht_std=0.1, seed=21),
    "fp32_d64_c32_gdn": scaled(TINY, B=10, T=70, H=16, Hg=8, chunk=32, gate="gdn", dht_std=0.1, seed=22),
    "bf16_d64_c64": scaled(KDA16, B=10, T=100, H=16, Hg=16, K=64, V=64, dht_std=0.1, seed=23),
    "bf16_d128_c64": scaled(KDA16, B=5, T=100, H=16, Hg=16, dht_std=0.1, seed=24),
    "f16_d128_c32_gqa": scaled(GDN, B=5, T=70, H=16, Hg=8, h0_std=0.1, seed=25),
}


# Sequences of more than 128 chunks on 32-column sweep tiles at chunk 64,
# every element compared: with K = 64 or fp32 io the register-set sweep
# refills its operands part by part within each step there; with 16-bit io at
# K = 128 the loader-wave sweep walks the same long sequences.
SPREAD = {
    "bf16_d128": scaled(KDA16, B=1, T=64 * 134 + 9, H=2, Hg=2, h0_std=0.1, dht_std=0.1, seed=71),
    "f16_d128": scaled(KDA16, B=1, T=64 * 130, H=2, Hg=1, io_dtype=torch.float16, gate_mult=0.25, dht_std=0.1,
                       seed=72),
    "bf16_d64": scaled(KDA16, B=2, T=64 * 129 + 1, H=2, Hg=2, K=64, V=64, dht_std=0.1, seed=73),
    "fp32_d64": scaled(TINY, B=1, T=64 * 131 + 30, H=2, Hg=2, h0_std=0.1, dht_std=0.1, seed=74),
}


@pytest.mark.parametrize("name", list(SPREAD))
def test_long_sequence_spread_refills(name):
    w = SPREAD[name]
    nch = (w.T + w.chunk - 1) // w.chunk
    assert w.chunk == 64 and nch > 128 and 2 * w.B * w.H * (w.V // 32) < 512
    _check(tu.parity(w), tu.tolerance(w), name)


WIDE_VARLEN = {
    # (base workload, io dtype, chunk, q/k heads): 8 sequences x 8 value heads
    # fill 2 x 8 x 8 x 4 = 512 >= 2 x 256 32-column tiles, so the sweep takes
    # 64-column tiles (the loader-wave sweep at 16-bit K = 128)
    "bf16_kda_c64": (KDA16, torch.bfloat16, 64, 8),
    "f16_gdn_gqa_c32": (GDN, torch.float16, 32, 4),
}


@pytest.mark.parametrize("name", list(WIDE_VARLEN))
def test_wide_sweep_tiles_varlen_short_and_empty(name):
    """64-column sweep tiles over packed sequences of 0, 1, one-chunk and
    ragged multi-chunk lengths (fewer chunks than the operands requested
    ahead, and empty ones): every output element compared with the oracle,
    and the empty sequences pass dht through to dh0."""
    base, io, chunk, hg = WIDE_VARLEN[name]
    lens = [0, 197, 1, 0, 64, 200, 33, 0]
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    w = scaled(base, B=1, T=int(cu[-1]), H=8, Hg=hg, n_seqs=1, chunk=chunk, io_dtype=io, seed=83)
    inp = make_inputs(w)
    gen = torch.Generator().manual_seed(83)
    inp["cu_seqlens"] = cu
    inp["h0"] = torch.randn(len(lens), w.H, w.K, w.V, generator=gen) * 0.1
    inp["dht"] = torch.randn(len(lens), w.H, w.K, w.V, generator=gen) * 0.1
    gpu = tu.run_gpu(inp)
    _check(tu.rel_errors(gpu, tu.run_oracle(inp), tu.real_token_mask(inp)), tu.tolerance(w), name)
    for n, ln in enumerate(lens):
        if ln == 0:
            assert torch.equal(gpu["dh0"][n], inp["dht"][n]), n


@pytest.mark.parametrize("name", list(WIDE))
def test_wide_sweep_tiles(name):
    w = WIDE[name]
    assert 2 * w.B * w.H * (w.V // 32) >= 512
    _check(tu.parity(w), tu.tolerance(w), name)
    import chunked_gated_delta_gdr_amd as gdr
    import oracle
    inp = make_inputs(w)
    t = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, ht = gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], scale=inp["scale"], chunk_size=w.chunk)
    torch.cuda.synchronize()
    r = oracle.run(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None, inp["h0"], None, None,
                   inp["scale"], w.gate, backward=False, forward_out=True)
    for nm, g, ref in (("o", o.cpu().double().numpy(), r["o"]), ("ht", ht.cpu().double().numpy(), r["ht"])):
        err = np.abs(g - ref).max() / np.abs(ref).max()
        assert err <= tu.tolerance(w), f"{name}: forward {nm} {err}"


# ---------------------------------------------------------------------------
# full-size workloads, sampled heads
# ---------------------------------------------------------------------------

def test_full_tiny_kda_fp32():
    _check(tu.parity(TINY), 1e-4)


def test_full_kda_fixed_h16():
    _check(tu.parity(KDA16, hks=[0, 9]), 2e-2)


def test_full_gdn_gqa_fp16():
    _check(tu.parity(GDN, hks=[5]), 2e-2)


def test_full_kda_varlen():
    _check(tu.parity(VARLEN, hks=[3, 12]), 2e-2)


def test_full_kda_long():
    _check(tu.parity(WORKLOADS["kda_long"], hks=[7, 30]), 2e-2)


# ---------------------------------------------------------------------------
# empty inputs
# ---------------------------------------------------------------------------

def test_empty_input_fixed_length():
    """T = 0: no token outputs, and dh0 is dht passed through (zero without it)."""
    w = scaled(KDA16, B=2, T=0, H=2, Hg=2, K=64, V=64, h0_std=0.1, dht_std=0.1)
    inp = make_inputs(w)
    got = tu.run_gpu(inp)
    for n in ("dq", "dk", "dv", "dg", "db"):
        assert got[n].numel() == 0, n
    assert torch.equal(got["dh0"], inp["dht"])
    assert torch.count_nonzero(tu.run_gpu(inp, with_dht=False)["dh0"]) == 0


def test_varlen_with_empty_sequences():
    inp = tu.varlen_with_empty_sequences()
    errs = tu.rel_errors(tu.run_gpu(inp), tu.run_oracle(inp), tu.real_token_mask(inp))
    _check(errs, 2e-2, "empty sequences")
    got = tu.run_gpu(inp)
    for n in (0, 2, 3, 6):   # the empty sequences pass dht through
        assert torch.equal(got["dh0"][n], inp["dht"][n]), n


def test_varlen_more_sequences_than_one_table_pass():
    """300 packed sequences (lengths 1..23, K = V = 64): the chunk table takes
    its sequences 256 at a time, so this runs its multi-pass path; every element
    of every output compared."""
    gen = torch.Generator().manual_seed(61)
    lens = torch.randint(1, 24, (300,), generator=gen)
    cu = torch.zeros(301, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    T = int(cu[-1])
    w = scaled(VARLEN, T=T, H=2, Hg=2, K=64, V=64, n_seqs=1, seed=61)
    inp = make_inputs(w)
    inp["cu_seqlens"] = cu
    inp["h0"] = torch.randn(300, w.H, w.K, w.V, generator=gen) * 0.1
    inp["dht"] = torch.randn(300, w.H, w.K, w.V, generator=gen) * 0.1
    gpu = tu.run_gpu(inp)
    ref = tu.run_oracle(inp)
    _check(tu.rel_errors(gpu, ref, tu.real_token_mask(inp)), tu.tolerance(w), "varlen 300 sequences")


def test_varlen_longest_first_order():
    """The chunk table's longest-first sequence order, which sets the state
    sweeps' block order: a permutation of the sequences with non-increasing
    chunk counts (counts of 1023 chunks or more share its top bucket), next to
    the chunk offsets; empty sequences and one sequence past the top bucket
    included, every output compared with the oracle."""
    import chunked_gated_delta_gdr_amd as gdr
    gen = torch.Generator().manual_seed(67)
    lens = torch.randint(0, 300, (40,), generator=gen)
    lens[3] = 0
    lens[17] = 1025 * 64 - 5          # 1025 chunks
    lens[29] = 1023 * 64              # 1023 chunks
    cu = torch.zeros(41, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    T = int(cu[-1])
    w = scaled(VARLEN, T=T, H=1, Hg=1, K=64, V=64, n_seqs=0, seed=67)   # lengths set below
    inp = make_inputs(w)
    inp["cu_seqlens"] = cu
    inp["h0"] = torch.randn(40, w.H, w.K, w.V, generator=gen) * 0.1
    inp["dht"] = torch.randn(40, w.H, w.K, w.V, generator=gen) * 0.1
    desc = gdr.make_desc(1, T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, n_seqs=40, io_dtype=w.io_dtype)
    offs = gdr.workspace_offsets(desc)
    ws = torch.zeros(offs["total"], dtype=torch.uint8, device="cuda")
    gpu = tu.run_gpu(inp, workspace=ws)
    words = ws[offs["seq_off"]: offs["seq_off"] + 4 * 81].cpu().view(torch.int32).numpy()
    nch = (lens.numpy() + 63) // 64
    assert list(words[:41]) == [0] + list(np.cumsum(nch))
    order = words[41:81]
    assert sorted(order.tolist()) == list(range(40))
    capped = np.minimum(nch[order], 1023)
    assert np.all(np.diff(capped) <= 0), capped
    assert set(order[:2].tolist()) == {17, 29}
    ref = tu.run_oracle(inp)
    _check(tu.rel_errors(gpu, ref, tu.real_token_mask(inp)), tu.tolerance(w), "varlen longest first")
