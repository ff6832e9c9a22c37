#!/usr/bin/env python3
"""Benchmark of the chunkwise gated delta-rule backward on one MI355X.

One step = one gdr_bwd call over one batch of seeded synthetic inputs already
resident in HBM: chunk table, per-chunk preparation, both state sweeps and
the chunk gradients (every step of the hot path). W untimed warmup steps,
then K timed steps between two device synchronisations, timed with HIP
events on the stream the kernels run on; the per-kernel times come from
events recorded at the kernel boundaries inside the same timed steps.

Prints one JSON line. `value` is tokens/s (B*T per second of the whole
backward). `roofline` is the whole backward against the HBM peak: the method's
algorithmic bytes (inputs read once, outputs written once, one write and one
read of the per-chunk state) over the time per step, with the summed counter
traffic of the four kernels; `roofline.kernels` holds the same record for
each kernel (its own algorithmic bytes in this four-kernel decomposition, its
time from the stage events, its counter traffic, MFMA busy and LDS bank
conflicts) and `roofline.dominant` names the longest one. `cpu_baseline`
times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 / fp16 MFMA, datasheet
MFMA_FP32_PEAK_TFS = 157.3
METRIC = "gated-delta-rule bwd tokens/s (B*T) at H=16,K=V=128; % of MFMA/HBM roofline"


def per_token_head_costs(w, n_chunks: int, n_seqs: int, tokens: int) -> dict:
    """Algorithmic bytes and FLOPs of the method, per value token-head.

    bytes: inputs read once + outputs written once + one write and one read of
    the per-chunk state h in io precision + h0 / dht / dh0 per (sequence, head).
    FLOPs: 8 K x V products of C rows per chunk (16 C K V), 14 C x C x D
    products on the lower triangle, C^3 for the triangular inverse and its
    gradient.
    """
    import torch
    es = 4 if w.io_dtype == torch.float32 else 2
    K, V, C, H, Hg = w.K, w.V, w.chunk, w.H, w.Hg
    gbytes = K * 4 if w.gate == "kda" else 4
    th = tokens * H
    qk = 2 * K * es * Hg / H
    inp = qk + 2 * V * es + gbytes + es
    out = qk + V * es + gbytes + es
    state = 2 * K * V * es * n_chunks * H / th          # h written once, read once
    ends = 3 * K * V * 4 * n_seqs * H / th              # h0, dht, dh0
    f = (C + 1) / (2 * C)
    flops_chunk = 16 * C * K * V + 2 * C * C * f * (9 * K + 5 * V) + C ** 3
    flops = flops_chunk * n_chunks * H / th
    return dict(method_bytes=inp + out + state + ends, io_bytes=inp + out + ends, flops=flops)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, budget_s: float = 20.0, min_s: float = 10.0) -> dict:
    """Time the fp64 oracle on a bounded head sample of the same workload."""
    import oracle
    from gdr_workloads import head_subset
    w = inp["workload"]
    # probe: one q/k head group (all sequences) gives the cost per group
    sub, _ = head_subset(inp, [0])
    t0 = time.perf_counter()
    oracle.run(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["do"], sub["h0"],
               sub["dht"], sub["cu_seqlens"], inp["scale"], w.gate)
    t_group = time.perf_counter() - t0
    threads = oracle.threads()
    n_groups = w.Hg
    # groups run in parallel across threads (one task per (sequence, group))
    est_all = t_group * max(1.0, n_groups * (w.B if not w.varlen else 1) / threads)
    if est_all <= budget_s:
        hks = list(range(n_groups))
    else:
        k = max(1, int(n_groups * budget_s / est_all))
        hks = list(range(k))
    sub, hv = head_subset(inp, hks)
    # repeat the sample until about min_s of CPU time has been measured
    reps, total = 0, 0.0
    while total < min_s and total < budget_s:
        t0 = time.perf_counter()
        oracle.run(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["do"], sub["h0"],
                   sub["dht"], sub["cu_seqlens"], inp["scale"], w.gate)
        total += time.perf_counter() - t0
        reps += 1
    t = total / reps
    frac = len(hv) / w.H
    tokens = inp["tokens"]
    return {"value": tokens * frac / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(hv)} of {w.H} value heads, all {tokens} tokens, {reps} run(s) "
                      f"({t:.2f} s each, fp64 on the host; value scaled to all heads)"}


# ---------------------------------------------------------------------------
# Algorithmic bytes of each kernel in the four-kernel decomposition
# ---------------------------------------------------------------------------
KERNELS = ("gdr_chunk_table", "gdr_prep", "gdr_sweep", "gdr_chunk_bwd")
STAGE_OF = dict(zip(KERNELS, ("chunk_table", "prep", "sweep", "chunk_bwd")))


def sweep_is_wide(w, n_seqs: int, cus: int = 256) -> bool:
    """The launcher's V-tile choice for a backward (both sweep directions):
    64-column tiles when 32-column tiles would fill the CUs twice over."""
    return 2 * n_seqs * w.H * (w.K // 32) >= 2 * cus


def kernel_bytes(w, n_chunks: int, n_seqs: int) -> dict:
    """Bytes each kernel must move (read once, write once) in this
    decomposition, per step: its inputs and outputs among the caller's tensors
    and the workspace regions it writes or reads. q / k count once per q/k
    head (a GQA group's value heads share them)."""
    import torch
    es = 4 if w.io_dtype == torch.float32 else 2
    C, D, H, G = w.chunk, w.K, w.H, w.H // w.Hg
    gb = D * 4 if w.gate == "kda" else 4
    ch = n_chunks * H            # (chunk, value head) items
    sh = n_seqs * H              # (sequence, value head) pairs
    qk = 2 * C * D * es / G      # q, k rows of one chunk, per value head
    tok_in = C * (D * es + gb + es)          # v, g, beta of one chunk-head
    # the preparation also stores w^T and k~^T for a sweep that does not
    # transpose w, k~ itself (fp32, K = 64, or 64-column tiles at C = 64)
    wide = sweep_is_wide(w, n_seqs)
    store_a2t = es == 4 or D != 128 or (C == 64 and wide)
    factors = 2 * C * C * es + 4 * C * D * es + D * 4        # scale Aqk^T, A, w, k~, u^T, scale q~^T, 2^G_last
    prep = ch * (qk + tok_in + factors + (2 * C * D * es if store_a2t else 0))
    states = 2 * D * D * es                                   # h, dh of one chunk-head
    xt = 2 * C * D * es                                       # X, T
    sweep = ch * (3 * C * D * es + D * 4                      # forward: w, k~ (or k~^T), u^T, 2^G_last
                  + 3 * C * D * es + D * 4 + C * D * es       # reverse: k~, w (or w^T), scale q~^T, 2^G_last, do
                  + states + xt) + sh * 3 * D * D * 4         # h0, dht, dh0
    grad_in = qk + C * D * es + tok_in + xt + states + 2 * C * C * es + D * 4   # + do, X, T, h, dh, A, Aqk^T
    grad_out = qk + C * (D * es + gb + es)                    # dq, dk, dv, dg, db
    chunk_bwd = ch * (grad_in + grad_out)
    table = n_seqs * 8 + n_chunks * 16
    return {"gdr_chunk_table": table, "gdr_prep": prep, "gdr_sweep": sweep, "gdr_chunk_bwd": chunk_bwd}


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries (profiles/gdr_counters_<workload>.md)
# ---------------------------------------------------------------------------
# Four passes over the same bench.py command, each a run of its own: FETCH_SIZE,
# WRITE_SIZE (both with --copy-probe, whose plain copy of known size scales the
# KiB they read into bytes), the derived MfmaUtil and LDSBankConflict, and raw
# MFMA / LDS counts. Every kernel's row carries a hash of that kernel's own
# sources; a row whose hash no longer matches the tree describes another build
# of the kernel and its figures are reported as null.
CSRC = "chunked_gated_delta_gdr_amd/csrc/"
KERNEL_SOURCES = {
    "gdr_chunk_table": ("gdr_prep.hpp", "gdr_common.hpp", "gdr_launch.hpp"),
    "gdr_prep": ("gdr_prep.hpp", "gdr_common.hpp", "gdr_launch.hpp"),
    "gdr_sweep": ("gdr_sweep.hpp", "gdr_sweep_ws.hpp", "gdr_common.hpp", "gdr_launch.hpp"),
    "gdr_chunk_bwd": ("gdr_chunk_bwd.hpp", "gdr_common.hpp", "gdr_launch.hpp"),
}
COPY_KERNEL_KEY = "neg_kernel"   # torch.neg(out=...): reads N bytes, writes N bytes
COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "util": ["MfmaUtil", "LDSBankConflict"],
    "raw": ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
            "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
}


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, CSRC, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"gdr_counters_{workload}.md")


def stored_counters(workload: str) -> dict:
    """{kernel: {field: value}} from the committed counter summary; a kernel
    whose stored source hash differs from the tree's maps to None."""
    p = counters_summary_path(workload)
    out = {k: None for k in KERNELS}
    if not os.path.exists(p):
        return out
    kv = {}
    for line in open(p):
        parts = line.strip().split(" = ")
        if len(parts) == 2 and "." in parts[0]:
            kv[parts[0].strip()] = parts[1].strip()
    for k in KERNELS:
        if kv.get(f"{k}.source_sha256") != kernel_source_hash(k):
            continue
        rec = {}
        for f in ("traffic_bytes", "read_bytes", "write_bytes", "mfma_util_pct", "lds_bank_conflict_pct",
                  "mfma_flops", "lds_conflict_cycles_per_active"):
            try:
                rec[f] = float(kv[f"{k}.{f}"])
            except (KeyError, ValueError):
                rec[f] = None
        out[k] = rec
    return out


def _read_counter_csv(path: str) -> dict:
    """{(kernel name, counter): [value per dispatch]} from a rocprofv3
    counter_collection.csv, plus {kernel: resource row} under key None."""
    import csv
    vals, res = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
            res[r["Kernel_Name"]] = {c: r.get(c, "") for c in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
                                                                "LDS_Block_Size", "Scratch_Size",
                                                                "Workgroup_Size", "Grid_Size")}
    return {"vals": vals, "res": res}


def _kernel_name(names, kernel: str):
    # the sweep has two kernels: gdr_sweep, and gdr_sweep_ws (loader waves)
    keys = (f"{kernel}<", f"{kernel}I") + ((f"{kernel}_wsI",) if kernel == "gdr_sweep" else ())
    m = [n for n in names if any(k in n for k in keys)]
    if len(m) > 1:
        raise SystemExit(f"several kernels match {kernel!r}: {m}")
    return m[0] if m else None


def summarize_counters(base: str, copy_mib: float, workload: str, command: str) -> str:
    """Text summary of the four counter passes found under base/<pass>/."""
    import glob
    data = {}
    for ps in COUNTER_PASSES:
        files = glob.glob(os.path.join(base, ps, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"pass {ps}: expected one counter_collection.csv under {base}/{ps}, found {files}")
        data[ps] = _read_counter_csv(files[0])

    def mean(ps, kname, counter):
        v = data[ps]["vals"].get((kname, counter))
        return sum(v) / len(v) if v else None

    names = set(n for d in data.values() for (n, _c) in d["vals"])
    copy_k = [n for n in names if COPY_KERNEL_KEY in n]
    if len(copy_k) != 1:
        raise SystemExit(f"expected one copy kernel, found {copy_k}")
    copy_bytes = copy_mib * 2 ** 20
    fs = copy_bytes / (mean("fetch", copy_k[0], "FETCH_SIZE") * 1024)
    ws = copy_bytes / (mean("write", copy_k[0], "WRITE_SIZE") * 1024)
    lines = [f"# rocprofv3 counters per kernel, workload {workload}", "",
             "Four passes of the same command, each a run of its own (FETCH_SIZE; WRITE_SIZE; the derived",
             "MfmaUtil and LDSBankConflict; raw MFMA / LDS counts). FETCH_SIZE and WRITE_SIZE (KiB per",
             f"dispatch) are scaled by what they read for a plain copy of {copy_mib:g} MiB run in the same",
             "program (torch.neg: reads and writes that many bytes). Each kernel's `source_sha256` hashes",
             "its own sources; bench.py reports a kernel's figures only while that hash matches the tree.",
             "", "Command of every pass (`<counters>` per pass as above):", "", "```", command, "```", "",
             "```", f"workload = {workload}", f"copy.fetch_scale = {fs:.4f}", f"copy.write_scale = {ws:.4f}"]
    table = ["| kernel | read MB | write MB | traffic MB | MfmaUtil % | LDSBankConflict % | MFMA GFLOP "
             "| LDS conflict / active | VGPR / AGPR | LDS bytes | scratch |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in KERNELS:
        kn = _kernel_name(names, k)
        if kn is None:
            continue
        fk, wk = mean("fetch", kn, "FETCH_SIZE"), mean("write", kn, "WRITE_SIZE")
        rd, wr = fk * 1024 * fs, wk * 1024 * ws
        mu, lb = mean("util", kn, "MfmaUtil"), mean("util", kn, "LDSBankConflict")
        mops = sum(mean("raw", kn, c) or 0.0 for c in COUNTER_PASSES["raw"][:3])
        la, lc = mean("raw", kn, "SQ_LDS_IDX_ACTIVE"), mean("raw", kn, "SQ_LDS_BANK_CONFLICT")
        ratio = lc / (la - lc) if la and la > lc else 0.0
        res = data["raw"]["res"].get(kn, {})
        lines += [f"{k}.source_sha256 = {kernel_source_hash(k)}", f"{k}.kernel_name = {kn[:120]}",
                  f"{k}.fetch_kib = {fk:.1f}", f"{k}.write_kib = {wk:.1f}",
                  f"{k}.read_bytes = {rd:.0f}", f"{k}.write_bytes = {wr:.0f}",
                  f"{k}.traffic_bytes = {rd + wr:.0f}", f"{k}.mfma_util_pct = {mu:.3f}",
                  f"{k}.lds_bank_conflict_pct = {lb:.3f}", f"{k}.mfma_flops = {mops * 512:.0f}",
                  f"{k}.lds_conflict_cycles_per_active = {ratio:.4f}"]
        table.append(f"| {k} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / 1e6:.1f} | {mu:.2f} | {lb:.2f} | "
                     f"{mops * 512 / 1e9:.2f} | {ratio:.3f} | {res.get('VGPR_Count', '')} / "
                     f"{res.get('Accum_VGPR_Count', '')} | {res.get('LDS_Block_Size', '')} | "
                     f"{res.get('Scratch_Size', '')} |")
    lines += ["```", "", "Per launch (one dispatch of each kernel; averages over the profiled dispatches):", ""]
    lines += table
    return "\n".join(lines) + "\n"


def summarize_kernel_stats(stats_csv: str) -> str:
    """Markdown table from a rocprofv3 --stats kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["| kernel | calls | average (us) | min (us) | max (us) | share (%) |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    return "\n".join(lines) + "\n"


def bench_fwd(args, w, inp, t, tokens, n_chunks, n_seqs, ws) -> int:
    """The forward pass (o and the final states) on the same workload: total
    time per call with HIP events on the launch stream."""
    import torch
    import chunked_gated_delta_gdr_amd as gdr
    dev = t["q"].device
    o = torch.empty_like(t["v"])
    ht = torch.empty((n_seqs, w.H, w.K, w.V), dtype=torch.float32, device=dev)

    def step():
        gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                scale=inp["scale"], chunk_size=w.chunk, workspace=ws, out=(o, ht))

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    es = 4 if w.io_dtype == torch.float32 else 2
    th = tokens * w.H
    # bytes: q, k, v, g, beta read once, o written once, the per-chunk state
    # written once and read once, h0 read and ht written per (sequence, head)
    qk = 2 * w.K * es * w.Hg / w.H
    gb = w.K * 4 if w.gate == "kda" else 4
    per_th = qk + w.V * es + gb + es + w.V * es + 2 * w.K * w.V * es * n_chunks * w.H / th \
        + 2 * w.K * w.V * 4 * n_seqs * w.H / th
    res = {
        "metric": "gated-delta-rule fwd tokens/s (B*T) at H=16,K=V=128",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[w.io_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "fwd", "tokens": tokens, "H": w.H, "Hg": w.Hg, "K": w.K,
                   "V": w.V, "chunk": w.chunk, "gate": w.gate, "n_seqs": n_seqs,
                   "parallelism": "single-gpu"},
        "step_roofline": {"method_bytes": per_th * th,
                          "hbm_frac": per_th * th / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_fused(args, w, inp, t, tokens, n_chunks, n_seqs) -> int:
    """The fused reverse backward (gdr_bwd_fused, chunk 32): the same backward
    as the headline step with the reverse sweep and the chunk gradients in one
    kernel per (sequence, value head); whole-call time with HIP events on the
    launch stream, the method's bytes as for the step."""
    import torch
    import chunked_gated_delta_gdr_amd as gdr
    dev = t["q"].device
    out = (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]),
           torch.empty_like(t["g"]), torch.empty_like(t["beta"]),
           torch.empty((n_seqs, w.H, w.K, w.V), dtype=torch.float32, device=dev))
    desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, n_seqs=w.n_seqs,
                         gate=0 if w.gate == "kda" else 1, io_dtype=w.io_dtype)
    ws = torch.empty(int(gdr._load().gdr_bwd_fused_workspace_bytes(__import__("ctypes").byref(desc))),
                     dtype=torch.uint8, device=dev)

    def step():
        gdr.bwd_fused(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=t["h0"], dht=t["dht"],
                      cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk, workspace=ws, out=out)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    costs = per_token_head_costs(w, n_chunks, n_seqs, tokens)
    mb = costs["method_bytes"] * tokens * w.H
    res = {
        "metric": "gated-delta-rule bwd tokens/s (B*T), fused reverse kernel (chunk 32)",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[w.io_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "fused", "tokens": tokens, "H": w.H, "Hg": w.Hg, "K": w.K,
                   "V": w.V, "chunk": w.chunk, "gate": w.gate, "n_seqs": n_seqs,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "scope": "step", "achieved": mb / (ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": mb},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_train(args, w, inp, t, tokens, n_chunks, n_seqs, ws) -> int:
    """A training step's kernels: the forward pass, then the backward after it
    on the same workspace (gdr_bwd_after_fwd). Times each half and the pair
    with HIP events on the launch stream."""
    import torch
    import chunked_gated_delta_gdr_amd as gdr
    dev = t["q"].device
    o = torch.empty_like(t["v"])
    ht = torch.empty((n_seqs, w.H, w.K, w.V), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]),
             torch.empty_like(t["g"]), torch.empty_like(t["beta"]),
             torch.empty((n_seqs, w.H, w.K, w.V), dtype=torch.float32, device=dev))
    common = dict(cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record(stream)
        gdr.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0=t["h0"], workspace=ws, out=(o, ht), **common)
        if e: e[1].record(stream)
        gdr.bwd_after_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], ws, dht=t["dht"], out=grads,
                          **common)
        if e: e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K plain steps; then K steps with events at the
    # fwd / bwd boundary for the split (those markers add a few us)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(stop) / args.steps
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    f = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    b = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    res = {
        "metric": "gated-delta-rule fwd + bwd-after-fwd tokens/s (B*T) at H=16,K=V=128",
        "value": tokens / (total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": total, "fwd_ms": f, "bwd_after_fwd_ms": b,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[w.io_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "train", "tokens": tokens, "H": w.H, "Hg": w.Hg, "K": w.K,
                   "V": w.V, "chunk": w.chunk, "gate": w.gate, "n_seqs": n_seqs,
                   "parallelism": "single-gpu"},
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="kda_fixed_h16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("bwd", "fwd", "train", "fused"), default="bwd",
                    help="bwd (the headline), fwd (the forward pass: o and final states), "
                         "train (the forward pass, then the backward after it on its workspace) or "
                         "fused (the backward through the fused reverse kernel, chunk 32 workloads)")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="MIB",
                    help="after the timed steps, run a plain copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the counter summary of the four rocprofv3 --pmc passes under "
                         "DIR/{fetch,write,util,raw} and exit")
    ap.add_argument("--pmc-command", default="",
                    help="the profiled command, recorded in the counter summary")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="print a table of a rocprofv3 --stats kernel_stats.csv and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.copy_probe or 1024.0, args.workload,
                                 args.pmc_command), end="")
        return 0
    if args.summarize_stats:
        print(summarize_kernel_stats(args.summarize_stats), end="")
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: there is no multi-GPU path here (the backward "
              "shards by sequence or head with no exchange, so N GPUs run N independent "
              "copies of this step). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import chunked_gated_delta_gdr_amd as gdr
    from gdr_workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    tokens = int(inp["cu_seqlens"][-1]) if w.varlen else w.B * w.T
    inp["tokens"] = tokens
    dev = torch.device("cuda", 0)
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    lens = (torch.diff(inp["cu_seqlens"]).tolist() if w.varlen else [w.T] * w.B)
    n_chunks = sum((L + w.chunk - 1) // w.chunk for L in lens)
    n_seqs = len(lens)

    desc = gdr.make_desc(w.B, w.T, w.H, w.Hg, w.K, w.V, chunk=w.chunk, n_seqs=w.n_seqs,
                         gate=0 if w.gate == "kda" else 1, io_dtype=w.io_dtype)
    ws = torch.empty(gdr.workspace_bytes(desc), dtype=torch.uint8, device=dev)
    out = (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]),
           torch.empty_like(t["g"]), torch.empty_like(t["beta"]),
           torch.empty_like(t["h0"]))

    if args.which == "fwd":
        return bench_fwd(args, w, inp, t, tokens, n_chunks, n_seqs, ws)
    if args.which == "train":
        return bench_train(args, w, inp, t, tokens, n_chunks, n_seqs, ws)
    if args.which == "fused":
        return bench_fused(args, w, inp, t, tokens, n_chunks, n_seqs)

    def step(events=None):
        gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=t["h0"], dht=t["dht"],
                cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk,
                workspace=ws, out=out, stage_events=events)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K back-to-back steps, nothing else on the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    # per-kernel durations: K more steps with an event between consecutive
    # kernels on the launch stream (the markers add ~3-4 us per kernel
    # boundary, so this pass is kept out of the timed region above)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    k1.record(stream)
    torch.cuda.synchronize()
    ms_instrumented = k0.elapsed_time(k1) / args.steps
    kernel_ms = {}
    for si, name in enumerate(gdr.STAGES):
        kernel_ms[name] = sum(r[si].elapsed_time(r[si + 1]) for r in evs) / args.steps

    costs = per_token_head_costs(w, n_chunks, n_seqs, tokens)
    th = tokens * w.H
    fp32 = w.io_dtype == torch.float32
    step_s = ms * 1e-3
    method_bytes = costs["method_bytes"] * th
    achieved = method_bytes / step_s / 1e9
    flops = costs["flops"] * th
    mfma_peak = MFMA_FP32_PEAK_TFS if fp32 else MFMA_BF16_PEAK_TFS
    kb = kernel_bytes(w, n_chunks, n_seqs)
    stored = stored_counters(w.name)
    kernels = {}
    for k in KERNELS:
        k_ms = kernel_ms[STAGE_OF[k]]
        rec = stored[k]
        traffic = rec["traffic_bytes"] if rec else None
        kach = kb[k] / (k_ms * 1e-3) / 1e9 if k_ms > 0 else None
        kernels[k] = {"ms": k_ms, "algorithmic_bytes": kb[k], "achieved": kach,
                      "frac": kach / HBM_PEAK_GBS if kach is not None else None,
                      "traffic": traffic,
                      "traffic_over_algorithmic": traffic / kb[k] if traffic and kb[k] else None,
                      "mfma_util_pct": rec["mfma_util_pct"] if rec else None,
                      "lds_bank_conflict_pct": rec["lds_bank_conflict_pct"] if rec else None,
                      "mfma_flops_counted": rec["mfma_flops"] if rec else None}
    traffic_all = [kernels[k]["traffic"] for k in KERNELS]
    res = {
        "metric": METRIC,
        "value": tokens / step_s,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[w.io_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "tokens": tokens, "H": w.H, "Hg": w.Hg,
                   "K": w.K, "V": w.V, "chunk": w.chunk, "sub_chunk": 16, "gate": w.gate,
                   "n_seqs": n_seqs, "parallelism": "single-gpu"},
        # the whole backward (all four kernels of one step) against the HBM peak
        "roofline": {"bound": "hbm", "scope": "step", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": sum(traffic_all) if all(x is not None for x in traffic_all) else None,
                     "algorithmic_bytes": method_bytes,
                     "decomposition_bytes": sum(kb.values()),
                     "io_floor_frac": costs["io_bytes"] * th / step_s / 1e9 / HBM_PEAK_GBS,
                     "mfma": {"flops": flops, "achieved": flops / step_s / 1e12, "peak": mfma_peak,
                              "unit": "TFLOP/s", "frac": flops / step_s / 1e12 / mfma_peak},
                     "dominant": max(KERNELS, key=lambda k: kernels[k]["ms"]),
                     "kernels": kernels},
        "kernels_ms": kernel_ms,
        # the per-kernel pass: its step time with the inter-kernel events
        "kernels_pass_ms_per_step": ms_instrumented,
        "wall_ms_per_step": t_wall * 1e3 / args.steps,
    }
    if args.copy_probe > 0:
        n = int(args.copy_probe * 2 ** 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
