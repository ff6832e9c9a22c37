#!/usr/bin/env python3
"""Benchmark of the chunkwise gated delta-rule backward on one MI355X.

One step = one gdr_bwd call over one batch of seeded synthetic inputs already
resident in HBM: chunk table, per-chunk preparation, both state sweeps and
the chunk gradients (every step of the hot path). W untimed warmup steps,
then K timed steps between two device synchronisations, timed with HIP
events on the stream the kernels run on; the per-kernel times come from
events recorded at the kernel boundaries inside the same timed steps.

Prints one JSON line. `value` is tokens/s (B*T per second of the whole
backward). `roofline` reports the dominant kernel against the HBM peak with
its algorithmic bytes; `cpu_baseline` times the fp64 oracle on the host.
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
    # the chunk-gradient kernel alone: its inputs, outputs and the two states it reads
    k_bytes = inp + out + state
    return dict(method_bytes=inp + out + state + ends, io_bytes=inp + out + ends,
                flops=flops, chunk_bwd_bytes=k_bytes)


def cpu_baseline(inp, budget_s: float = 20.0, min_s: float = 10.0) -> dict:
    """Time the fp64 oracle on a bounded head sample of the same workload."""
    import numpy as np  # noqa: F401
    import oracle
    from gdr_workloads import head_subset
    w = inp["workload"]
    G = w.H // w.Hg
    # probe: one q/k head group on the first sequence only gives the per-token cost
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
            "sample": f"{len(hv)} of {w.H} value heads, all {tokens} tokens, {reps} run(s) "
                      f"({t:.2f} s each, fp64 on the host; value scaled to all heads)"}


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel from rocprofv3 counters
# ---------------------------------------------------------------------------
# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same counters
# read for a plain elementwise copy of known size (`--copy-probe`), so the
# result is in true bytes. The figures live in a text summary under profiles/
# together with a hash of the kernel's sources; once the sources change the
# stored figure no longer describes the kernel and `traffic` is reported null.
KERNEL_SOURCES = ("chunked_gated_delta_gdr_amd/csrc/gdr_chunk_bwd.hpp",
                  "chunked_gated_delta_gdr_amd/csrc/gdr_common.hpp")
COPY_KERNEL_KEY = "neg_kernel"   # torch.neg(out=...): reads N bytes, writes N bytes


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"gdr_chunk_bwd_{workload}_traffic.md")


def stored_traffic(workload: str):
    """Bytes per launch from the committed counter summary, or None if there is
    none or it was taken on other sources of the kernel."""
    p = traffic_summary_path(workload)
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        parts = line.strip().split("=")
        if len(parts) == 2 and parts[0].strip().isidentifier():
            kv[parts[0].strip()] = parts[1].strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _read_counter_csv(path: str, counter: str) -> dict:
    """{kernel name: [value per dispatch in KiB]} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(d: dict, key: str):
    names = [n for n in d if key in n]
    if len(names) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {names}")
    return d[names[0]]


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: float, workload: str) -> str:
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * 2 ** 20
    cf, cw = _pick(fetch, COPY_KERNEL_KEY), _pick(write, COPY_KERNEL_KEY)
    f_copy = copy_bytes / (sum(cf) / len(cf) * 1024)
    w_copy = copy_bytes / (sum(cw) / len(cw) * 1024)
    kf, kw = _pick(fetch, "gdr_chunk_bwd"), _pick(write, "gdr_chunk_bwd")
    rd = sum(kf) / len(kf) * 1024 * f_copy
    wr = sum(kw) / len(kw) * 1024 * w_copy
    lines = [
        f"# gdr_chunk_bwd HBM traffic, workload {workload}",
        "",
        "rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one pass each, scaled by the",
        f"same counters on a plain copy of {copy_mib:g} MiB (torch.neg, reads and writes "
        f"{copy_mib:g} MiB).",
        "",
        "```",
        f"workload = {workload}",
        f"kernel_source_sha256 = {kernel_source_hash()}",
        f"copy_fetch_kib = {sum(cf) / len(cf):.1f}",
        f"copy_write_kib = {sum(cw) / len(cw):.1f}",
        f"fetch_scale = {f_copy:.4f}",
        f"write_scale = {w_copy:.4f}",
        f"kernel_fetch_kib = {sum(kf) / len(kf):.1f}",
        f"kernel_write_kib = {sum(kw) / len(kw):.1f}",
        f"read_bytes_per_launch = {rd:.0f}",
        f"write_bytes_per_launch = {wr:.0f}",
        f"traffic_bytes_per_launch = {rd + wr:.0f}",
        "```",
        "",
        "Per dispatch (KiB, raw):",
        "",
        "| kernel | FETCH_SIZE | WRITE_SIZE |",
        "|---|---|---|",
    ]
    for name in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(name, [0.0]), write.get(name, [0.0])
        lines.append(f"| `{name[:90]}` | {sum(fv) / len(fv):.1f} | {sum(wv) / len(wv):.1f} |")
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
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    f = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    b = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    res = {
        "metric": "gated-delta-rule fwd + bwd-after-fwd tokens/s (B*T) at H=16,K=V=128",
        "value": tokens / ((f + b) * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": f + b, "fwd_ms": f, "bwd_after_fwd_ms": b,
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
    ap.add_argument("--pass", dest="which", choices=("bwd", "fwd", "train"), default="bwd",
                    help="bwd (the headline), fwd (the forward pass: o and final states) or "
                         "train (the forward pass, then the backward after it on its workspace)")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="MIB",
                    help="after the timed steps, run a plain copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="print a table of a rocprofv3 --stats kernel_stats.csv and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.copy_probe or 1024.0, args.workload),
              end="")
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

    def step(events=None):
        gdr.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], h0=t["h0"], dht=t["dht"],
                cu_seqlens=t["cu_seqlens"], scale=inp["scale"], chunk_size=w.chunk,
                workspace=ws, out=out, stage_events=events)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-step stage events (created by one record so their handles exist)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    kernel_ms = {}
    for si, name in enumerate(gdr.STAGES):
        kernel_ms[name] = sum(r[si].elapsed_time(r[si + 1]) for r in evs) / args.steps

    costs = per_token_head_costs(w, n_chunks, n_seqs, tokens)
    th = tokens * w.H
    k_ms = kernel_ms["chunk_bwd"]
    k_bytes = costs["chunk_bwd_bytes"] * th
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    fp32 = w.io_dtype == torch.float32
    step_s = ms * 1e-3
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
        "roofline": {"bound": "hbm", "kernel": "gdr_chunk_bwd", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic(w.name),
                     "algorithmic_bytes": k_bytes, "ms": k_ms},
        "step_roofline": {
            "method_bytes": costs["method_bytes"] * th,
            "hbm_frac": costs["method_bytes"] * th / step_s / 1e9 / HBM_PEAK_GBS,
            "io_floor_frac": costs["io_bytes"] * th / step_s / 1e9 / HBM_PEAK_GBS,
            "flops": costs["flops"] * th,
            "mfma_frac": costs["flops"] * th / step_s / 1e12 /
                         (MFMA_FP32_PEAK_TFS if fp32 else MFMA_BF16_PEAK_TFS)},
        "kernels_ms": kernel_ms,
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
