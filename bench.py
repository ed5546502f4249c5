"""Benchmark of the Engram layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--no-cpu-baseline]

One step is one full layer forward (hash, gather, projections, gate, conv and
residual) over one batch of the workload, with every input already resident
in HBM.  Prints one JSON line (see the design notes for the fields).

The default workload is the single-branch bf16 layer: B = 1 sequence of
T = 4096 tokens (Zipf(1.1) ids over a 128,000-id vocabulary, projected to
98,560), 2 orders x 8 heads of 64-dim bf16 rows in 16 prime-sized tables
(10,344,164 rows, 1.32 GB), d = d_mem = 1024.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram layer tokens/s at T=4096 (lookup+gate+conv); gather HBM GB/s"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=[1, 2])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    return ap.parse_args()


def stage_units(w, lay):
    """Algorithmic bytes (HBM-bound kernels) or flops (matrix-core kernels)
    per launch of each kernel of the layer forward, keyed by the kernel names
    the library reports."""
    n_tok = w.B * w.T
    nt = lay.hash.n_tables
    dim = lay.tables.dim
    d, M = lay.d, lay.branches
    es = 2 if w.dtype == "bf16" else 4
    i8 = lay.tables.dtype == "i8"
    row_bytes = dim * (1 if i8 else es) + (4 if i8 else 0)
    d_mem = nt * dim
    fused = w.dtype == "bf16" and d % 128 == 0
    n_stat = (1 + M) * d // 128 if fused else 1 + M
    flops = 2.0 * n_tok * (1 + M) * d * d_mem
    return {
        # token ids in; rows in; e out
        "gather_kernel<hashed>": ("hbm", n_tok * (4 + nt * (row_bytes + dim * es))),
        "proj_gate_kernel": ("mfma", flops),
        "gemm_kernel": ("mfma", flops),
        # h, k, v in; statistics out
        "gate_stats_kernel": ("hbm", n_tok * (M * 2 * d * 4 + d * 4 + M * d * es + 16 * n_stat)),
        # v (float32) and statistics in; H in and out; alpha, gamma out
        "conv_kernel": ("hbm", n_tok * (d * 4 + 16 * n_stat + M * (2 * d * es + 8))),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not part "
                                   "of this build (see the design notes on sharding)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from hashed_gram_embedding_amd import engram as eg
    from hashed_gram_embedding_amd import inputs

    dev = "cuda"
    w = inputs.make_config(args.config)
    lay = w.layers[0]
    L = eg.Layer(lay, w.dtype, dev)
    tok = torch.from_numpy(w.tokens).to(dev)
    H = eg.to_device(w.H, w.dtype, dev)
    n_tok = w.B * w.T
    ws = torch.empty(eg.forward_workspace(w.B, w.T, L), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        eg.forward(tok, H, L, ws=ws)            # on the current stream

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the step is captured once into a HIP graph and replayed, so that host
    # launch overhead does not pace a step of a few tens of microseconds
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):           # captures on a side stream
            step()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps

    # per-kernel durations: HIP events that the library records on the launch
    # stream around each kernel of the same forward (eager launches)
    eg.profile_enable(True)
    acc = {}
    for it in range(args.warmup + args.steps):
        step()
        for name, t in eg.profile_read():
            if it >= args.warmup:
                acc[name] = acc.get(name, 0.0) + t
    eg.profile_enable(False)
    stage_ms = {k: v / args.steps for k, v in acc.items()}

    units = stage_units(w, lay)
    rates = {}
    for k, t in stage_ms.items():
        if k in units:
            kind, amount = units[k]
            rates[k] = amount / (t * 1e-3) / (1e9 if kind == "hbm" else 1e12)
    dominant = max((k for k in stage_ms if k in units), key=lambda k: stage_ms[k])
    kind, amount = units[dominant]
    if kind == "mfma":
        roof = {"bound": "mfma", "kernel": dominant, "achieved": round(rates[dominant], 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(rates[dominant] / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "units_per_launch": amount}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": round(rates[dominant], 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(rates[dominant] / PEAK_HBM_GBPS, 4),
                "traffic": None, "units_per_launch": amount}
    gather_gbps = rates.get("gather_kernel<hashed>")
    gemm_tflops = rates.get("proj_gate_kernel", rates.get("gemm_kernel"))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_budget_s)

    out = {
        "metric": METRIC,
        "value": round(n_tok / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) tables, N(0,1) hidden states)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "branches": lay.branches, "d": lay.d,
                   "d_mem": lay.d_mem, "tables": lay.hash.n_tables, "table_rows": lay.tables.total_rows,
                   "table_dtype": lay.tables.dtype},
        "timing": "HIP graph replay" if graph is not None else "eager launches",
        "gather_GBps": None if gather_gbps is None else round(gather_gbps, 1),
        "gemm_TFLOPs": None if gemm_tflops is None else round(gemm_tflops, 2),
        "kernel_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "kernel_rate": {k: round(v, 2) for k, v in rates.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, budget_s):
    """The CPU oracle (float64, numpy) on a bounded sample of the same workload:
    whole forward passes over the first T_s tokens, repeated until the budget is
    used; reported as tokens/s."""
    from oracle import engram_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    lay = w.layers[0]
    Ts = min(w.T, 1024)
    tok = w.tokens[:1, :Ts]
    Hs = w.H[:1, :Ts]
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.forward(tok, Hs, lay, w.dtype)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    return {"value": round(n * Ts / el, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} forward passes of the float64 oracle over the first {Ts} tokens of sequence 0 "
                      f"({el:.1f} s); cores = BLAS threads (the rest of the oracle is single-threaded numpy)"}


if __name__ == "__main__":
    main()
