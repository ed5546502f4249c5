"""Benchmark of the Engram layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--no-cpu-baseline] [--eager]

One step is one pass of the whole layer path (hash, gather, projections,
gate, conv and residual) over one batch, with every input already resident
(in HBM, or in pinned host memory for the host-table configuration).  The
timed steps go round a rotation of distinct seeded batches (token ids and
hidden states), enough of them that the table rows one batch reads have left
the 256 MB Infinity Cache before that batch comes round again; rows shared
between batches (frequent n-grams) stay cached as they would in a stream of
real text.  Prints one JSON line.

--config 1 (default; the metric's workload): single-branch bf16 layer, B = 1
    sequence of T = 4096 tokens (Zipf(1.1) ids over a 128,000-id vocabulary,
    projected to 98,560), 2 orders x 8 heads of 64-dim bf16 rows in 16
    prime-sized tables (10,344,164 rows, 1.32 GB), d = d_mem = 1024.  The
    line also carries the other workloads under "secondary" (--no-secondary
    skips them).
--config 2: the same tables with M = 4 branches, B = 8, T = 4096.
--config 3: decode: 256 sequences x 1 new token through 2 layers with int8
    rows (+ float32 row scales), after a 16-token prefill of each sequence.
--config 4: B = 4, T = 4096 through 2 layers whose tables (33,556,876 rows,
    4.3 GB each) live in pinned host memory, with an HBM cache of the 10 % most
    frequent rows (static LFU admission over a 2^24-token warm-up stream).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram layer tokens/s at T=4096 (lookup+gate+conv); gather HBM GB/s"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_PCIE_GBPS = 64.0        # PCIe Gen5 x16, one direction (host-resident table rows)

WARMUP_FLOOR_MS = 100.0   # least untimed warm-up before the timed steps
PROFILE_CHUNK_STEPS = 10  # steps launched back to back between reads of the kernel events (a graph's length)
QUEUE_AHEAD_MS = 2.0      # spin ahead of each such run, while the host queues its launches
QUEUE_AHEAD_MAX_STEP_MS = 0.2   # ... for steps shorter than this (longer ones keep the queue full)
ROTATION_BYTES = 512 << 20   # table rows a rotation of batches touches: twice the Infinity Cache
CPU_HALO = 11                # positions before a token that its layer output depends on: (N-1) + (w-1)*N


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="config 1: skip the other workloads (multi-branch, decode, host tables) in the line")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of HIP graphs")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="CPU time of the oracle baseline (whole batch on every core, then one core)")
    ap.add_argument("--ring", type=int, default=0,
                    help="distinct batches in the timed rotation (default: enough to touch 512 MiB of rows; "
                         "1 replays one batch, the cache-resident control)")
    ap.add_argument("--overlap", action="store_true",
                    help="also measure retrieval (Steps 1-4) run ahead on a second stream: hidden behind a "
                         "stand-in for the preceding layers, and pipelined across batches")
    ap.add_argument("--mxfp8", action="store_true",
                    help="configs 1-2: Step 5 as the MXFP8 product (E4M3 operands with 32-value block scales) "
                         "instead of bf16")
    ap.add_argument("--hot-tier", type=int, default=0, metavar="N",
                    help="configs 1-2: attach an Engram-Nine hot tier holding the N most frequent 2-grams and the "
                         "N most frequent 3-grams of a seeded 2M-token Zipf(1.1) warm-up stream")
    ap.add_argument("--realtime-lfu", action="store_true",
                    help="host-table workload: drift the token distribution and measure the static cache against "
                         "the real-time LFU update (hit rate, step time, update time)")
    ap.add_argument("--hbm-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "run with --copy-calibration-mib into the per-kernel HBM bytes table and exit")
    ap.add_argument("--no-layer-prefetch", action="store_true",
                    help="config 3: the same as --decode-schedule plain")
    ap.add_argument("--decode-schedule", choices=["ahead", "prefetch", "plain"], default="ahead",
                    help="config 3: 'ahead' runs both layers' Steps 1-5 in one launch (engram_project_ahead) and "
                         "each layer's Steps 6-8 in one (engram_forward_projected); 'prefetch' carries the next "
                         "layer's retrieval in the conv launch (engram_forward_retrieved_prefetch); 'plain' is "
                         "engram_forward per layer")
    ap.add_argument("--no-controls", action="store_true",
                    help="configs 1-2: skip the control measurements (one batch replayed, a cold-cache pass that "
                         "overwrites 512 MiB between steps, and the gather over uniform tokens)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB device to device three times "
                         "(a plain copy kernel of known size for scaling HBM byte counters)")
    return ap.parse_args(argv)


def log(msg):
    """Progress to stderr (the JSON line alone goes to stdout)."""
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def rotation_size(rows_bytes_per_batch, per_graph, override=0, least=8):
    """Distinct batches in the timed rotation: enough that they touch
    ROTATION_BYTES of table rows (at least `least`), rounded up to whole
    graphs of per_graph steps."""
    if override > 0:
        n = override
    else:
        n = max(least, math.ceil(ROTATION_BYTES / max(rows_bytes_per_batch, 1)))
    return per_graph * math.ceil(n / per_graph)



def kernel_units(n_tok, lay, hdtype, hot_hit=None, mx=False):
    """Algorithmic bytes (HBM-bound kernels) or flops (matrix-core kernels)
    per launch of each kernel of one layer forward over n_tok tokens, keyed by
    the kernel names the library reports.  hot_hit: the fraction of hot
    n-grams per order when the Engram-Nine tier is attached (a hit reads one
    pilot, one 32-byte slot and its K*dim row; a miss reads its K cold rows
    after the same pilot and slot).  mx: the layer runs the MXFP8 product, so
    the gather writes one E4M3 code per element plus a scale byte per 32."""
    nt = lay.hash.n_tables
    dim = lay.tables.dim
    d, M = lay.d, lay.branches
    es = 2 if hdtype == "bf16" else 4
    i8 = lay.tables.dtype == "i8"
    row_bytes = dim * (1 if i8 else es) + (4 if i8 else 0)
    e_bytes = dim + dim // 32 if mx else dim * es     # gathered bytes per row
    d_mem = nt * dim
    fused = hdtype == "bf16" and d % 128 == 0
    n_stat = (1 + M) * d // 128 if fused else 1 + M
    N = (1 + M) * d
    flops = 2.0 * n_tok * N * d_mem
    # Below the matrix cores' ridge (the library's small-batch projection, used
    # up to 7 * 2^18 token-features) the projection is bound by reading W:
    # W, e and h in, v and statistics out.
    # (the FP8 product takes it up to 3 * 2^19 and only when K is a multiple of
    # 512; its W and e are one byte per value plus a scale byte per 32)
    small = fused and n_tok * N <= (3 << 19 if mx else 7 << 18) and (not mx or d_mem % 512 == 0)
    op = 1 + 1 / 32 if mx else es
    proj = ("hbm", N * d_mem * op + n_tok * (d_mem * op + M * d * es + d * 4 + 16 * N // 64)) if small \
        else ("mfma", flops)
    units = {
        # token ids in; rows in; e out
        "gather_kernel<hashed>": ("hbm", n_tok * (4 + nt * (row_bytes + e_bytes))),
        "proj_gate_kernel": proj,
        "gemm_kernel": ("mfma", flops),
        # h, k, v in; statistics out
        "gate_stats_kernel": ("hbm", n_tok * (M * 2 * d * 4 + d * 4 + M * d * es + 16 * n_stat)),
        # v (float32) and statistics in; H in and out; alpha, gamma out
        "conv_kernel": ("hbm", n_tok * (d * 4 + 16 * n_stat + M * (2 * d * es + 8))),
        # v and gamma in; conv input of the newest position out; ids, pos
        "state_commit_kernel": ("hbm", n_tok * (d * 4 + M * (d * 4 + 4) + 16)),
        # two identical layers per launch (engram_project_ahead): both layers'
        # gathers; both layers' small-batch products (W and e in, the float32
        # product out)
        "gather2_kernel": ("hbm", 2 * n_tok * (4 + nt * (row_bytes + e_bytes))),
        "proj_kv_kernel": ("hbm", 2 * (N * d_mem * op + n_tok * (d_mem * op + N * 4))),
        # both layers' Steps 1-5 in one launch: token ids and rows in, W in,
        # the float32 product out (the gathered rows stay on chip)
        "gather_proj_kernel": ("hbm", 2 * (N * d_mem * op + n_tok * (4 + nt * row_bytes + N * 4))),
    }
    if hot_hit is not None:
        K = lay.hash.heads
        per_tok = 4 + nt * e_bytes
        for h in hot_hit:
            per_tok += 36 + h * K * dim * es + (1 - h) * K * row_bytes
        units["gather_kernel<hashed,hot>"] = ("hbm", n_tok * per_tok)
    return units


class Case:
    """One workload on the device, ready to time.

    calls(i): the library calls (zero-argument callables, launched on the
    current stream) of step i, which runs batch i % ring of the rotation."""

    def __init__(self, w, lays, n_tok, n_layers, ring, calls):
        self.w, self.lays, self.n_tok, self.n_layers = w, lays, n_tok, n_layers
        self.ring, self.calls = ring, calls
        self.extra = {}      # reported keys
        self.pipe = None     # (layers, tokens, H) of batch 0, for the overlap and LFU reports
        self.hot = None      # (hot tier, keys, rows, hit rate per order)
        self.keep = []       # device objects kept alive with the case


def hot_tier_host(n_hot, inputs, w, lay):
    """Engram-Nine hot tier on the host: per order the n_hot most frequent
    n-grams of a seeded warm-up stream (projected with the layer's P, as
    part of building the workload) and their N(0, 0.02) rows."""
    hp, tab = lay.hash, lay.tables
    warm = inputs.hot_warmup_tokens(w.config, 0)
    xc = hp.proj[warm]
    t0 = time.perf_counter()
    keys, rows = {}, {}
    for n in range(2, hp.max_n + 1):
        keys[n] = inputs.frequent_ngrams(xc, n, n_hot)
        rows[n] = inputs.hot_rows(w.config, 0, n, keys[n].shape[0], hp.heads * tab.dim, tab.dtype)
    return keys, rows, {"warm_tokens": int(warm.size), "host_select_s": round(time.perf_counter() - t0, 2)}


def hot_tier_device(eg, L, tok, tab_dtype, keys, rows, info):
    dev_rows = {n: eg.to_device(r, tab_dtype, "cuda") for n, r in rows.items()}
    t0 = time.perf_counter()
    hot = eg.HotTier(keys, dev_rows, device="cuda")
    t_build = time.perf_counter() - t0
    L.set_hot(hot)
    hit = (eg.hot_lookup(tok, L, hot) >= 0).float().mean(dim=(0, 1)).cpu().numpy()
    info = dict(info)
    info.update({"n_hot_per_order": {str(n): int(k.shape[0]) for n, k in keys.items()},
                 "hit_rate_per_order": {str(n): round(float(hit[n - 2]), 4) for n in keys},
                 "hot_rows_MiB": round(sum(r.nbytes for r in rows.values()) / 2 ** 20, 1),
                 "host_mphf_build_s": round(t_build, 2)})
    return (hot, keys, rows, [float(h) for h in hit]), info


def rows_per_batch(lays, n_tok):
    """Bytes of table rows one batch reads (every layer)."""
    out = 0
    for lay in lays:
        tab = lay.tables
        row = tab.dim * {"f32": 4, "bf16": 2, "i8": 1}[tab.dtype] + (4 if tab.dtype == "i8" else 0)
        out += n_tok * lay.hash.n_tables * row
    return out


def build_case(args, cfg, torch, eg, inputs, w=None, per_graph=10, hot_host=None, mxfp8=False):
    """Workload cfg on the device with its rotation of batches."""
    dev = "cuda"
    if cfg in (1, 2):
        w = w if w is not None else inputs.make_config(cfg)
        lay = w.layers[0]
        L = eg.Layer(lay, w.dtype, dev, mxfp8=mxfp8)
        n_tok = w.B * w.T
        ring = rotation_size(rows_per_batch([lay], n_tok), per_graph, args.ring, least=8)
        h_bytes = w.H.nbytes
        ring_h = min(ring, max(2, math.ceil(ROTATION_BYTES / h_bytes))) if ring > 1 else 1
        log(f"{w.name}: {ring} token batches, {ring_h} hidden-state batches in the rotation")
        toks = [torch.from_numpy(w.tokens).to(dev)] + \
            [torch.from_numpy(inputs.token_batch(cfg, i, (w.B, w.T))).to(dev) for i in range(1, ring)]
        Hs = [eg.to_device(w.H, w.dtype, dev)] + \
            [eg.to_device(inputs.hidden_batch(cfg, i, w.H.shape, w.dtype), w.dtype, dev) for i in range(1, ring_h)]
        ws = torch.empty(eg.forward_workspace(w.B, w.T, L), dtype=torch.uint8, device=dev)
        case = Case(w, [lay], n_tok, 1, ring,
                    lambda i: [lambda: eg.forward(toks[i % ring], Hs[i % ring_h], L, ws=ws)])
        case.extra["rotation"] = {"token_batches": ring, "hidden_batches": ring_h,
                                  "table_row_bytes_per_batch": rows_per_batch([lay], n_tok)}
        case.pipe = ([L], toks[0], Hs[0])
        case.keep = [L, toks, Hs, ws]
        if hot_host is not None:
            keys, rows, info = hot_host
            case.hot, case.extra["hot_tier"] = hot_tier_device(eg, L, toks[0], lay.tables.dtype, keys, rows, info)
        return case
    if cfg == 3:
        w = w if w is not None else inputs.make_config(3)
        S = w.B
        Ls = [eg.Layer(l, "bf16", dev, mxfp8=mxfp8) for l in w.layers]
        states = [eg.DecodeState(S, 3, 1, 9, 1024, dev) for _ in Ls]
        ctx = torch.from_numpy(w.context).to(dev)
        Hc = eg.to_device(w.H_context, "bf16", dev)
        for L, st in zip(Ls, states):               # prefill the context (not timed)
            eg.forward(ctx, Hc, L, state=st)
        ring = rotation_size(rows_per_batch(w.layers, S), per_graph, args.ring, least=64)
        log(f"{w.name}: {ring} decode batches in the rotation")
        toks = [torch.from_numpy(w.tokens).to(dev)] + \
            [torch.from_numpy(inputs.token_batch(3, i, (S, 1))).to(dev) for i in range(1, ring)]
        Hs = [eg.to_device(w.H, "bf16", dev)] + \
            [eg.to_device(inputs.hidden_batch(3, i, w.H.shape), "bf16", dev) for i in range(1, ring)]
        wss = [torch.empty(eg.forward_workspace(S, 1, L), dtype=torch.uint8, device=dev) for L in Ls]
        es = [eg.rows_buffer(S, 1, L, dev) for L in Ls]
        schedule = "plain" if args.no_layer_prefetch else args.decode_schedule
        kvs = [eg.kv_buffer(S, 1, L, dev) for L in Ls]
        ws_ahead = torch.empty(max(eg.project_ahead_workspace(S, 1, Ls), 256), dtype=torch.uint8, device=dev)

        def calls(i):
            tok, H = toks[i % ring], Hs[i % ring]
            if schedule == "ahead":
                # both layers' Steps 1-5 as soon as the token is known, then
                # each layer's Steps 6-8 on its hidden state
                return [lambda: eg.project_ahead(tok, Ls, kv=kvs, states=states, ws=ws_ahead)] + \
                    [(lambda j=j: eg.forward_projected(kvs[j], H, Ls[j], S, 1, state=states[j], ws=wss[j]))
                     for j in range(len(Ls))]
            if schedule == "plain":
                return [(lambda L=L, st=st, ws=ws: eg.forward(tok, H, L, state=st, ws=ws))
                        for L, st, ws in zip(Ls, states, wss)]

            # every layer but the last carries the next layer's retrieval (same
            # tokens, that layer's id history) in its conv launch
            def layer(j):
                if j + 1 < len(Ls):
                    eg.forward_retrieved_prefetch(tok, es[j], H, Ls[j], tok, es[j + 1], ws=wss[j],
                                                  next_layer=Ls[j + 1], state=states[j], next_state=states[j + 1])
                else:
                    eg.forward_retrieved(tok, es[j], H, Ls[j], state=states[j], ws=wss[j])
            return [lambda: eg.retrieve(tok, Ls[0], es[0], state=states[0])] + \
                [(lambda j=j: layer(j)) for j in range(len(Ls))]
        case = Case(w, w.layers, S, len(Ls), ring, calls)
        case.extra["decode"] = "256 sequences x 1 token, 2 layers, after a 16-token prefill" + {
            "plain": "; engram_forward per layer",
            "prefetch": "; layer 1's retrieval runs inside layer 0's conv launch",
            "ahead": "; both layers' Steps 1-5 in one launch ahead of the hidden states, then one gate+conv "
                     "launch per layer"}[schedule]
        case.extra["rotation"] = {"token_batches": ring, "hidden_batches": ring,
                                  "table_row_bytes_per_batch": rows_per_batch(w.layers, S)}
        case.keep = [Ls, states, toks, Hs, wss, es, kvs, ws_ahead]
        return case
    # cfg == 4: host tables + HBM cache
    w = w if w is not None else inputs.make_config(4)
    n_tok = w.B * w.T
    ring = rotation_size(rows_per_batch(w.layers, n_tok), per_graph, args.ring, least=8)
    ring_h = min(ring, max(2, math.ceil(ROTATION_BYTES / w.H.nbytes))) if ring > 1 else 1
    log(f"{w.name}: {ring} token batches, {ring_h} hidden-state batches in the rotation")
    toks = [torch.from_numpy(w.tokens).to(dev)] + \
        [torch.from_numpy(inputs.token_batch(4, i, (w.B, w.T))).to(dev) for i in range(1, ring)]
    Hs = [eg.to_device(w.H, "bf16", dev)] + \
        [eg.to_device(inputs.hidden_batch(4, i, w.H.shape), "bf16", dev) for i in range(1, ring_h)]
    Ls, bufs, hits = [], [], []
    for li, lay in enumerate(w.layers):
        hb = eg.HostBuffer(lay.tables.rows.nbytes)
        hb.numpy(lay.tables.rows.dtype, lay.tables.rows.shape)[:] = lay.tables.rows
        bufs.append(hb)
        L = eg.Layer(lay, "bf16", dev, rows_ptr=hb.dev)
        warm = torch.from_numpy(inputs.lfu_warmup_tokens(4, li).reshape(16, -1)).to(dev)
        slot, rows, _ = eg.cache_build(warm, L, lay.tables.total_rows // 10)
        L.set_cache(slot, rows)
        z = eg.hash_indices(toks[0], L).long() + torch.from_numpy(lay.tables.row_offset).to(dev)
        hits.append(round(float((slot[z] >= 0).float().mean().item()), 4))
        Ls.append(L)
    ws = torch.empty(max(eg.forward_workspace(w.B, w.T, L) for L in Ls), dtype=torch.uint8, device=dev)
    case = Case(w, w.layers, n_tok, len(Ls), ring,
                lambda i: [(lambda L=L: eg.forward(toks[i % ring], Hs[i % ring_h], L, ws=ws)) for L in Ls])
    case.extra["cache_hit_rate"] = hits
    case.extra["rotation"] = {"token_batches": ring, "hidden_batches": ring_h,
                              "table_row_bytes_per_batch": rows_per_batch(w.layers, n_tok)}
    case.pipe = (Ls, toks[0], Hs[0])
    case.keep = [Ls, bufs, toks, Hs, ws]
    return case



# ---- HBM traffic from rocprofv3 counters ----
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# library stage name -> (pattern of the rocprofv3 kernel name, sources whose text fixes the kernel)
KERNEL_SOURCES = {
    "gather_kernel<hashed>": (r"hashed_gather_kernel<[^>]*false, \d>",
                              ["gather.hip", "gather_device.h", "hash_device.h", "hot_device.h"]),
    "gather_kernel<hashed,hot>": (r"hashed_gather_kernel<[^>]*true, \d>",
                                  ["gather.hip", "gather_device.h", "hash_device.h", "hot_device.h"]),
    "proj_gate_kernel": (r"proj_gate(_small|_mx_resident)?_kernel<", ["proj_gate.hip"]),
    "gather2_kernel": (r"hashed_gather2_kernel<", ["gather.hip", "gather_device.h", "hash_device.h", "hot_device.h"]),
    "proj_kv_kernel": (r"proj_(gate_small2|frag2)_kernel<", ["proj_gate.hip", "ahead.hip"]),
    "gather_proj_kernel": (r"ahead_fused_kernel<", ["ahead.hip", "gather_device.h", "hash_device.h", "hot_device.h"]),
    "conv_kernel": (r"conv_(strip_|decode_)?kernel<", ["gate_conv.hip"]),
    "conv_gather_kernel": (r"conv_gather_kernel<",
                           ["gate_conv.hip", "gather_device.h", "hash_device.h", "hot_device.h"]),
}
COMMON_SOURCES = ["device_util.h", "engram_internal.h"]


def kernel_source_hash(stage):
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES[stage][1] + COMMON_SOURCES:
        with open(os.path.join(ROOT, "hashed_gram_embedding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def read_traffic_table():
    """{(workload, stage): (fetch_bytes, write_bytes, source_hash)} from the committed table."""
    out = {}
    if not os.path.exists(TRAFFIC_TABLE):
        return out
    import re
    for line in open(TRAFFIC_TABLE):
        m = re.match(r"\|\s*([\w-]+)\s*\|\s*`([^`]+)`\s*\|\s*(\d+)\s*\|\s*(\d+)\s*\|\s*\d+\s*\|\s*([0-9a-f]+)\s*\|", line)
        if m:
            out[(m.group(1), m.group(2))] = (int(m.group(3)), int(m.group(4)), m.group(5))
    return out


def traffic_for(workload, stage):
    """Measured HBM bytes per launch, or None when the table has no row for
    the kernel or its sources changed since the counters were taken."""
    row = read_traffic_table().get((workload, stage))
    if row is None or stage not in KERNEL_SOURCES or row[2] != kernel_source_hash(stage):
        return None
    return row[0] + row[1]


def hbm_summary(fetch_csv, write_csv, workload, n_true):
    """Per-launch HBM bytes of each library kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) averaged over the run's dispatches, each scaled by the
    ratio of the true bytes of the calibration copy to what the same counter
    read for it.  Prints the table rows for this workload."""
    import csv
    import re

    def per_kernel(path):
        acc = {}
        for r in csv.DictReader(open(path)):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)

    # the calibration copy: the largest copyBuffer dispatch reads and writes n_true bytes
    def copy_bytes(d):
        vals = [max(v) for k, v in d.items() if "copyBuffer" in k]
        return max(vals) if vals else None
    cf, cw = copy_bytes(fetch), copy_bytes(write)
    if cf is None or cw is None:
        raise SystemExit("no calibration copy in the counter files (run with --copy-calibration-mib)")
    f_scale, w_scale = n_true / cf, n_true / cw
    rows = []
    for stage, (pat, _) in KERNEL_SOURCES.items():
        # of the kernel's instantiations in the run, the one dispatched most
        # often (the timed workload's, not e.g. a decode prefill's)
        names = [k for k in fetch if re.search(pat, k) and k in write]
        if not names:
            continue
        k = max(names, key=lambda n: len(fetch[n]))
        fb = sum(fetch[k]) / len(fetch[k]) * f_scale
        wb = sum(write[k]) / len(write[k]) * w_scale
        rows.append((stage, int(round(fb)), int(round(wb)), len(fetch[k])))
    print(f"calibration: copy of {n_true / 2**20:.0f} MiB; FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}")
    for stage, fb, wb, n in rows:
        print(f"| {workload} | `{stage}` | {fb} | {wb} | {n} | {kernel_source_hash(stage)} |")



def overlap_report(torch, eg, w, lay, steps, warmup):
    """Retrieval run ahead of the layer (the pages' prefetch from token ids).

    1. Hidden behind the preceding layers: a stand-in for one dense transformer
       block at the same batch (bf16 matmuls of d = 1024 with a 4x MLP:
       x W_qkv, q W_o, x W_up, u W_down; torch / hipBLASLt) runs on the main
       stream while engram_retrieve runs on a second stream; hidden = (t_block
       + t_retrieve - t_both) / t_retrieve.
    2. Pipelined batches: engram_retrieve of batch s+1 on the second stream
       while engram_forward_retrieved of batch s runs on the main stream (two
       alternating synthetic batches, each step the whole layer for its
       batch), captured as a two-step HIP graph.
    Every variant is captured in a HIP graph and replayed, so the streams'
    fork and join are graph edges rather than host-side event waits."""
    dev = "cuda"
    B, T = w.B, w.T
    n_tok = B * T
    L = eg.Layer(lay, w.dtype, dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn(n_tok, 1024, device=dev, dtype=torch.bfloat16, generator=g)
    wq = torch.randn(1024, 3072, device=dev, dtype=torch.bfloat16, generator=g) / 32
    wo = torch.randn(1024, 1024, device=dev, dtype=torch.bfloat16, generator=g) / 32
    wu = torch.randn(1024, 4096, device=dev, dtype=torch.bfloat16, generator=g) / 32
    wd = torch.randn(4096, 1024, device=dev, dtype=torch.bfloat16, generator=g) / 64
    flops = 2.0 * n_tok * 1024 * (3072 + 1024 + 4096 + 4096)

    def block():
        q = torch.matmul(x, wq)
        torch.matmul(q[:, :1024].contiguous(), wo)
        torch.matmul(torch.matmul(x, wu), wd)

    tok = torch.from_numpy(w.tokens).to(dev)
    rng = __import__("numpy").random.default_rng(11)
    tok2 = torch.from_numpy(inputs_zipf_like(w.tokens, rng)).to(dev)
    e = [eg.rows_buffer(B, T, L, dev) for _ in range(2)]
    H = eg.to_device(w.H, w.dtype, dev)
    ws = torch.empty(eg.forward_retrieved_workspace(B, T, L), dtype=torch.uint8, device=dev)

    def graph_of(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def timed(gr, reps):
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(main)
        for _ in range(reps):
            gr.replay()
        t1.record(main)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e3          # us

    # every function launches on the stream current at call time (the capture
    # stream inside a graph capture) plus the side stream forked from it
    def retr():
        eg.retrieve(tok, L, e[0])

    def both():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            eg.retrieve(tok, L, e[0], stream=side)
        block()
        cur.wait_stream(side)

    reps = max(steps, 20)
    t_block = timed(graph_of(block), reps)
    t_retr = timed(graph_of(retr), reps)
    t_both = timed(graph_of(both), reps)
    hidden = (t_block + t_retr - t_both) / t_retr

    # pipelined: a two-step cycle captured once
    def cycle():
        cur = torch.cuda.current_stream()
        for tc, tn, ec, en in ((tok, tok2, 0, 1), (tok2, tok, 1, 0)):
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                eg.retrieve(tn, L, e[en], stream=side)
            eg.forward_retrieved(tc, e[ec], H, L, ws=ws, stream=cur)
            cur.wait_stream(side)

    eg.retrieve(tok, L, e[0])
    g_cycle = graph_of(cycle)
    eg.retrieve(tok, L, e[0])
    t_cycle = timed(g_cycle, max(steps // 2, 10))
    step_us = t_cycle / 2

    # the same two batches without overlap, for comparison
    def seq():
        for tc in (tok, tok2):
            eg.retrieve(tc, L, e[0])
            eg.forward_retrieved(tc, e[0], H, L, ws=ws)
    t_seq = timed(graph_of(seq), max(steps // 2, 10)) / 2
    return {
        "standin_block": {"what": "one dense transformer block's matmuls, d=1024, 4x MLP, bf16 (torch)",
                          "us": round(t_block, 2), "TFLOP/s": round(flops / (t_block * 1e-6) / 1e12, 1)},
        "retrieve_us": round(t_retr, 2),
        "block_plus_retrieve_concurrent_us": round(t_both, 2),
        "retrieve_hidden_fraction": round(hidden, 3),
        "sequential_two_batch_ms_per_step": round(t_seq / 1e3, 5),
        "pipelined": {"ms_per_step": round(step_us / 1e3, 5), "tokens_per_s": round(n_tok / (step_us * 1e-6), 1),
                      "how": "retrieve(batch s+1) on a second stream during forward_retrieved(batch s); "
                             "two alternating batches; HIP graph of a two-step cycle"},
    }


def pipelined_report(torch, eg, w, pipe, steps):
    """Steps of all layers with the retrieval of step s+1 (every layer's
    Steps 1-4, token ids only) on a second stream while step s computes
    (Steps 5-8 of every layer) on the main stream; two alternating token
    batches, a two-step cycle captured as a HIP graph.  Compared with the
    same two batches run in order in one graph."""
    import numpy as np
    Ls, tok, H = pipe
    B, T = tok.shape
    dev = "cuda"
    side = torch.cuda.Stream()
    tok2 = torch.from_numpy(inputs_zipf_like(tok.cpu().numpy(), np.random.default_rng(11))).to(dev)
    toks = (tok, tok2)
    e = [[eg.rows_buffer(B, T, L, dev) for L in Ls] for _ in range(2)]
    ws = torch.empty(max(eg.forward_retrieved_workspace(B, T, L) for L in Ls), dtype=torch.uint8, device=dev)

    def retrieve_all(par, stream=None):
        for li, L in enumerate(Ls):
            eg.retrieve(toks[par], L, e[par][li], stream=stream)

    def compute_all(par, stream=None):
        for li, L in enumerate(Ls):
            eg.forward_retrieved(toks[par], e[par][li], H, L, ws=ws, stream=stream)

    def cycle():
        cur = torch.cuda.current_stream()
        for par in (0, 1):
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                retrieve_all(1 - par, stream=side)
            compute_all(par, stream=cur)
            cur.wait_stream(side)

    def seq():
        for par in (0, 1):
            retrieve_all(par)
            compute_all(par)

    def compute_only():
        for par in (0, 1):
            compute_all(par)

    def fused():
        # each layer's compute carries the next retrieval in its conv launch
        # (engram_forward_retrieved_prefetch): the next layer's rows of the same
        # batch, and after the last layer the first layer's rows of the next batch
        for par in (0, 1):
            for li, L in enumerate(Ls):
                if li + 1 < len(Ls):
                    nl, nt, ne = Ls[li + 1], toks[par], e[par][li + 1]
                else:
                    nl, nt, ne = Ls[0], toks[1 - par], e[1 - par][0]
                eg.forward_retrieved_prefetch(toks[par], e[par][li], H, L, nt, ne, ws=ws, next_layer=nl)

    def timed_graph(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        retrieve_all(0)
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            gr.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps / 2 * 1e3       # us per step

    def timed_eager(fn, reps):
        retrieve_all(0)
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps / 2 * 1e3

    retrieve_all(0)
    reps = max(steps // 2, 5)
    t_pipe = timed_graph(cycle, reps)
    t_seq = timed_graph(seq, reps)
    t_pipe_eager = timed_eager(cycle, reps)
    t_seq_eager = timed_eager(seq, reps)
    t_fused = timed_graph(fused, reps)
    t_compute = timed_graph(compute_only, reps)
    t_retr = t_seq - t_compute
    return {"layers_per_step": len(Ls), "sequential_us_per_step": round(t_seq, 2),
            "pipelined_us_per_step": round(t_pipe, 2),
            "pipelined_tokens_per_s": round(B * T / (t_pipe * 1e-6), 1),
            "eager_sequential_us_per_step": round(t_seq_eager, 2), "eager_pipelined_us_per_step": round(t_pipe_eager, 2),
            "fused_us_per_step": round(t_fused, 2), "fused_tokens_per_s": round(B * T / (t_fused * 1e-6), 1),
            "compute_only_us_per_step": round(t_compute, 2),
            "fused_retrieval_hidden_fraction": round((t_seq - t_fused) / t_retr, 3) if t_retr > 0 else None,
            "how": "retrieval of step s+1 (all layers) on a second stream during the compute of step s; "
                   "two alternating token batches; HIP graphs of two-step cycles.  fused: the same two "
                   "batches, one stream, each layer call carrying the next retrieval (the next layer's rows, "
                   "or after the last layer the next batch's) inside its conv launch "
                   "(engram_forward_retrieved_prefetch); hidden fraction = (sequential - fused) "
                   "/ (sequential - compute only)"}


def realtime_lfu_report(torch, eg, inputs, w, pipe, rounds=4, steps_per_round=8):
    """The hot cache under a shifted token distribution (the Zipf ranks mapped
    to ids by a different seeded permutation than the warm-up stream's; fresh
    batches every round):
    static LFU cache vs. the real-time LFU update.  Each round runs
    steps_per_round steps of every layer with access counting on, then
    updates every layer's cache from its counts (aged by one bit at each
    update).  Reports
    per round the hit rate over the round's accesses, the step time and the
    update time."""
    import numpy as np
    Ls, tok, H = pipe
    B, T = tok.shape
    dev = "cuda"
    rng = np.random.default_rng(21)
    perm = rng.permutation(128_000).astype(np.int32)
    def new_batches():
        # every round draws fresh batches from the same shifted distribution
        return [torch.from_numpy(np.ascontiguousarray(
            perm[inputs.zipf_tokens(rng, 128_000, 1.1, (B, T))])).to(dev) for _ in range(steps_per_round)]
    ws = torch.empty(max(eg.forward_workspace(B, T, L) for L in Ls), dtype=torch.uint8, device=dev)
    counts = [torch.zeros(L.s.tables.total_rows, dtype=torch.int32, device=dev) for L in Ls]
    for L, c in zip(Ls, counts):
        L.set_access_counts(c)

    def hit_rate(before):
        hits = acc = 0
        for L, c, c0 in zip(Ls, counts, before):
            delta = (c.to(torch.int64) - c0.to(torch.int64))
            acc += int(delta.sum().item())
            hits += int(delta[L.cache_slot >= 0].sum().item())
        return hits / max(acc, 1)

    out = []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for r in range(rounds + 1):
        batches = new_batches()
        before = [c.clone() for c in counts]
        torch.cuda.synchronize()
        ev[0].record()
        for b in batches:
            for L in Ls:
                eg.forward(b, H, L, ws=ws)
        ev[1].record()
        torch.cuda.synchronize()
        step_ms = ev[0].elapsed_time(ev[1]) / steps_per_round
        hr = hit_rate(before)
        del before
        upd_ms = None
        if r < rounds:
            ev[2].record()
            for L, c in zip(Ls, counts):
                eg.cache_update(L, c, decay_shift=1)
            ev[3].record()
            torch.cuda.synchronize()
            upd_ms = ev[2].elapsed_time(ev[3]) / len(Ls)
        out.append({"round": r, "hit_rate": round(hr, 4), "ms_per_step": round(step_ms, 4),
                    "update_ms_per_layer": None if upd_ms is None else round(upd_ms, 3)})
    for L in Ls:
        L.set_access_counts(None)
    return {"rounds": out, "steps_per_round": steps_per_round,
            "how": "round 0 uses the static cache from the warm-up stream; every later round follows an update "
                   "from the counts so far (aged by one bit at each update); eager steps; hit rate = cached "
                   "accesses / all accesses of the round"}


def inputs_zipf_like(tokens, rng):
    """A second token batch of the same shape and distribution: the first
    batch's ids permuted within each sequence."""
    import numpy as np
    out = np.array(tokens, copy=True)
    for b in range(out.shape[0]):
        out[b] = out[b][rng.permutation(out.shape[1])]
    return np.ascontiguousarray(out)


def measured_peaks(torch, shape=None):
    """The box's practical peaks, re-measured in the same run: a 1 GiB
    device-to-device copy (bytes read + written per second) and a large bf16
    matmul through torch (hipBLASLt), 8192 x 8192 x 8192, with its operands in
    the layer's layout (both K-contiguous: C = A B^T) and, for reference, in
    the plain layout (C = A B).  shape = (tokens, N, K) adds the library's
    matmul at the layer's own product shape, timed as a replayed graph of 20
    back-to-back calls."""
    main = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(main)
        for _ in range(reps):
            fn()
        t1.record(main)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e-3          # s

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    bt = b.t()
    t_nt = timed(lambda: torch.matmul(a, bt), 10)
    t_nn = timed(lambda: torch.matmul(a, b), 10)
    del a, b, bt
    out = {"hbm_copy_GBps": round(2 * n / t_copy / 1e9, 1),
           "bf16_gemm_TFLOPs": round(2.0 * m ** 3 / t_nt / 1e12, 1),
           "bf16_gemm_plain_layout_TFLOPs": round(2.0 * m ** 3 / t_nn / 1e12, 1),
           "how": "1 GiB device-to-device copy (read + write bytes); 8192^3 bf16 torch.matmul (hipBLASLt), "
                  "A B^T with both operands K-contiguous as in the layer, and A B"}
    if shape is not None:
        M, N, K = shape
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        bt = torch.randn(N, K, device="cuda", dtype=torch.bfloat16).t()
        for _ in range(3):
            torch.matmul(a, bt)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                torch.matmul(a, bt)
        t = timed(g.replay, 3) / 20
        out["library_gemm_at_layer_shape"] = {"M": M, "N": N, "K": K, "us": round(t * 1e6, 2),
                                              "TFLOPs": round(2.0 * M * N * K / t / 1e12, 1)}
        del a, bt, g
    return out



_SPIN = {}


def queue_ahead(torch, ms):
    """Puts a spin kernel of about `ms` milliseconds on the current stream,
    so that the host has queued the launches that follow before the GPU
    reaches them: they then run back to back, as in a graph replay, instead
    of waiting on host launch overhead."""
    if "cycles_per_ms" not in _SPIN:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1 << 22)
        b.record()
        b.synchronize()
        _SPIN["cycles_per_ms"] = (1 << 22) / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SPIN["cycles_per_ms"]))


def time_case(torch, eg, case, steps, warmup, eager=False, per_graph=10):
    """Times `steps` steps of the case (HIP graphs of per_graph consecutive
    steps, one graph per stretch of the rotation, replayed in rotation
    order), then each kernel's duration from events its own dispatch records
    (eager launches over the same rotation), and the eager step with host
    launches.  Returns a dict of measurements."""
    stream = torch.cuda.current_stream()
    R = case.ring

    def step(i):
        for c in case.calls(i):
            c()                                 # on the current stream

    for i in range(max(warmup, min(R, 200))):
        step(i)
    torch.cuda.synchronize()
    n_graphs = R // math.gcd(R, per_graph)      # graph g runs steps g*per_graph .. (g+1)*per_graph - 1
    graphs = []
    if not eager:
        for g in range(n_graphs):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):          # captures on a side stream
                for s in range(per_graph):
                    step(g * per_graph + s)
            graphs.append(gr)
        torch.cuda.synchronize()
    pos = [0]

    def run():                                  # the next per_graph steps of the rotation
        if eager:
            for s in range(per_graph):
                step(pos[0] * per_graph + s)
        else:
            graphs[pos[0] % n_graphs].replay()
        pos[0] += 1

    # warm-up: whole cycles of the rotation, at least `warmup` steps and
    # WARMUP_FLOOR_MS of back-to-back work (the first ~100 ms on a fresh GPU
    # run up to 7 % slower while clocks and caches settle)
    warm_steps = 0
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_ms = 0.0
    while warm_steps < warmup or warm_ms < WARMUP_FLOOR_MS or pos[0] % n_graphs != 0:
        w0.record(stream)
        run()
        w1.record(stream)
        w1.synchronize()
        warm_ms += w0.elapsed_time(w1)
        warm_steps += per_graph
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps // per_graph):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del graphs

    # eager steps with host launches (no profiling), the same rotation
    n_eager = max(min(R, 200), 20)
    t0.record(stream)
    for i in range(n_eager):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / n_eager

    # per-kernel durations: events recorded by each kernel's own dispatch
    # (the library's stage timing), eager steps over the same rotation run
    # back to back and read every `chunk` steps; the first step of a chunk
    # starts on an idle GPU and is left out
    eg.profile_enable(2)
    step(0)
    per_call = len(eg.profile_read())           # stages of one step
    chunk = max(2, min(PROFILE_CHUNK_STEPS, eg.PROFILE_MAX_STAGES // max(per_call, 1)))
    samples = {}
    n_timed = 0
    i = 0
    # a spin ahead only where the host could fall behind: steps longer than
    # QUEUE_AHEAD_MAX_STEP_MS keep the queue full by themselves, and an idle
    # spin before them would let the clocks drop for the steps that follow
    spin = ms < QUEUE_AHEAD_MAX_STEP_MS
    while n_timed < n_eager:
        if spin:
            queue_ahead(torch, QUEUE_AHEAD_MS)
        for s in range(chunk):
            step(i + s)
        for name, t in eg.profile_read()[per_call:]:
            samples.setdefault(name, []).append(t)
        n_timed += chunk - 1
        i += chunk
    eg.profile_enable(False)
    n_eager_timed = n_timed
    per_step = {k: len(v) / n_eager_timed for k, v in samples.items()}   # launches of each kernel per step
    kernel_ms = {k: sum(v) / len(v) for k, v in samples.items()}

    def pcts(v):
        q = np.percentile(np.asarray(v) * 1000.0, [10, 50, 90])
        return [round(float(x), 2) for x in q]
    return {"ms_per_step": ms, "warmup_steps_run": warm_steps, "graphs": 0 if eager else n_graphs,
            "eager_ms_per_step": eager_ms, "kernel_ms": kernel_ms,
            "kernel_launches_per_step": per_step,
            "kernel_us_p10_p50_p90": {k: pcts(v) for k, v in samples.items()}}


def rates_and_roofline(t, case, mxfp8=False, workload=None):
    """Kernel rates (algorithmic units per second) and the roofline of the
    longest kernel."""
    lay = case.lays[0]
    n_per_layer = case.n_tok
    units = kernel_units(n_per_layer, lay, case.w.dtype, case.hot[3] if case.hot else None, mx=mxfp8)
    rates = {}
    for k, ms in t["kernel_ms"].items():
        if k in units:
            kind, amount = units[k]
            rates[k] = amount / (ms * 1e-3) / (1e9 if kind == "hbm" else 1e12)
    dominant = max((k for k in t["kernel_ms"] if k in units), key=lambda k: t["kernel_ms"][k])
    kind, amount = units[dominant]
    wl = workload or case.w.name
    if kind == "mfma":
        peak = PEAK_FP8_TFLOPS if mxfp8 else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "kernel": dominant, "achieved": round(rates[dominant], 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(rates[dominant] / peak, 4),
                "traffic": traffic_for(wl, dominant), "units_per_launch": amount}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": round(rates[dominant], 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(rates[dominant] / PEAK_HBM_GBPS, 4),
                "traffic": traffic_for(wl, dominant), "units_per_launch": amount}
    return units, rates, roof


def kernel_block(t, rates, case):
    """The per-kernel part of a report: mean durations, percentiles, rates,
    and the sum of one step's kernel durations beside the graph step time."""
    ks = sum(t["kernel_ms"][k] * t["kernel_launches_per_step"][k] for k in t["kernel_ms"])
    return {"kernel_ms": {k: round(v, 5) for k, v in t["kernel_ms"].items()},
            "kernel_us_p10_p50_p90": t["kernel_us_p10_p50_p90"],
            "kernel_rate": {k: round(v, 2) for k, v in rates.items()},
            "kernel_timing": {"how": "events recorded by each kernel's own dispatch over eager steps of the same "
                                     f"rotation, run back to back (steps under {QUEUE_AHEAD_MAX_STEP_MS:g} ms queued behind a "
                                     f"{QUEUE_AHEAD_MS:g} ms spin kernel so that the host stays ahead), read every "
                                     f"{PROFILE_CHUNK_STEPS} steps (the first step after each read left out)",
                              "sum_of_kernels_ms_per_step": round(ks, 5),
                              "graph_step_minus_kernel_sum_ms": round(t["ms_per_step"] - ks, 5),
                              "eager_ms_per_step": round(t["eager_ms_per_step"], 5)}}


def config_block(w, case, args, mxfp8):
    lay = case.lays[0]
    return {"workload": w.name, "B": w.B, "T": w.T, "layers_per_step": case.n_layers, "branches": lay.branches,
            "d": lay.d, "d_mem": lay.d_mem, "tables": lay.hash.n_tables,
            "table_rows": int(lay.tables.n_rows.sum()), "table_dtype": lay.tables.dtype,
            "product": "mxfp8" if mxfp8 else w.dtype,
            "hot_ngrams_per_order": args.hot_tier if w.config in (1, 2) else 0}


_CPU_JOB = None   # (workload, hot tier) for the forked oracle workers


def _cpu_chunk(bounds):
    """The oracle's layer forward on tokens [lo, hi) of every sequence, with the
    CPU_HALO positions before lo that the outputs there depend on."""
    from oracle import engram_oracle as orc
    lo, hi = bounds
    w, hot = _CPU_JOB
    s = max(0, lo - CPU_HALO)
    orc.forward(w.tokens[:, s:hi], w.H[:, s:hi], w.layers[0], w.dtype, hot=hot)
    return w.B * (hi - lo)


def cpu_baseline(w, budget_s, hot=None):
    """The CPU oracle (float64 numpy) on the whole batch of the workload, on
    every core this process may use (at most 16): the batch's positions are
    split into chunks (each with the 11 positions before it that its outputs
    depend on) over one forked worker process per core, each with one BLAS
    thread; whole-batch passes repeat for about 2/3 of the budget.  Then the
    same oracle on one core (one process, one BLAS thread) over the whole
    batch for the rest.  Runs before the GPU is touched (the workers are
    forked)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    global _CPU_JOB
    try:
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores))
    T = w.T
    n_chunks = cores * 2
    step = max(CPU_HALO + 1, math.ceil(T / n_chunks))
    chunks = [(lo, min(T, lo + step)) for lo in range(0, T, step)]
    _CPU_JOB = (w, hot)
    n_tok = w.B * w.T
    with threadpool_limits(1):
        ctx = mp.get_context("fork")
        with ctx.Pool(cores) as pool:
            pool.map(_cpu_chunk, chunks[:cores])          # workers started and warm
            passes, t0 = 0, time.perf_counter()
            while True:
                done = sum(pool.map(_cpu_chunk, chunks, chunksize=1))
                assert done == n_tok
                passes += 1
                el = time.perf_counter() - t0
                if el >= budget_s * 2 / 3:
                    break
        one, t1 = 0, time.perf_counter()
        while True:
            _cpu_chunk((0, T))
            one += 1
            el1 = time.perf_counter() - t1
            if el1 >= budget_s / 3:
                break
    _CPU_JOB = None
    return {"value": round(passes * n_tok / el, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole batch ({w.B} x {w.T} tokens) per pass, {passes} passes in {el:.1f} s over "
                      f"{cores} forked worker processes (one BLAS thread each; {len(chunks)} chunks of <= {step} "
                      f"positions, each with the {CPU_HALO} positions before it)",
            "single_core": {"value": round(one * n_tok / el1, 1), "unit": "tokens/s", "cores": 1,
                            "sample": f"{one} whole-batch passes in {el1:.1f} s, one process, one BLAS thread"}}


def report_case(args, torch, eg, case, steps, warmup, eager, mxfp8, per_graph):
    t = time_case(torch, eg, case, steps, warmup, eager=eager, per_graph=per_graph)
    wl = case.w.name + ("-mxfp8" if mxfp8 else "")
    units, rates, roof = rates_and_roofline(t, case, mxfp8=mxfp8, workload=wl)
    out = {"value": round(case.n_tok / (t["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
           "ms_per_step": round(t["ms_per_step"], 5), "steps": steps, "warmup_steps_run": t["warmup_steps_run"],
           "timing": (f"HIP graph replay, {per_graph} steps per graph, {t['graphs']} graphs over the rotation"
                      if not eager else "eager launches")}
    out.update(kernel_block(t, rates, case))
    out["roofline"] = roof
    g = rates.get("gather_kernel<hashed>", rates.get("gather_kernel<hashed,hot>"))
    out["gather_GBps"] = None if g is None else round(g, 1)
    if case.n_layers > 1:
        out["tokens_per_s_per_layer"] = round(case.n_tok * case.n_layers / (t["ms_per_step"] * 1e-3), 1)
    return out, units


def secondary_report(args, torch, eg, inputs):
    """The other workloads, each timed like the headline one (20 steps over its
    rotation of batches, HIP graphs of 10 steps) with its kernels' rates and
    the roofline of its longest kernel."""
    out = {}
    for cfg in (2, 3, 4):
        log(f"secondary: building {inputs.CONFIG_NAMES[cfg]}")
        t0 = time.perf_counter()
        case = build_case(args, cfg, torch, eg, inputs)
        log(f"secondary: {inputs.CONFIG_NAMES[cfg]} ready in {time.perf_counter() - t0:.1f} s; timing")
        rep, _ = report_case(args, torch, eg, case, 20, 5, False, False, 10)
        rep["config"] = config_block(case.w, case, args, False)
        if cfg == 4:
            # rows missing from the HBM cache cross PCIe: the gather's bound
            hit = sum(case.extra["cache_hit_rate"]) / len(case.extra["cache_hit_rate"])
            lay = case.lays[0]
            miss_bytes = case.n_tok * lay.hash.n_tables * lay.tables.dim * 2 * (1 - hit)
            g_ms = rep["kernel_ms"]["gather_kernel<hashed>"]
            rep["roofline"] = {"bound": "pcie", "kernel": "gather_kernel<hashed>",
                               "achieved": round(miss_bytes / (g_ms * 1e-3) / 1e9, 1), "peak": PEAK_PCIE_GBPS,
                               "unit": "GB/s", "frac": round(miss_bytes / (g_ms * 1e-3) / 1e9 / PEAK_PCIE_GBPS, 4),
                               "traffic": None, "units_per_launch": round(miss_bytes),
                               "note": "bytes of the rows that miss the HBM cache (host rows read over PCIe) per "
                                       "launch, over the gather's duration"}
        for k, v in case.extra.items():
            rep[k] = v
        out[case.w.name] = rep
        log(f"secondary: {case.w.name} {rep['ms_per_step'] * 1e3:.1f} us per step, {rep['value'] / 1e6:.2f} M tokens/s")
        del case, rep
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse(argv)
    if args.hbm_summary:
        from hashed_gram_embedding_amd import inputs
        if args.copy_calibration_mib <= 0:
            raise SystemExit("--hbm-summary needs --copy-calibration-mib: the size of the calibration copy")
        hbm_summary(args.hbm_summary[0], args.hbm_summary[1],
                    inputs.CONFIG_NAMES[args.config] + ("-mxfp8" if args.mxfp8 else ""),
                    args.copy_calibration_mib << 20)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not part "
                                   "of this build (see the design notes on sharding)", "n_gpus": args.gpus}))
        sys.exit(2)
    from hashed_gram_embedding_amd import inputs

    per_graph = next(k for k in (10, 5, 2, 1) if args.steps % k == 0)
    log(f"building {inputs.CONFIG_NAMES[args.config]}")
    w = inputs.make_config(args.config)
    hot_host = None
    if args.hot_tier > 0 and args.config in (1, 2):
        hot_host = hot_tier_host(args.hot_tier, inputs, w, w.layers[0])
    cpu = None
    if not args.no_cpu_baseline and args.config in (1, 2):
        log("CPU oracle baseline")
        hot = None
        if hot_host is not None:
            keys, rows, _ = hot_host
            hot = {"keys": {n: [tuple(int(v) for v in r) for r in k] for n, k in keys.items()}, "rows": rows}
        cpu = cpu_baseline(w, args.cpu_budget_s, hot)

    import torch
    from hashed_gram_embedding_amd import engram as eg

    log("device setup")
    case = build_case(args, args.config, torch, eg, inputs, w=w, per_graph=per_graph, hot_host=hot_host,
                      mxfp8=args.mxfp8)
    log("timing")
    rep, units = report_case(args, torch, eg, case, args.steps, args.warmup, args.eager, args.mxfp8, per_graph)
    lay0 = case.lays[0]
    peaks = measured_peaks(torch, (case.n_tok, (1 + lay0.branches) * lay0.d, lay0.d_mem)
                           if args.config in (1, 2) else None)
    roof = rep["roofline"]
    # (no FP8 matmul is re-measured, so an MXFP8 product has no measured peak)
    ref = None if (roof["bound"] == "mfma" and args.mxfp8) else \
        (peaks["bf16_gemm_TFLOPs"] if roof["bound"] == "mfma" else peaks["hbm_copy_GBps"])
    roof["frac_of_measured_peak"] = None if ref is None else round(roof["achieved"] / ref, 4)

    out = {
        "metric": METRIC,
        "value": rep["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": rep["warmup_steps_run"],
        "ms_per_step": rep["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 projection, bf16 storage" if args.mxfp8 else w.dtype,
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) tables, N(0,1) hidden states); a rotation of "
                "distinct batches so that table rows come from HBM",
        "config": config_block(w, case, args, args.mxfp8),
        "timing": rep["timing"],
        "gather_GBps": rep["gather_GBps"],
    }
    for k in ("kernel_ms", "kernel_us_p10_p50_p90", "kernel_rate", "kernel_timing", "tokens_per_s_per_layer"):
        if k in rep:
            out[k] = rep[k]
    out["roofline"] = roof
    out["measured_peaks"] = peaks
    out["cpu_baseline"] = cpu
    for k, v in case.extra.items():
        out[k] = v
    if args.config in (1, 2) and not args.no_controls:
        log("controls")
        out["controls"] = control_report(torch, eg, inputs, w, lay0, case.pipe, units)
    if args.overlap and args.config in (1, 2):
        out["retrieval_overlap"] = overlap_report(torch, eg, w, lay0, args.steps, args.warmup)
    if args.realtime_lfu and args.config == 4:
        out["realtime_lfu"] = realtime_lfu_report(torch, eg, inputs, w, case.pipe)
    if args.overlap and case.pipe is not None:
        out["retrieval_pipelined"] = pipelined_report(torch, eg, w, case.pipe, args.steps)
    if args.config == 1 and not args.no_secondary and not args.mxfp8 and args.hot_tier == 0:
        del case
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["secondary"] = secondary_report(args, torch, eg, inputs)
    print(json.dumps(out), flush=True)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def control_report(torch, eg, inputs, w, lay, pipe, units, steps=20):
    """Three controls of the measured kernel rates.
    one batch: the rotation's first batch called back to back, so that its rows stay in
    the on-chip caches (what a benchmark that reuses one batch measures).
    cold: before every eager layer call a 512 MiB buffer is overwritten (more
    than the 256 MB Infinity Cache), so tables, W and e start outside the
    on-chip caches; per-kernel times from the dispatch events.
    uniform tokens: the gather alone over tokens drawn uniformly from the raw
    vocabulary instead of Zipf(1.1), i.e. with almost no row reuse."""
    Ls, tok, H = pipe
    L = Ls[0]
    ws = torch.empty(eg.forward_workspace(w.B, w.T, L), dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def back_to_back(call):
        """Stage durations of `steps` back-to-back calls after 3 untimed ones."""
        eg.profile_enable(2)
        for _ in range(3):
            call()
        eg.profile_read()
        queue_ahead(torch, QUEUE_AHEAD_MS)
        for _ in range(steps):
            call()
        got = {}
        for name, t in eg.profile_read():
            got.setdefault(name, []).append(t)
        eg.profile_enable(False)
        return got

    one = back_to_back(lambda: eg.forward(tok, H, L, ws=ws))
    eg.profile_enable(True)
    cold = {}
    for it in range(3 + steps):
        flush.fill_(it & 0xff)
        eg.forward(tok, H, L, ws=ws)
        for name, t in eg.profile_read():
            if it >= 3:
                cold.setdefault(name, []).append(t)
    del flush
    utok = torch.from_numpy(inputs.uniform_control_tokens(w.config, w.B, w.T, lay.hash.vocab)).to("cuda")
    e = eg.rows_buffer(w.B, w.T, L, "cuda")
    eg.profile_enable(False)
    uni = [t for v in back_to_back(lambda: eg.retrieve(utok, L, e)).values() for t in v]
    cold_ms = {k: sum(v) / len(v) for k, v in cold.items()}
    one_ms = {k: sum(v) / len(v) for k, v in one.items()}

    def rate(name, ms):
        kind, amount = units[name]
        return round(amount / (ms * 1e-3) / (1e9 if kind == "hbm" else 1e12), 1)
    g_name = next(k for k in cold_ms if k.startswith("gather"))
    uni_ms = sum(uni) / len(uni)
    return {"one_batch_kernel_us": {k: round(v * 1000, 2) for k, v in one_ms.items()},
            "one_batch_rate": {k: rate(k, v) for k, v in one_ms.items() if k in units},
            "cold_kernel_us": {k: round(v * 1000, 2) for k, v in cold_ms.items()},
            "cold_rate": {k: rate(k, v) for k, v in cold_ms.items() if k in units},
            "uniform_tokens_gather_us": round(uni_ms * 1000, 2),
            "uniform_tokens_gather_GBps": rate(g_name, uni_ms),
            "how": "one batch: the first batch of the rotation, 20 back-to-back calls (its rows stay in the "
                   "caches); cold: a 512 MiB buffer overwritten before each of 20 eager layer calls; uniform: "
                   "engram_retrieve over seeded uniform raw ids, 20 back-to-back calls; rates are algorithmic "
                   "units per second"}



if __name__ == "__main__":
    main()
