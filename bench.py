#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X ADAMAS path (one GPU).

Workload: batch 1, 32 heads (MHA), head_dim 128, 131072 cached tokens per
layer, 32 layers, bf16 K/V, token budget 256 (Llama-2-7B-shaped 128K decode).
A step runs the fused decode step of every layer in sequence: encode the
query heads, scan the 2-bit code cache, select the budget, attend over the
selected rows.  K/V and the code cache are resident in HBM before timing
(the code cache is built once, untimed, by adamas_encode_keys, like a
prefill).  Inputs are seeded synthetic draws (synth.py).

Prints ONE JSON line with:
  value        decode tokens/s (batch / step time), step timed as a replayed
               HIP graph of the 32 layer calls;
  roofline     algorithmic bytes of one decode-step launch (code cache +
               gathered K/V rows + q/out) / its average duration, from HIP
               events recorded on the launch stream around every launch of an
               eager pass over the same steps, against 8 TB/s;
  cpu_baseline the CPU oracle timed on a bounded sample of layers on the host
               cores, scaled to tokens/s.

--workload selects one of two further measurements (same JSON fields):
  llama3.2-3b-gqa-1m        one GQA layer (24 query / 8 KV heads) over 1,048,576
                            tokens, budget 1024; four layers' caches are cycled
                            so the code cache never sits in the last-level cache;
  batch16-mha-64k-append4k  16 sequences x 32 heads x 65536 rows, budget 512: the
                            ragged decode step that appends each sequence's new
                            token (adamas_decode_append_step) on one stream while
                            a 4096-token prefill chunk for one sequence is
                            encoded and copied on a second stream.  With
                            --paged the caches are a shuffled pool of
                            1024-token pages (adamas_decode_paged_step) and
                            the chunk fills four spare pool pages.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "llama2-mha-128k-32layers"
METRIC = "decode-step tokens/s + achieved HBM GB/s at 128K ctx, budget 256, 1 GPU"


def algorithmic_bytes(B, Hq, Hkv, d, n_ctx, budget, elem_bytes):
    """Bytes one layer's decode step must move: every cached code once,
    the selected K and V rows, the query in and the output out."""
    codes = B * Hkv * n_ctx * d // 4
    rows = B * Hq * min(budget, n_ctx) * d * 2 * elem_bytes
    qo = B * Hq * d * elem_bytes * 2
    return codes + rows + qo


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--budget", type=int, default=256)
    ap.add_argument("--layers", type=int, default=None, help="override the 32-layer stack")
    ap.add_argument("--n-ctx", type=int, default=None)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target oracle CPU time for the baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a conversion kernel of known traffic (HBM counter scaling)")
    ap.add_argument("--workload", default=HEADLINE,
                    choices=(HEADLINE, "llama3.2-3b-gqa-1m", "batch16-mha-64k-append4k"))
    ap.add_argument("--paged", action="store_true",
                    help="batch16 workload: caches in a shuffled pool of 1024-token pages")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="print a compact summary of rocprofv3 CSV output under DIR and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- profiles
KERNEL_SOURCES = ("compressed_key_sparse_amd/csrc/adamas.hip",
                  "compressed_key_sparse_amd/csrc/kernels.hpp",
                  "compressed_key_sparse_amd/csrc/device_common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_llama2-128k_hbm_traffic.json")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed PMC summary, or None if
    the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def summarize(dirpath: str):
    """Compact text summary of rocprofv3 --stats / --pmc CSV files."""
    import csv
    import glob
    from collections import defaultdict
    for f in sorted(glob.glob(os.path.join(dirpath, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# kernel stats ({os.path.basename(f)})")
        print("calls  avg_us    min_us    max_us    total_%  kernel")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Name"]
                if "adm::" not in name and "copy" not in name.lower():
                    continue
                print(f"{int(r['Calls']):5d} {float(r['AverageNs'])/1e3:8.2f} "
                      f"{float(r['MinNs'])/1e3:8.2f} {float(r['MaxNs'])/1e3:8.2f} "
                      f"{float(r['Percentage']):8.2f}  {name[:110]}")
    for f in sorted(glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"),
                              recursive=True)):
        acc = defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                if "adm::" not in name and "copy" not in name.lower():
                    continue
                acc[(name, r["Counter_Name"], r.get("Grid_Size", ""))].append(
                    float(r["Counter_Value"]))
        print(f"# counters ({os.path.basename(f)}): mean per dispatch")
        print("dispatches  counter      mean_value  grid  kernel")
        for (name, cn, grid), vals in sorted(acc.items()):
            print(f"{len(vals):10d}  {cn:11s} {sum(vals)/len(vals):12.1f}  {grid}  {name[:100]}")


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU by design: no collectives).", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: multi-rank launch is not supported (single-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compressed_key_sparse_amd as adamas
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adamas.load()
    if args.workload == "llama3.2-3b-gqa-1m":
        return bench_gqa(args, dev)
    if args.workload == "batch16-mha-64k-append4k":
        return bench_batch_append(args, dev)
    w = synth.LLAMA2_128K_32L
    if args.n_ctx:
        w = w.replace(n_ctx=args.n_ctx, cap=args.n_ctx)
    L = args.layers or w.layers
    B, Hq, Hkv, d, n, bud = w.batch, w.hq, w.hkv, w.head_dim, w.n_ctx, args.budget
    print(f"[bench] setup: {L} layers x {Hq} heads x {n} tokens x d{d} {w.dtype}, budget {bud}",
          file=sys.stderr, flush=True)
    t_setup = time.time()
    layers = []
    for l in range(L):
        lay = synth.make_layer(w, l, dev)
        codes = torch.empty((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=dev)
        adamas.encode_keys(lay["k"], codes)
        layers.append({"q": lay["q"], "k": lay["k"], "v": lay["v"], "codes": codes,
                       "out": torch.empty_like(lay["q"]), "needles": lay["needles"]})
    torch.cuda.synchronize()
    print(f"[bench] setup done in {time.time() - t_setup:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream(dev)
    ws = adamas.Workspace(dev)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, n, bud, d))

    def run_step():
        for lay in layers:
            adamas.decode_step(lay["q"], lay["k"], lay["v"], lay["codes"], n, bud, out=lay["out"],
                               ws=ws, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_step()
    torch.cuda.synchronize()

    # -- eager pass: HIP events around every launch, on the launch stream
    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(L)] for _ in range(K)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(K):
        for l, lay in enumerate(layers):
            ev[s][l][0].record(stream)
            adamas.decode_step(lay["q"], lay["k"], lay["v"], lay["codes"], n, bud, out=lay["out"],
                               ws=ws, stream=stream)
            ev[s][l][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / K
    launch_us = float(np.mean([a.elapsed_time(b) for row in ev for a, b in row]) * 1e3)

    # -- graph pass: the 32-layer step captured once and replayed K times
    graph_ms = None
    step_times = []
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                run_step()
            for _ in range(args.warmup):
                g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        g0.record(stream)
        with torch.cuda.stream(stream):
            gev[0].record(stream)
            for i in range(K):
                g.replay()
                gev[i + 1].record(stream)
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        step_times = [gev[i].elapsed_time(gev[i + 1]) for i in range(K)]
    ms = graph_ms if graph_ms is not None else eager_ms

    # what plain streaming reads reach on this device (4 GiB, beyond the
    # last-level cache), with the decode scan's own load instructions
    sr = torch.ones(1 << 30, dtype=torch.int32, device=dev)
    sink = adamas.stream_read(sr)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(5):
        adamas.stream_read(sr, sink)
    s1.record()
    torch.cuda.synchronize()
    stream_gbs = sr.numel() * 4 * 5 / (s0.elapsed_time(s1) * 1e-3) / 1e9
    del sr, sink

    if args.copy_calibration:
        # a plain conversion kernel of known traffic (reads 1 GiB of fp32,
        # writes 512 MiB of bf16) to scale the HBM byte counters
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        bb = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()

    per_layer = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 2)
    step_bytes = per_layer * L
    # The step is one decode launch per layer on one stream, so the average
    # launch duration over the timed region is the step time over L.
    avg_launch_us = ms * 1e3 / L
    achieved = per_layer / (avg_launch_us * 1e-6) / 1e9

    # recall of planted needles in the last step's selection (sanity signal)
    idx = torch.empty((B, Hq, bud), dtype=torch.int32, device=dev)
    lay = layers[0]
    adamas.decode_step(lay["q"], lay["k"], lay["v"], lay["codes"], n, bud, idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    found = sum(len(set(lay["needles"][0, h, 0].tolist()) & set(sel[0, h].tolist()))
                for h in range(Hq))
    recall = found / (Hq * w.needles)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(layers, w, n, bud, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": round(B / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "n_ctx": n, "layers": L, "budget": bud,
                   "timing": "hip-graph replay" if graph_ms is not None else "eager"},
        "hbm_gbs_step": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "eager_ms_per_step": round(eager_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "adamas_decode_step (one layer)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": per_layer, "launch_us": round(avg_launch_us, 3),
                     "eager_event_launch_us": round(launch_us, 3)},
        "step_ms": ({"p10": round(float(np.percentile(step_times, 10)), 4),
                     "p50": round(float(np.percentile(step_times, 50)), 4),
                     "p90": round(float(np.percentile(step_times, 90)), 4)}
                    if step_times else None),
        "stream_read": {"kernel": "adamas_stream_read over 4 GiB", "gbs": round(stream_gbs, 1),
                        "frac_of_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
                        "decode_over_stream": round(achieved / stream_gbs, 4)},
        "needle_recall": round(recall, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def stream_read_gbs(dev):
    """What plain streaming reads reach on this device (4 GiB, beyond the
    last-level cache), with the decode scan's own load instructions."""
    import torch

    import compressed_key_sparse_amd as adamas
    sr = torch.ones(1 << 30, dtype=torch.int32, device=dev)
    sink = adamas.stream_read(sr)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(5):
        adamas.stream_read(sr, sink)
    s1.record()
    torch.cuda.synchronize()
    return sr.numel() * 4 * 5 / (s0.elapsed_time(s1) * 1e-3) / 1e9


def timed_launches(launch, n_launch, stream, K):
    """Call launch(i) for i in [0, n_launch) K times, HIP events around each
    call on `stream` -> (ms per pass of n_launch calls, mean launch us)."""
    import numpy as np
    import torch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_launch)] for _ in range(K)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(K):
        for i in range(n_launch):
            ev[s][i][0].record(stream)
            launch(i)
            ev[s][i][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return (e0.elapsed_time(e1) / K,
            float(np.mean([a.elapsed_time(b) for row in ev for a, b in row]) * 1e3))


def result_line(metric, w, B, ms, K, warmup, cfg, kernel, per_launch, launch_us, stream_gbs,
                extra, cpu):
    achieved = per_launch / (launch_us * 1e-6) / 1e9
    res = {
        "metric": metric, "value": round(B / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": per_launch,
                     "launch_us": round(launch_us, 3)},
        "stream_read": {"kernel": "adamas_stream_read over 4 GiB", "gbs": round(stream_gbs, 1),
                        "frac_of_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
                        "decode_over_stream": round(achieved / stream_gbs, 4)},
        "cpu_baseline": cpu,
    }
    res.update(extra)
    print(json.dumps(res), flush=True)


def bench_gqa(args, dev):
    """One 1M-token GQA layer per step; four layers' caches cycled (1 GiB of
    codes, beyond the 256 MB last-level cache).  Timed as a replayed HIP graph
    of four steps."""
    import torch

    import compressed_key_sparse_amd as adamas
    import synth
    w = synth.LLAMA32_GQA_1M
    B, Hq, Hkv, d, n = w.batch, w.hq, w.hkv, w.head_dim, w.n_ctx
    bud = w.budget if args.budget == 256 else args.budget
    print(f"[bench] setup: 4 x GQA {Hq}/{Hkv} heads x {n} tokens, budget {bud}", file=sys.stderr,
          flush=True)
    layers = []
    for l in range(4):
        lay = synth.make_layer(w, l, dev)
        codes = torch.empty((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=dev)
        adamas.encode_keys(lay["k"], codes)
        layers.append((lay, codes, torch.empty_like(lay["q"])))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(dev)
    ws = adamas.Workspace(dev)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, n, bud, d))

    def launch(i):
        lay, codes, out = layers[i]
        adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, bud, out=out, ws=ws,
                           stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for i in range(4):
                launch(i)
    K = args.steps
    eager_ms, launch_us = timed_launches(launch, 4, stream, K)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(4):
                launch(i)
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(K):
            g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms = g0.elapsed_time(g1) / (4 * K)
    per_launch = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 2)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline([layers[0][0]], w.replace(layers=1), n, bud, args.cpu_seconds)
    result_line(
        f"decode-step tokens/s + achieved HBM GB/s, GQA 24/8 heads at 1M ctx, budget {bud}, 1 GPU",
        w, B, ms, K, args.warmup,
        {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
         "n_ctx": n, "budget": bud, "layers_cycled": 4, "timing": "hip-graph replay"},
        "adamas_decode_step (one layer)", per_launch, ms * 1e3, stream_read_gbs(dev),
        {"eager_ms_per_step": round(eager_ms / 4, 4),
         "eager_event_launch_us": round(launch_us, 3),
         "decode_path": adamas.decode_path(B, Hq, Hkv, n, bud, d)}, cpu)


def bench_batch_append(args, dev):
    """16 sequences of 65536 rows: each step appends one token per sequence
    and decodes (one launch on stream 1) while a 4096-token chunk for sequence
    (step mod 16) is encoded and its K rows copied into the reserved tail rows
    [65536, 69632) on stream 2.  Timed eagerly (the chunk's sequence changes
    every step): step = both streams done."""
    import numpy as np
    import torch

    import compressed_key_sparse_amd as adamas
    import synth
    w = synth.BATCH16_64K
    B, Hq, Hkv, d, n = w.batch, w.hq, w.hkv, w.head_dim, w.n_ctx
    bud = w.budget if args.budget == 256 else args.budget
    print(f"[bench] setup: batch {B} x {Hq} heads x {n} rows, budget {bud}, append", file=sys.stderr,
          flush=True)
    lay = synth.make_layer(w, 0, dev)
    codes = torch.empty((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=dev)
    for b in range(B):
        adamas.encode_keys(lay["k"][b:b + 1], codes[b:b + 1])
    P = 1024
    if args.paged:
        # the same rows moved into a shuffled pool of pages (+4 for the chunk)
        per = n // P
        n_pages = B * per + 4
        perm = np.random.default_rng(5).permutation(n_pages)
        table = torch.from_numpy(perm[:B * per].reshape(B, per).astype(np.int32)).to(dev)
        spare = [int(x) for x in perm[B * per:]]
        kp = torch.empty((n_pages, Hkv, P, d), dtype=w.torch_dtype, device=dev)
        vp = torch.empty_like(kp)
        cp = torch.empty((n_pages, Hkv, P, d // 4), dtype=torch.uint8, device=dev)
        for b in range(B):
            for i in range(per):
                pg = int(perm[b * per + i])
                kp[pg] = lay["k"][b, :, i * P:(i + 1) * P]
                vp[pg] = lay["v"][b, :, i * P:(i + 1) * P]
                cp[pg] = codes[b, :, i * P:(i + 1) * P]
        del lay["k"], lay["v"], codes
        torch.cuda.empty_cache()
    # every sequence holds n - 1 rows; the step appends row n - 1 and attends n
    lens = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
    kn = synth.random_values((B, Hkv, d), w.torch_dtype, 77, device=dev)
    vn = synth.random_values((B, Hkv, d), w.torch_dtype, 78, device=dev)
    chunks = [synth.make_chunk(w, s, dev) for s in range(4)]
    out = torch.empty_like(lay["q"])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    ws = adamas.Workspace(dev)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, n, bud, d))
    ev = {}

    def decode():
        if args.paged:
            adamas.decode_paged_step(lay["q"], kp, vp, cp, table, lens, n, bud, k_new=kn,
                                     v_new=vn, out=out, ws=ws, stream=s1)
        else:
            adamas.decode_append_step(lay["q"], lay["k"], lay["v"], codes, lens, n, bud, k_new=kn,
                                      v_new=vn, out=out, ws=ws, stream=s1)

    def step(i, timed=None):
        b = i % B
        s2.wait_stream(s1)
        with torch.cuda.stream(s2):
            ch = chunks[i % len(chunks)]
            if args.paged:   # the chunk's four pages, one encode call each
                for j, pg in enumerate(spare):
                    adamas.encode_keys(ch[:, :, j * P:(j + 1) * P].contiguous(),
                                       cp[pg:pg + 1], x_copy=kp[pg:pg + 1], stream=s2)
            else:
                adamas.encode_keys(ch, codes[b:b + 1], pos=n, x_copy=lay["k"][b:b + 1],
                                   stream=s2)
        if timed is not None:
            timed[0].record(s1)
        decode()
        if timed is not None:
            timed[1].record(s1)
        s1.wait_stream(s2)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(K)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    marks[0].record(s1)
    for i in range(K):
        step(i, pairs[i])
        marks[i + 1].record(s1)
    torch.cuda.synchronize()
    step_times = [marks[i].elapsed_time(marks[i + 1]) for i in range(K)]
    ms = marks[0].elapsed_time(marks[K]) / K
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in pairs]) * 1e3)
    # decode alone (no chunk on stream 2), for the launch's uncontended rate
    alone_ms, alone_us = timed_launches(lambda i: decode(), 1, s1, K)
    # plus the new rows: k_new, v_new read, K, V and code rows written
    per_launch = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 2) + B * Hkv * (4 * d * 2 + d // 4)
    chunk_bytes = Hkv * w.chunk * (2 * d * 2 + d // 4)   # read K, copy K, write codes
    cpu = None
    if args.cpu_seconds > 0 and not args.paged:
        cpu = cpu_baseline_append(lay, codes, lens, kn, vn, w, n, bud, args.cpu_seconds)
    result_line(
        f"batched decode+append tokens/s + achieved HBM GB/s, 16 x 64K ctx, budget {bud}, 1 GPU",
        w, B, ms, K, args.warmup,
        {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
         "n_ctx": n, "budget": bud, "prefill_chunk": w.chunk,
         "layout": "paged, 1024-token pages, shuffled" if args.paged else "contiguous",
         "timing": "eager, two streams, step = both done"},
        ("adamas_decode_paged_step" if args.paged else "adamas_decode_append_step")
        + " (16 sequences, 4096-token chunk encoding beside it)",
        per_launch, launch_us, stream_read_gbs(dev),
        {"step_ms": {"p10": round(float(np.percentile(step_times, 10)), 4),
                     "p50": round(float(np.percentile(step_times, 50)), 4),
                     "p90": round(float(np.percentile(step_times, 90)), 4)},
         "hbm_gbs_step": round((per_launch + chunk_bytes) / (ms * 1e-3) / 1e9, 1),
         "decode_alone_us": round(alone_us, 3),
         "decode_alone_gbs": round(per_launch / (alone_us * 1e-6) / 1e9, 1)}, cpu)


def cpu_baseline_append(lay, codes, lens, kn, vn, w, n, bud, seconds):
    """The oracle's append step on single sequences of the batch (cycled) until
    about `seconds` of oracle time; scaled to the 16-sequence step."""
    import numpy as np

    import oracle
    import synth
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    staged = []
    for b in (0, 5, 10):
        sl = slice(b, b + 1)
        k = synth.to_numpy_bits(lay["k"][sl, :, :n])
        staged.append((synth.to_numpy_bits(lay["q"][sl]), k, synth.to_numpy_bits(lay["v"][sl, :, :n]),
                       oracle.encode_keys(k), synth.to_numpy_bits(kn[sl]),
                       synth.to_numpy_bits(vn[sl])))
    spent, done = 0.0, 0
    while spent < seconds or done == 0:
        q, k, v, c, a, bvals = staged[done % len(staged)]
        t = time.perf_counter()
        oracle.decode_append_step(q, k, v, c, np.array([n - 1]), n, bud, a, bvals)
        spent += time.perf_counter() - t
        done += 1
    print(f"[bench] oracle: {done} single-sequence append steps in {spent:.1f}s", file=sys.stderr,
          flush=True)
    step = spent / done * w.batch
    return {"value": round(w.batch / step, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} single-sequence append+decode steps cycling over 3 sequences "
                      f"({w.hq} heads x {n} rows, budget {bud}), {spent:.1f}s of oracle time, "
                      f"scaled to the {w.batch}-sequence step"}


def cpu_baseline(layers, w, n, bud, seconds):
    """Time the CPU oracle's decode step on whole layers of the same workload
    (up to 4 distinct layers, cycled) until about `seconds` of oracle time has
    accumulated; scale to tokens/s for the full stack."""
    import oracle
    import synth

    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    staged = []
    for lay in layers[:4]:
        q, k, v = (synth.to_numpy_bits(lay[x]) for x in ("q", "k", "v"))
        staged.append((q, k, v, oracle.encode_keys(k)))   # prefill state, untimed
    spent, done = 0.0, 0
    while spent < seconds or done == 0:
        q, k, v, codes = staged[done % len(staged)]
        t = time.perf_counter()
        oracle.decode_step(q, k, v, codes, n, bud)
        spent += time.perf_counter() - t
        done += 1
    print(f"[bench] oracle: {done} layer steps in {spent:.1f}s", file=sys.stderr, flush=True)
    step = spent / done * w.layers
    return {"value": round(w.batch / step, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} single-layer decode steps cycling over {len(staged)} layers "
                      f"({w.hq} heads x {n} tokens, budget {bud}), {spent:.1f}s of oracle time, "
                      f"scaled to the {w.layers}-layer step"}


if __name__ == "__main__":
    main()
