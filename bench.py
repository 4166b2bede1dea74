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
                            the chunk fills four spare pool pages
                            (adamas_encode_keys_paged).
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
    ap.add_argument("--steps", type=int, default=50)
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
                    choices=(HEADLINE, "llama3.2-3b-gqa-1m", "batch16-mha-64k-append4k",
                             "llama2-mha-32k", "tiny-1h-d64-1k"))
    ap.add_argument("--replicas", type=int, default=8,
                    help="single-layer workloads: distinct copies of the layer cycled so that "
                         "no launch finds its caches in the last-level cache")
    ap.add_argument("--paged", action="store_true",
                    help="batch16 workload: caches in a shuffled pool of 1024-token pages")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="print a compact summary of rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--last", type=int, default=None,
                    help="with --summarize: per-kernel statistics of the last N dispatches of a "
                         "kernel trace (the timed graph replays of a --graph-only run)")
    ap.add_argument("--graph-only", action="store_true",
                    help="skip the eager timed pass and the trailing recall launch, so the last "
                         "steps*layers decode dispatches of a kernel trace are the timed replays")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write the headline HBM traffic file from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--decode-mode", default="auto",
                    choices=("auto", "last-arrival", "group-wait", "split"),
                    help="schedule of the decode step (adamas_set_decode_mode); auto by default")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase timeline of the workload's decode launches from the "
                         "measurement build (libadamas_phases.so); prints a table, no JSON line")
    return ap.parse_args()


# ---------------------------------------------------------------- profiles
KERNEL_SOURCES = ("compressed_key_sparse_amd/csrc/adamas.hip",
                  "compressed_key_sparse_amd/csrc/decode_inst.hip",
                  "compressed_key_sparse_amd/csrc/plan.hpp",
                  "compressed_key_sparse_amd/csrc/kernels.hpp",
                  "compressed_key_sparse_amd/csrc/device_common.hpp",
                  "include/adamas.h")
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


def _counter_means(dirpath: str, counter: str):
    """{(kernel name, grid): mean value per dispatch} of one PMC counter."""
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(list)
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc[(r.get("Kernel_Name", ""), r.get("Grid_Size", ""))].append(
                        float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(fetch_dir: str, write_dir: str, out: str = TRAFFIC_FILE):
    """HBM bytes per headline decode launch from a FETCH_SIZE and a
    WRITE_SIZE run (each of bench.py --no-graph --copy-calibration), each
    counter scaled by what it reads for the calibration conversion (1 GiB
    fp32 read, 512 MiB bf16 written, grid 2^25); written with the kernel
    source hash so that a later kernel change voids it."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")

    def pick(m, pred):
        hits = [v for (name, grid), v in m.items() if pred(name, grid)]
        if len(hits) != 1:
            raise SystemExit(f"bench.py --traffic-from: expected one matching kernel, got {len(hits)}")
        return hits[0]

    dec = lambda name, grid: name.startswith("void adm::k_decode<128, 1, true, 0,")
    cal = lambda name, grid: "bfloat16_copy_kernel" in name and grid == str(1 << 25)
    fk, wk = pick(fetch, dec), pick(write, dec)
    fs, ws = (1 << 30) / 1024 / pick(fetch, cal), (1 << 29) / 1024 / pick(write, cal)
    traffic = int(round((fk * fs + wk * ws) * 1024))
    alg = algorithmic_bytes(1, 32, 32, 128, 131072, 256, 2)
    res = {"kernel": "k_decode<128,1,bf16,plain>", "workload": "llama2-mha-128k-32layers budget 256",
           "kernel_source_hash": kernel_source_hash(), "fetch_kib_per_dispatch": round(fk, 1),
           "write_kib_per_dispatch": round(wk, 1), "fetch_scale": round(fs, 5),
           "write_scale": round(ws, 5), "traffic_bytes_per_launch": traffic,
           "algorithmic_bytes_per_launch": alg}
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))
    print(f"# traffic {traffic} bytes per launch = {traffic / alg:.4f} x algorithmic")


def summarize_trace(dirpath: str, last: int):
    """Per-kernel durations of the last `last` dispatches in a rocprofv3
    --kernel-trace CSV (End_Timestamp - Start_Timestamp, ns)."""
    import csv
    import glob
    from collections import defaultdict

    import numpy as np
    for f in sorted(glob.glob(os.path.join(dirpath, "**", "*kernel_trace.csv"), recursive=True)):
        runs = defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if "adm::" not in name:
                    continue
                runs[name].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        print(f"# kernel trace ({os.path.basename(f)}): last {last} dispatches per kernel")
        print("dispatches  avg_us   median_us  min_us   max_us   gap_avg_us  kernel")
        for name, rs in sorted(runs.items()):
            rs.sort()
            sel = rs[-last:]
            dur = np.array([(e - s) / 1e3 for s, e in sel])
            gaps = np.array([(sel[i + 1][0] - sel[i][1]) / 1e3 for i in range(len(sel) - 1)])
            print(f"{len(sel):10d} {dur.mean():8.3f} {np.median(dur):9.3f} {dur.min():8.3f} "
                  f"{dur.max():8.3f} {gaps.mean() if gaps.size else 0.0:10.3f}  {name[:100]}")


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
        # ratios of the LDS and occupancy counters, per kernel and grid
        per = defaultdict(dict)
        for (name, cn, grid), vals in acc.items():
            per[(name, grid)][cn] = sum(vals) / len(vals)
        rows = []
        for (name, grid), c in sorted(per.items()):
            if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
                conf = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
                occ = (c["SQ_WAVE_CYCLES"] / c["SQ_BUSY_CU_CYCLES"]
                       if c.get("SQ_BUSY_CU_CYCLES") else float("nan"))
                valu = (100 * c["SQ_ACTIVE_INST_VALU"] / (256 * c["GRBM_GUI_ACTIVE"])
                        if c.get("GRBM_GUI_ACTIVE") and "SQ_ACTIVE_INST_VALU" in c else float("nan"))
                rows.append(f"{conf:9.4f}  {occ:10.2f}  {valu:9.1f}  {grid}  {name[:90]}")
        if rows:
            print("# derived: LDS bank-conflict cycles / LDS-active cycles; waves resident per busy CU "
                  "(SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES); VALU busy % "
                  "(100 * SQ_ACTIVE_INST_VALU / (256 CUs * GRBM_GUI_ACTIVE))")
            print("conflict  waves/CU    valu_%  grid  kernel")
            print("\n".join(rows))


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.summarize:
        if args.last:
            summarize_trace(args.summarize, args.last)
        else:
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
    adamas.load(variant="phases" if args.phases else None)
    adamas.set_decode_mode({"auto": adamas.DECODE_AUTO, "last-arrival": adamas.DECODE_LAST_ARRIVAL,
                            "group-wait": adamas.DECODE_GROUP_WAIT,
                            "split": adamas.DECODE_SPLIT}[args.decode_mode])
    if args.phases:
        return bench_phases(args, dev)
    if args.workload == "llama3.2-3b-gqa-1m":
        return bench_gqa(args, dev)
    if args.workload == "batch16-mha-64k-append4k":
        return bench_batch_append(args, dev)
    if args.workload in ("llama2-mha-32k", "tiny-1h-d64-1k"):
        return bench_single(args, dev, synth.WORKLOADS[args.workload])
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
    eager_ms = launch_us = None
    if not args.graph_only:
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(K)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(K):
            for l, lay in enumerate(layers):
                ev[s][l][0].record(stream)
                adamas.decode_step(lay["q"], lay["k"], lay["v"], lay["codes"], n, bud,
                                   out=lay["out"], ws=ws, stream=stream)
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
    if ms is None:
        raise SystemExit("bench.py: --graph-only with --no-graph times nothing")
    if ws.status() != 0:
        raise SystemExit("bench.py: a group-wait decode step gave up waiting (workspace status "
                         "word set): the timed outputs are invalid")

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
    cr_us, cr_gbs = code_read_floor([lay["codes"] for lay in layers], stream, K, args.warmup)

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
    recall = None
    if not args.graph_only:
        idx = torch.empty((B, Hq, bud), dtype=torch.int32, device=dev)
        lay = layers[0]
        adamas.decode_step(lay["q"], lay["k"], lay["v"], lay["codes"], n, bud, idx_out=idx,
                           ws=ws)
        torch.cuda.synchronize()
        sel = idx.cpu().numpy()
        found = sum(len(set(lay["needles"][0, h, 0].tolist()) & set(sel[0, h].tolist()))
                    for h in range(Hq))
        recall = round(found / (Hq * w.needles), 4)

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
        "eager_ms_per_step": round(eager_ms, 4) if eager_ms is not None else None,
        "roofline": {"bound": "hbm", "kernel": "adamas_decode_step (one layer)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # the counters were taken on this configuration only
                     "traffic": measured_traffic() if (bud, n, B, Hq, d) == (256, 131072, 1, 32, 128)
                     else None,
                     "bytes_per_launch": per_layer, "launch_us": round(avg_launch_us, 3),
                     "eager_event_launch_us": round(launch_us, 3) if launch_us else None},
        "step_ms": ({"p10": round(float(np.percentile(step_times, 10)), 4),
                     "p50": round(float(np.percentile(step_times, 50)), 4),
                     "p90": round(float(np.percentile(step_times, 90)), 4)}
                    if step_times else None),
        "stream_read": {"kernel": "adamas_stream_read over 4 GiB", "gbs": round(stream_gbs, 1),
                        "frac_of_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
                        "decode_over_stream": round(achieved / stream_gbs, 4)},
        "code_read": code_read_entry(cr_us, cr_gbs, achieved, L),
        "needle_recall": recall,
        "decode_path": adamas.decode_path(B, Hq, Hkv, n, bud, d),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


PHASE_NAMES = {
    "decode": {0: "entry", 1: "query encoded", 2: "scan end", 3: "chunk threshold",
               4: "candidates staged", 5: "handed over / histograms published",
               6: "final: candidates loaded", 7: "final: threshold", 8: "final: selected",
               9: "rows gathered + weighted", 10: "partials merged", 11: "final: out stored",
               12: "merged out stored", 13: "rows gathered, last wavefront",
               14: "slot sums, last wavefront", 16: "chunk: thresholds (grouped heads)",
               17: "chunk: masks, last wavefront", 18: "chunk: prefix over workgroup",
               19: "chunk: tokens emitted, last wavefront", 20: "final: counts, last wavefront",
               21: "final: prefix", 22: "final: placed, last wavefront"},
    "split": {0: "entry", 1: "threshold", 2: "placement", 3: "tokens copied",
              9: "rows gathered + weighted", 10: "partials merged", 11: "partial handed over",
              12: "merged out stored", 13: "rows gathered, last wavefront",
              14: "slot sums, last wavefront"},
    "attend": {0: "entry", 9: "rows gathered + weighted", 10: "partials merged",
               11: "partial handed over", 12: "merged out stored",
               13: "rows gathered, last wavefront", 14: "slot sums, last wavefront"},
}


def phase_table(samples, ticks_per_us):
    """Per-phase times of the workgroups of each launch, relative to the
    launch's first workgroup start (slot 0 of the decode region), in us:
    medians over launches of the per-launch median, 90th percentile and
    maximum over the workgroups that reached the slot."""
    import numpy as np
    from collections import defaultdict
    acc = defaultdict(list)
    for st in samples:                      # [regions][workgroups][slots] per launch
        starts = st[:, :, 0][st[:, :, 0] > 0]
        if starts.size == 0:
            continue
        t0 = starts.min()
        for ri, region in enumerate(("decode", "split", "attend")):
            for slot in range(st.shape[2]):
                v = st[ri, :, slot]
                v = v[v > 0]
                if v.size:
                    us = (v - t0) / ticks_per_us
                    acc[(ri, region, slot)].append(
                        (np.median(us), np.percentile(us, 90), us.max(), v.size))
    lines = ["region  slot  phase                                  wgs   median_us  p90_us   max_us"]
    for (ri, region, slot), rows in sorted(acc.items()):
        r = np.median(np.array(rows), axis=0)
        name = PHASE_NAMES[region].get(slot, f"slot {slot}")
        lines.append(f"{region:7s} {slot:4d}  {name:38s} {int(r[3]):5d} {r[0]:10.2f} {r[1]:8.2f} "
                     f"{r[2]:8.2f}")
    return "\n".join(lines)


def bench_phases(args, dev):
    """Per-phase timeline of decode launches, from the measurement build:
    every launch runs alone (synchronised before and after) and its
    workgroups' stamps are read back.  Workloads as in the timed runs: the
    128K layer stack (cycling --layers, default 8, layers' caches so the
    codes do not sit in the last-level cache), the GQA 1M layer (4 layers
    cycled) or the batch-16 append step."""
    import torch

    import compressed_key_sparse_amd as adamas
    import synth
    rec = adamas.PhaseRecorder(dev)
    launches = []
    if args.workload == "batch16-mha-64k-append4k":
        w = synth.BATCH16_64K
        bud = w.budget if args.budget == 256 else args.budget
        st = BatchAppendState(w, dev, bud, paged=args.paged)
        launches = [lambda: st.decode()]
        desc = f"{w.name}{' paged' if args.paged else ''}, budget {bud}"
    else:
        if args.workload == "llama3.2-3b-gqa-1m":
            w, L = synth.LLAMA32_GQA_1M, 4
            bud = w.budget if args.budget == 256 else args.budget
        else:
            w, L, bud = synth.LLAMA2_128K_32L, args.layers or 8, args.budget
            if args.n_ctx:
                w = w.replace(n_ctx=args.n_ctx, cap=args.n_ctx)
        ws = adamas.Workspace(dev)
        ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, w.batch, w.hq, w.hkv, w.n_ctx, bud,
                                      w.head_dim))
        stack = []
        for l in range(L):
            lay = synth.make_layer(w, l, dev)
            codes = torch.empty((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8,
                                device=dev)
            adamas.encode_keys(lay["k"], codes)
            stack.append((lay, codes, torch.empty_like(lay["q"])))
        for lay, codes, out in stack:
            launches.append(lambda lay=lay, codes=codes, out=out: adamas.decode_step(
                lay["q"], lay["k"], lay["v"], codes, w.n_ctx, bud, out=out, ws=ws))
        desc = (f"{w.name}, {w.hq}/{w.hkv} heads x {w.n_ctx} tokens, budget {bud}, "
                f"path {adamas.decode_path(w.batch, w.hq, w.hkv, w.n_ctx, bud, w.head_dim)}")
    torch.cuda.synchronize()
    for f in launches:                      # warm-up
        f()
    samples = []
    reps = max(1, args.steps // len(launches)) * len(launches)
    for i in range(reps):
        rec.clear()
        torch.cuda.synchronize()
        launches[i % len(launches)]()
        samples.append(rec.read())
    # the same launches back to back (as in a step), timed on the stream: the
    # read-ahead of one launch feeds the next one only when they follow closely
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        launches[i % len(launches)]()
    e1.record()
    torch.cuda.synchronize()
    print(f"# back to back: {e0.elapsed_time(e1) * 1e3 / reps:.2f} us per launch", flush=True)
    rec.close()
    print(f"# phase timeline: {desc}; {len(samples)} launches, wall clock "
          f"{rec.ticks_per_us:.0f} ticks/us", flush=True)
    print(phase_table(samples, rec.ticks_per_us), flush=True)


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


def code_read_floor(code_caches, stream, K, warmup):
    """The same streaming read over each layer's code cache in turn (the
    bytes one decode launch scans, nothing else), replayed as a HIP graph like
    the decode steps: the time a launch needs to read its codes at this size,
    ramp-up and drain included.  -> (us per cache, GB/s)."""
    import torch

    import compressed_key_sparse_amd as adamas
    sinks = [adamas.stream_read(c, stream=stream) for c in code_caches]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for c, k in zip(code_caches, sinks):
                adamas.stream_read(c, k, stream=stream)
        for _ in range(warmup):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(K):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (K * len(code_caches))
    nbytes = code_caches[0].numel() * code_caches[0].element_size()
    return us, nbytes / (us * 1e-6) / 1e9


def code_read_entry(us, gbs, achieved, n_caches):
    return {"kernel": f"adamas_stream_read of each code cache in turn ({n_caches}), graph replay",
            "us_per_cache": round(us, 3), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "decode_over_code_read": round(achieved / gbs, 4)}


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


def bench_single(args, dev, w):
    """Latency of one decode-step launch of a single-layer workload (the
    32K-token Llama-2-shaped layer, or the tiny single-head fp32 case):
    --replicas distinct copies of the layer (caches and codes) are cycled in
    a replayed HIP graph, so that each launch reads its codes from HBM rather
    than from the last-level cache.  value = batch / launch time."""
    import numpy as np
    import torch

    import compressed_key_sparse_amd as adamas
    import synth
    B, Hq, Hkv, d, n = w.batch, w.hq, w.hkv, w.head_dim, w.n_ctx
    bud = w.budget if args.budget == 256 else args.budget
    R = max(1, args.replicas)
    print(f"[bench] setup: {R} replicas of {w.name}, budget {bud}", file=sys.stderr, flush=True)
    reps = []
    for r in range(R):
        lay = synth.make_layer(w, r, dev)
        codes = torch.empty((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=dev)
        adamas.encode_keys(lay["k"], codes)
        reps.append((lay, codes, torch.empty_like(lay["q"])))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(dev)
    ws = adamas.Workspace(dev)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, n, bud, d))

    def launch(i):
        lay, codes, out = reps[i]
        adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, bud, out=out, ws=ws,
                           stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for i in range(R):
                launch(i)
    K = args.steps
    eager_ms, launch_us = timed_launches(launch, R, stream, K)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(R):
                launch(i)
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    marks[0].record(stream)
    with torch.cuda.stream(stream):
        for i in range(K):
            g.replay()
            marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [marks[i].elapsed_time(marks[i + 1]) * 1e3 / R for i in range(K)]
    us = marks[0].elapsed_time(marks[K]) * 1e3 / (R * K)
    if ws.status() != 0:
        raise SystemExit("bench.py: a group-wait decode step gave up waiting")
    per_launch = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 4 if w.dtype == "f32" else 2)
    cr_us, cr_gbs = code_read_floor([r[1] for r in reps], stream, K, args.warmup)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline([r[0] for r in reps[:4]], w.replace(layers=1), n, bud,
                           args.cpu_seconds)
    result_line(
        f"decode-step latency + achieved HBM GB/s, {w.name}, budget {bud}, 1 GPU",
        w, B, us * 1e-3, K, args.warmup,
        {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
         "n_ctx": n, "budget": bud, "replicas_cycled": R, "timing": "hip-graph replay"},
        "adamas_decode_step (one layer)", per_launch, us, stream_read_gbs(dev),
        {"launch_us": {"mean": round(us, 3), "p10": round(float(np.percentile(per, 10)), 3),
                       "p50": round(float(np.percentile(per, 50)), 3),
                       "p90": round(float(np.percentile(per, 90)), 3)},
         "eager_event_launch_us": round(launch_us, 3),
         "code_read": code_read_entry(cr_us, cr_gbs, per_launch / (us * 1e-6) / 1e9, R),
         "decode_path": adamas.decode_path(B, Hq, Hkv, n, bud, d)}, cpu)


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
    if ws.status() != 0:
        raise SystemExit("bench.py: a group-wait decode step gave up waiting (workspace status "
                         "word set): the timed outputs are invalid")
    per_launch = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 2)
    cr_us, cr_gbs = code_read_floor([c for _, c, _ in layers], stream, K, args.warmup)
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
         "code_read": code_read_entry(cr_us, cr_gbs, per_launch / (ms * 1e-3) / 1e9, 4),
         "decode_path": adamas.decode_path(B, Hq, Hkv, n, bud, d)}, cpu)


class BatchAppendState:
    """The batch-16 append workload as the benchmark runs it: 16 sequences of
    65536 rows, each holding n - 1 rows so that the step appends row n - 1 and
    attends over n; one decode launch per step on stream s1 while a
    4096-token chunk for sequence (step mod 16) is encoded and its K rows
    copied into the reserved tail rows [65536, 69632) on stream s2.  With
    paged=True the same rows sit in a shuffled pool of 1024-token pages and
    the chunk fills four spare pool pages (one adamas_encode_keys_paged
    call).  The parity tests build the same state and check the same calls."""

    PAGE = 1024

    def __init__(self, w, dev, bud, paged=False):
        import numpy as np
        import torch

        import compressed_key_sparse_amd as adamas
        import synth
        self.w, self.dev, self.bud, self.paged = w, dev, bud, paged
        B, Hkv, d, n = w.batch, w.hkv, w.head_dim, w.n_ctx
        lay = synth.make_layer(w, 0, dev)
        codes = torch.empty((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=dev)
        for b in range(B):
            adamas.encode_keys(lay["k"][b:b + 1], codes[b:b + 1])
        P = self.PAGE
        self.q = lay["q"]
        if paged:
            per = n // P
            n_pages = B * per + 4
            perm = np.random.default_rng(5).permutation(n_pages)
            self.table = torch.from_numpy(perm[:B * per].reshape(B, per).astype(np.int32)).to(dev)
            self.spare = [int(x) for x in perm[B * per:]]
            self.spare_table = torch.tensor([self.spare], dtype=torch.int32, device=dev)
            self.kp = torch.empty((n_pages, Hkv, P, d), dtype=w.torch_dtype, device=dev)
            self.vp = torch.empty_like(self.kp)
            self.cp = torch.empty((n_pages, Hkv, P, d // 4), dtype=torch.uint8, device=dev)
            for b in range(B):
                for i in range(per):
                    pg = int(perm[b * per + i])
                    self.kp[pg] = lay["k"][b, :, i * P:(i + 1) * P]
                    self.vp[pg] = lay["v"][b, :, i * P:(i + 1) * P]
                    self.cp[pg] = codes[b, :, i * P:(i + 1) * P]
            del lay, codes
            torch.cuda.empty_cache()
        else:
            self.k, self.v, self.codes = lay["k"], lay["v"], codes
        self.lens = torch.full((B,), n - 1, dtype=torch.int32, device=dev)
        self.kn = synth.random_values((B, Hkv, d), w.torch_dtype, 77, device=dev)
        self.vn = synth.random_values((B, Hkv, d), w.torch_dtype, 78, device=dev)
        self.chunks = [synth.make_chunk(w, s, dev) for s in range(4)]
        self.out = torch.empty_like(self.q)
        torch.cuda.synchronize()
        self.s1, self.s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
        self.ws = adamas.Workspace(dev)
        self.ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, w.hq, Hkv, n, bud, d))

    def decode(self, idx_out=None):
        import compressed_key_sparse_amd as adamas
        n = self.w.n_ctx
        if self.paged:
            adamas.decode_paged_step(self.q, self.kp, self.vp, self.cp, self.table, self.lens, n,
                                     self.bud, k_new=self.kn, v_new=self.vn, out=self.out,
                                     idx_out=idx_out, ws=self.ws, stream=self.s1)
        else:
            adamas.decode_append_step(self.q, self.k, self.v, self.codes, self.lens, n, self.bud,
                                      k_new=self.kn, v_new=self.vn, out=self.out,
                                      idx_out=idx_out, ws=self.ws, stream=self.s1)

    def encode_chunk(self, i, stream=None):
        """Enqueue step i's prefill chunk (its sequence is i mod 16) on s2, or
        on `stream`."""
        import torch

        import compressed_key_sparse_amd as adamas
        b, n, P = i % self.w.batch, self.w.n_ctx, self.PAGE
        s = self.s2 if stream is None else stream
        with torch.cuda.stream(s):
            ch = self.chunks[i % len(self.chunks)]
            if self.paged:   # the chunk into its four spare pool pages, one call
                adamas.encode_keys_paged(ch, self.cp, self.spare_table, x_pool=self.kp,
                                         stream=s)
            else:
                adamas.encode_keys(ch, self.codes[b:b + 1], pos=n, x_copy=self.k[b:b + 1],
                                   stream=s)

    def step(self, i, timed=None, idx_out=None):
        self.s2.wait_stream(self.s1)
        self.encode_chunk(i)
        if timed is not None:
            timed[0].record(self.s1)
        self.decode(idx_out)
        if timed is not None:
            timed[1].record(self.s1)
        self.s1.wait_stream(self.s2)


def bench_batch_append(args, dev):
    """16 sequences of 65536 rows: each step appends one token per sequence
    and decodes (one launch on stream 1) while a 4096-token chunk for sequence
    (step mod 16) is encoded and its K rows copied into the reserved tail rows
    [65536, 69632) on stream 2 (BatchAppendState).  Timed eagerly (the
    chunk's sequence changes every step).  The chunk writes rows no decode
    step reads, so stream 1 never waits for stream 2 inside the timed region:
    step i's chunk starts once step i - 1's decode is done (an event that
    stream 2 waits for) and runs beside step i's decode; both streams are
    joined at the ends of the K steps, and step time = that region / K.  The
    same K steps with both streams joined after every step (step_joined_ms)
    add a cross-stream wait each way per step."""
    import numpy as np
    import torch

    import synth
    w = synth.BATCH16_64K
    B, Hq, Hkv, d, n = w.batch, w.hq, w.hkv, w.head_dim, w.n_ctx
    bud = w.budget if args.budget == 256 else args.budget
    print(f"[bench] setup: batch {B} x {Hq} heads x {n} rows, budget {bud}, append", file=sys.stderr,
          flush=True)
    st = BatchAppendState(w, dev, bud, paged=args.paged)
    s1, s2, step, decode = st.s1, st.s2, st.step, st.decode
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps

    def event_pairs():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(K)]

    # the timed run: chunk i on stream 2 after decode i - 1, beside decode i
    pairs = event_pairs()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s1)
    s2.wait_stream(s1)
    for i in range(K):
        if i > 0:
            s2.wait_event(pairs[i - 1][1])
        st.encode_chunk(i)
        pairs[i][0].record(s1)
        decode()
        pairs[i][1].record(s1)
    s1.wait_stream(s2)
    e1.record(s1)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in pairs]) * 1e3)
    # the same steps with both streams joined after each one
    jpairs = event_pairs()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    marks[0].record(s1)
    for i in range(K):
        step(i, jpairs[i])
        marks[i + 1].record(s1)
    torch.cuda.synchronize()
    step_times = [marks[i].elapsed_time(marks[i + 1]) for i in range(K)]
    # and with each chunk on stream 1, before its step's decode (no overlap)
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0.record(s1)
    for i in range(K):
        st.encode_chunk(i, stream=s1)
        decode()
    o1.record(s1)
    torch.cuda.synchronize()
    one_stream_ms = o0.elapsed_time(o1) / K
    # decode alone (no chunk on stream 2), for the launch's uncontended rate
    alone_ms, alone_us = timed_launches(lambda i: decode(), 1, s1, K)
    # plus the new rows: k_new, v_new read, K, V and code rows written
    per_launch = algorithmic_bytes(B, Hq, Hkv, d, n, bud, 2) + B * Hkv * (4 * d * 2 + d // 4)
    chunk_bytes = Hkv * w.chunk * (2 * d * 2 + d // 4)   # read K, copy K, write codes
    cpu = None
    if args.cpu_seconds > 0 and not args.paged:
        cpu = cpu_baseline_append(st, w, n, bud, args.cpu_seconds)
    result_line(
        f"batched decode+append tokens/s + achieved HBM GB/s, 16 x 64K ctx, budget {bud}, 1 GPU",
        w, B, ms, K, args.warmup,
        {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
         "n_ctx": n, "budget": bud, "prefill_chunk": w.chunk,
         "layout": "paged, 1024-token pages, shuffled" if args.paged else "contiguous",
         "timing": "eager; chunk i on stream 2 beside decode i, streams joined at the ends"},
        ("adamas_decode_paged_step" if args.paged else "adamas_decode_append_step")
        + " (16 sequences, 4096-token chunk encoding beside it)",
        per_launch, launch_us, stream_read_gbs(dev),
        {"step_joined_ms": {"mean": round(marks[0].elapsed_time(marks[K]) / K, 4),
                            "p10": round(float(np.percentile(step_times, 10)), 4),
                            "p50": round(float(np.percentile(step_times, 50)), 4),
                            "p90": round(float(np.percentile(step_times, 90)), 4)},
         "one_stream_ms": round(one_stream_ms, 4),
         "hbm_gbs_step": round((per_launch + chunk_bytes) / (ms * 1e-3) / 1e9, 1),
         "decode_alone_us": round(alone_us, 3),
         "decode_alone_gbs": round(per_launch / (alone_us * 1e-6) / 1e9, 1)}, cpu)


def cpu_baseline_append(st, w, n, bud, seconds):
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
        k = synth.to_numpy_bits(st.k[sl, :, :n])
        staged.append((synth.to_numpy_bits(st.q[sl]), k, synth.to_numpy_bits(st.v[sl, :, :n]),
                       oracle.encode_keys(k), synth.to_numpy_bits(st.kn[sl]),
                       synth.to_numpy_bits(st.vn[sl])))
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
