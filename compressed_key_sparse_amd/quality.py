"""Synthetic quality sweep of the decode path (run: python -m compressed_key_sparse_amd.quality).

The ADAMAS article reports accuracy against the token budget (§5.2: 54 % at
64 tokens, 71 % at 128, 98 % at 1024 on a 128K-token model) and an ablation
with and without the Hadamard rotation (§3.2).  Neither model nor dataset is
available here; this sweep measures the same two questions on the synthetic
128K-token workload, whose heads carry planted "needle" keys close to the
query among outlier-channel noise:

  * recall   -- the fraction of planted needles that the selection keeps;
  * mass     -- the share of the dense softmax weight that falls on the
                selected rows (mean over heads); best_mass is the same for the
                budget's true top scores, the most any selection of that size
                can hold;
  * rel_err  -- ||o_sparse - o_dense|| / ||o_dense|| over all heads, with
                o_dense exact softmax attention over every cached row
                (plain fp32 PyTorch on the GPU, the reference), and o_sparse
                the library's decode step at that budget.  When the dense
                softmax sits on one or two rows, missing them costs about
                sqrt(2), whatever else is selected.

for budgets 64, 128, 256, 1024, with the rotation on and off.  Every step of
the sparse path runs in the library's kernels; PyTorch only computes the
dense reference.
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import torch

import compressed_key_sparse_amd as adamas


def dense_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, with_probs=False):
    """q [B][Hq][d], k/v [B][Hkv][n][d] -> exact softmax attention in fp32
    (and, with_probs, the softmax weights [B][Hq][n])."""
    B, Hq, d = q.shape
    Hkv, n = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    probs = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device) if with_probs else None
    for b in range(B):
        for h in range(Hq):
            kk = k[b, h // G].float()
            s = (kk @ q[b, h].float()) / math.sqrt(d)
            p = torch.softmax(s, dim=0)
            out[b, h] = p @ v[b, h // G].float()
            if with_probs:
                probs[b, h] = p
    return (out, probs) if with_probs else out


def sweep(layers: int = 4, budgets=(64, 128, 256, 1024), device: str = "cuda:0") -> list[dict]:
    import synth

    w = synth.LLAMA2_128K_32L
    dev = torch.device(device)
    rows = []
    try:
        for rotate in (True, False):
            adamas.set_rotation(rotate)
            stats = {bud: {"found": 0, "planted": 0, "err2": 0.0, "ref2": 0.0, "mass": 0.0,
                           "best": 0.0, "heads": 0} for bud in budgets}
            for l in range(layers):
                lay = synth.make_layer(w, l, dev)
                codes = torch.empty((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8,
                                    device=dev)
                adamas.encode_keys(lay["k"], codes)
                ref, probs = dense_attention(lay["q"], lay["k"], lay["v"], with_probs=True)
                G = w.hq // w.hkv
                for bud in budgets:
                    idx = torch.empty((w.batch, w.hq, bud), dtype=torch.int32, device=dev)
                    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, bud,
                                             idx_out=idx)
                    sel = idx.cpu().numpy()
                    st = stats[bud]
                    for b in range(w.batch):
                        for h in range(w.hq):
                            needles = lay["needles"][b, h // G, h % G]
                            planted = set(int(p) for p in needles if p >= 0)
                            st["found"] += len(planted & set(sel[b, h].tolist()))
                            st["planted"] += len(planted)
                    keep = idx.long().clamp(min=0)
                    got = torch.gather(probs, 2, keep) * (idx >= 0)
                    st["mass"] += float(got.sum())
                    st["best"] += float(torch.topk(probs, bud, dim=2).values.sum())
                    st["heads"] += w.batch * w.hq
                    st["err2"] += float(((out.float() - ref) ** 2).sum())
                    st["ref2"] += float((ref ** 2).sum())
                del lay, codes, ref, probs
                torch.cuda.empty_cache()
            for bud in budgets:
                st = stats[bud]
                rows.append({"rotation": rotate, "budget": bud,
                             "recall": round(st["found"] / max(st["planted"], 1), 4),
                             "mass": round(st["mass"] / st["heads"], 4),
                             "best_mass": round(st["best"] / st["heads"], 4),
                             "rel_err": round(math.sqrt(st["err2"] / st["ref2"]), 4),
                             "heads": layers * w.hq, "n_ctx": w.n_ctx})
    finally:
        adamas.set_rotation(True)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--layers", type=int, default=4)
    args = ap.parse_args(argv)
    adamas.load()
    rows = sweep(args.layers)
    for r in rows:
        print(json.dumps(r), flush=True)
    print("| rotation | budget | needle recall | softmax mass kept | best possible | "
          "rel. error vs dense |", file=sys.stderr)
    print("|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {'on' if r['rotation'] else 'off'} | {r['budget']} | {r['recall']:.3f} | "
              f"{r['mass']:.3f} | {r['best_mass']:.3f} | {r['rel_err']:.3f} |", file=sys.stderr)


if __name__ == "__main__":
    main()
