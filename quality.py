"""Synthetic quality sweep of the decode path (evaluation code, not part of
the library; run: python quality.py).

The ADAMAS article reports accuracy against the token budget (§5.2: 54 % at
64 tokens, 71 % at 128, 98 % at 1024 on a 128K-token model) and an ablation
with and without the Hadamard rotation (§3.2).  Neither model nor dataset is
available here; this sweep asks the same two questions on four seeded
128K-token stand-ins (synth.QUALITY_STANDINS):

  * needles: outlier channels (x20) in keys and queries alike, each query
    head with 8 planted keys near it (the benchmark's input);
  * needle-ramp: 6 outlier channels of gain 4 shared by queries and keys,
    8 planted keys whose noise ramps from 0.3 to 3;
  * needle-ramp-kout: the same ramp with the x20 outliers in the keys only;
  * kout-graded: outlier channels in the keys only, no planted keys, the
    query scaled so that the exact softmax spreads its weight over many rows.

For budgets 64, 128, 256 and 1024, with the rotation on and off (and, for
--alphas, other bucketing fractions), it reports

  * recall    -- the fraction of the exact top-budget rows (by q.k) that the
                 selection keeps;
  * needles   -- the fraction of planted needles kept ("needles" only);
  * mass      -- the share of the exact softmax weight on the selected rows
                 (mean over heads); best_mass is the same for the exact
                 top-budget rows, the most any selection of that size holds;
  * rel_err   -- ||o_sparse - o_dense|| / ||o_dense|| over all heads, with
                 o_dense exact softmax attention over every cached row and
                 o_sparse the library's decode step at that budget.

Every step of the sparse path runs in the library's kernels; PyTorch (fp32,
on the GPU) computes only the dense reference here.
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


def _configs(alphas):
    """(rotation, alpha) pairs: both rotations at the fixed rule, then each
    extra alpha with the rotation on."""
    out = [(True, 0.5), (False, 0.5)]
    out += [(True, a) for a in alphas if a != 0.5]
    return out


def sweep(standins=None, layers: int = 4, budgets=(64, 128, 256, 1024), alphas=(),
          device: str = "cuda:0") -> list[dict]:
    import synth

    standins = standins or synth.QUALITY_STANDINS
    dev = torch.device(device)
    rows = []
    try:
        for w in standins:
            cfgs = _configs(alphas)
            stats = {(c, bud): {"found": 0, "planted": 0, "hit": 0, "want": 0, "err2": 0.0,
                                "ref2": 0.0, "mass": 0.0, "best": 0.0, "heads": 0}
                     for c in cfgs for bud in budgets}
            G = w.hq // w.hkv
            for l in range(layers):
                lay = synth.make_layer(w, l, dev)
                ref, probs = dense_attention(lay["q"], lay["k"], lay["v"], with_probs=True)
                top = {bud: torch.topk(probs, bud, dim=2) for bud in budgets}
                for cfg in cfgs:
                    rotate, alpha = cfg
                    adamas.set_rotation(rotate)
                    adamas.set_bucket_alpha(None if alpha == 0.5 else [alpha])
                    codes = torch.empty((w.batch, w.hkv, w.cap, w.head_dim // 4),
                                        dtype=torch.uint8, device=dev)
                    adamas.encode_keys(lay["k"], codes)
                    for bud in budgets:
                        idx = torch.empty((w.batch, w.hq, bud), dtype=torch.int32, device=dev)
                        out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx,
                                                 bud, idx_out=idx)
                        st = stats[(cfg, bud)]
                        sel = idx.cpu().numpy()
                        for b in range(w.batch):
                            for h in range(w.hq):
                                planted = set(int(p) for p in lay["needles"][b, h // G, h % G]
                                              if p >= 0)
                                st["found"] += len(planted & set(sel[b, h].tolist()))
                                st["planted"] += len(planted)
                        # overlap with the exact top-budget rows
                        hit = (idx.long().unsqueeze(-1) == top[bud].indices.unsqueeze(-2))
                        st["hit"] += int(hit.any(dim=-1).sum())
                        st["want"] += w.batch * w.hq * bud
                        keep = idx.long().clamp(min=0)
                        got = torch.gather(probs, 2, keep) * (idx >= 0)
                        st["mass"] += float(got.sum())
                        st["best"] += float(top[bud].values.sum())
                        st["heads"] += w.batch * w.hq
                        st["err2"] += float(((out.float() - ref) ** 2).sum())
                        st["ref2"] += float((ref ** 2).sum())
                    del codes
                del lay, ref, probs, top
                torch.cuda.empty_cache()
            for cfg in cfgs:
                for bud in budgets:
                    st = stats[(cfg, bud)]
                    rows.append({
                        "standin": w.name, "rotation": cfg[0],
                        "alpha": cfg[1], "budget": bud,
                        "recall": round(st["hit"] / max(st["want"], 1), 4),
                        "needles": (round(st["found"] / st["planted"], 4) if st["planted"]
                                    else None),
                        "mass": round(st["mass"] / st["heads"], 4),
                        "best_mass": round(st["best"] / st["heads"], 4),
                        "rel_err": round(math.sqrt(st["err2"] / st["ref2"]), 4),
                        "heads": layers * w.hq, "n_ctx": w.n_ctx})
    finally:
        adamas.set_rotation(True)
        adamas.set_bucket_alpha(None)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--alphas", default="", help="extra bucketing fractions, comma separated")
    args = ap.parse_args(argv)
    adamas.load()
    alphas = tuple(float(a) for a in args.alphas.split(",") if a.strip())
    rows = sweep(layers=args.layers, alphas=alphas)
    for r in rows:
        print(json.dumps(r), flush=True)
    print("| stand-in | rotation | alpha | budget | top-B recall | needles kept | softmax mass "
          "kept | best possible | rel. error vs dense |", file=sys.stderr)
    print("|---|---|---|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        nd = "–" if r["needles"] is None else f"{r['needles']:.3f}"
        print(f"| {r['standin']} | {'on' if r['rotation'] else 'off'} | {r['alpha']} | "
              f"{r['budget']} | {r['recall']:.3f} | {nd} | {r['mass']:.3f} | "
              f"{r['best_mass']:.3f} | {r['rel_err']:.3f} |", file=sys.stderr)


if __name__ == "__main__":
    main()
