"""Seeded synthetic inputs for the ADAMAS decode path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, bucketing, scoring, selection or attention),
so both the HIP path and the CPU oracle can take their inputs from it.

The pages measure on model activations (Llama-2-7B, Yarn-Llama-2-7B-128K,
Llama-3.2-3B) and datasets that are not available here; these seeded caches
stand in for them with the same shapes:
  * per-channel lognormal scales (sigma 0.5) with about 2 % outlier channels
    multiplied by 20, the outlier structure the ADAMAS article's §2.1 describes
    the rotation smoothing out;
  * queries correlated with planted "needle" keys, a synthetic analogue of the
    needle-retrieval evaluations the pages mention;
  * for the quality sweep only, three more stand-ins (QUALITY_STANDINS): graded
    relevance with outlier channels in the keys alone (no planted keys; the
    query scaled so that its softmax weight spreads over many rows), and
    needles of increasing noise (equal expected scores, decreasing similarity
    to the query) with milder outliers shared by queries and keys, or with
    the x20 outliers in the keys alone.

Bulk normal draws use a torch generator on the requested device (so large
caches are produced on the GPU); structural choices (outlier channels, scales,
needle positions) use numpy's PCG64 so that they do not depend on the device.
The oracle always receives byte-identical copies of whatever was generated.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    n_ctx: int
    cap: int
    budget: int
    dtype: str            # "f32" | "bf16"
    layers: int
    seed: int
    kind: str             # "tiny" (single planted key) | "needles" | "graded"
    outlier_channels: int
    outlier_gain: float = 20.0
    sigma: float = 0.5    # lognormal sigma of the per-channel scales
    needles: int = 8      # planted needle keys per query head
    noise: float = 0.3    # standard deviation of the needle / query noise
    noise_max: float = 0.0  # > noise: needle i's noise grows geometrically up to this
    chunk: int = 0        # prefill chunk appended per step (0: none)
    score_std: float = 3.3  # "graded": std of the scores q.k/sqrt(d) over the keys
    q_outliers: bool = True   # the query shares the keys' channel scales (outlier gain too)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the path is specified on.
TINY = Workload("tiny-1h-d64-1k", 1, 1, 1, 64, 1024, 1024, 64, "f32", 1, 1001, "tiny", 2)
LLAMA2_32K = Workload("llama2-mha-32k", 1, 32, 32, 128, 32768, 32768, 256, "bf16", 1, 1002,
                      "needles", 3)
LLAMA2_128K_32L = Workload("llama2-mha-128k-32layers", 1, 32, 32, 128, 131072, 131072, 256,
                           "bf16", 32, 1003, "needles", 3)
LLAMA32_GQA_1M = Workload("llama3.2-3b-gqa-1m", 1, 24, 8, 128, 1048576, 1048576, 1024, "bf16",
                          1, 1004, "needles", 3)
BATCH16_64K = Workload("batch16-mha-64k-append4k", 16, 32, 32, 128, 65536, 65536 + 4096, 512,
                       "bf16", 1, 1005, "needles", 3, chunk=4096)

WORKLOADS = {w.name: w for w in (TINY, LLAMA2_32K, LLAMA2_128K_32L, LLAMA32_GQA_1M, BATCH16_64K)}

# Quality-sweep stand-in with graded relevance (not a benchmark workload): the
# 128K-token shape, outlier channels in K only.  With scores of standard
# deviation 3.3 over 131072 keys, the exact softmax puts about half its weight
# on the top 64 rows and about 80 % on the top 1024 (the weight of a Gaussian
# score tilts to N(3.3, 1)), so the budget has something to gain.
LLAMA2_128K_GRADED = LLAMA2_128K_32L.replace(name="llama2-mha-128k-kout-graded", kind="graded",
                                             seed=1006, q_outliers=False)
# Needles whose noise ramps from 0.3 to 3 (so a larger budget reaches more of
# them), with 6 outlier channels of gain 4 shared by queries and keys (the
# planted keys then hold most of the softmax weight, not random keys aligned
# with the outliers), or with the x20 outliers in the keys alone.
LLAMA2_128K_RAMP = LLAMA2_128K_32L.replace(name="llama2-mha-128k-needle-ramp", seed=1009,
                                           noise_max=3.0, outlier_gain=4.0, outlier_channels=6)
LLAMA2_128K_RAMP_KOUT = LLAMA2_128K_32L.replace(name="llama2-mha-128k-needle-ramp-kout",
                                                seed=1007, noise_max=3.0, q_outliers=False)
QUALITY_STANDINS = (LLAMA2_128K_32L, LLAMA2_128K_RAMP, LLAMA2_128K_RAMP_KOUT, LLAMA2_128K_GRADED)
HEADLINE_BUDGETS = (64, 128, 256, 1024)


def _np_rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _torch_gen(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    # fold the key into one 63-bit seed deterministically
    s = 0x9E3779B97F4A7C15
    for k in key:
        s = (s * 6364136223846793005 + (k & 0xFFFFFFFFFFFF) + 1442695040888963407) % (1 << 63)
    g.manual_seed(s)
    return g


def channel_scales(w: Workload, layer: int, b: int, hkv: int, tensor: int,
                   gain: bool = True) -> np.ndarray:
    """Per-channel scale vector (float32, head_dim) for one KV head and tensor
    (0=K, 1=V, 2=the graded stand-in's query); gain=False leaves the outlier
    channels unscaled."""
    r = _np_rng(w.seed, layer, b, hkv, tensor, 7)
    d = w.head_dim
    if w.kind == "tiny":
        s = np.ones(d)
    else:
        s = np.exp(w.sigma * r.standard_normal(d))
    ch = r.choice(d, size=w.outlier_channels, replace=False)
    if gain:
        s[ch] *= w.outlier_gain
    return s.astype(np.float32)


def needle_noise(w: Workload, i: int) -> float:
    """Noise level of needle i: w.noise, or a geometric ramp from w.noise to
    w.noise_max over the needles (equal expected scores, decreasing
    similarity to the query)."""
    if w.noise_max <= w.noise or w.needles < 2:
        return w.noise
    return w.noise * (w.noise_max / w.noise) ** (i / (w.needles - 1))


def needle_positions(w: Workload, layer: int, b: int, hkv: int, n_ctx: int) -> np.ndarray:
    """Distinct planted positions, shape [G][needles] (G = query heads per KV head)."""
    G = w.hq // w.hkv
    r = _np_rng(w.seed, layer, b, hkv, 11)
    per = 1 if w.kind == "tiny" else w.needles
    k = min(G * per, n_ctx) if w.kind != "graded" else 0
    pos = r.choice(n_ctx, size=k, replace=False)
    out = np.full(G * per, -1, np.int64)
    out[:k] = pos
    return out.reshape(G, per)


def make_layer(w: Workload, layer: int = 0, device="cpu", n_ctx: int | None = None,
               k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None):
    """One layer's q [B][Hq][d], k/v [B][Hkv][cap][d] in the workload's dtype.

    Rows [n_ctx, cap) are filled with draws from the same distribution (they
    are cache rows the decode step does not read).  Returns a dict with q, k,
    v and the planted needle positions [B][Hkv][G][needles].
    """
    n_ctx = w.n_ctx if n_ctx is None else n_ctx
    cap = max(w.cap, n_ctx) if n_ctx > w.n_ctx else w.cap
    B, Hq, Hkv, d = w.batch, w.hq, w.hkv, w.head_dim
    G = Hq // Hkv
    dt = w.torch_dtype
    dev = torch.device(device)
    k = k_out if k_out is not None else torch.empty((B, Hkv, cap, d), dtype=dt, device=dev)
    v = v_out if v_out is not None else torch.empty((B, Hkv, cap, d), dtype=dt, device=dev)
    assert tuple(k.shape) == (B, Hkv, cap, d) and tuple(v.shape) == (B, Hkv, cap, d)
    q = torch.empty((B, Hq, d), dtype=dt, device=dev)
    needles = np.full((B, Hkv, G, 1 if w.kind == "tiny" else w.needles), -1, np.int64)
    for b in range(B):
        for h in range(Hkv):
            sk = torch.from_numpy(channel_scales(w, layer, b, h, 0)).to(dev)
            sv = torch.from_numpy(channel_scales(w, layer, b, h, 1)).to(dev)
            g = _torch_gen(dev, w.seed, layer, b, h, 1)
            zk = torch.randn((cap, d), generator=g, device=dev, dtype=torch.float32)
            zv = torch.randn((cap, d), generator=g, device=dev, dtype=torch.float32)
            kf = zk * sk
            pos = needle_positions(w, layer, b, h, n_ctx)
            needles[b, h] = pos
            gq = _torch_gen(dev, w.seed, layer, b, h, 2)
            # a query scale vector without the outlier gain (q_outliers False)
            sq_free = torch.from_numpy(channel_scales(w, layer, b, h, 2, gain=False)).to(dev)
            for j in range(G):
                if w.kind == "tiny":
                    # q = a planted key plus N(0, noise) noise
                    p = int(pos[j, 0])
                    qf = kf[p] + w.noise * torch.randn((d,), generator=gq, device=dev)
                elif w.kind == "graded":
                    # q = kappa * (y * s_q), s_q without outlier gain; the keys'
                    # scores q.k/sqrt(d) then have standard deviation
                    # kappa * sqrt(sum_i y_i^2 s_q,i^2 s_k,i^2 / d) = score_std
                    sq = sk if w.q_outliers else sq_free
                    y = torch.randn((d,), generator=gq, device=dev) * sq
                    spread = torch.sqrt(torch.sum((y.double() * sk.double()) ** 2) / d)
                    qf = (y * (w.score_std / float(spread))).float()
                else:
                    # q = u; the needle keys are u plus scaled noise
                    u = torch.randn((d,), generator=gq, device=dev) * (
                        sk if w.q_outliers else sq_free)
                    for i, p in enumerate(pos[j]):
                        if p >= 0:
                            kf[int(p)] = u + needle_noise(w, i) * torch.randn(
                                (d,), generator=gq, device=dev) * sk
                    qf = u
                q[b, h * G + j] = qf.to(dt)
            k[b, h] = kf.to(dt)
            v[b, h] = (zv * sv).to(dt)
            del zk, zv, kf
    return {"q": q, "k": k, "v": v, "needles": needles, "n_ctx": n_ctx, "cap": cap}


def make_chunk(w: Workload, step: int, device="cpu", n: int | None = None) -> torch.Tensor:
    """A prefill chunk of keys [1][Hkv][n][d] for the batched-append workload."""
    n = w.chunk if n is None else n
    dev = torch.device(device)
    out = torch.empty((1, w.hkv, n, w.head_dim), dtype=w.torch_dtype, device=dev)
    for h in range(w.hkv):
        s = torch.from_numpy(channel_scales(w, 1000 + step, 0, h, 0)).to(dev)
        g = _torch_gen(dev, w.seed, 1000 + step, h, 3)
        out[0, h] = (torch.randn((n, w.head_dim), generator=g, device=dev) * s).to(w.torch_dtype)
    return out


def random_values(shape, dtype, seed: int, device="cpu", scale: float = 1.0) -> torch.Tensor:
    """Plain N(0, scale^2) draws in the given dtype (edge-case and property tests)."""
    g = _torch_gen(torch.device(device), seed, 99)
    return (torch.randn(shape, generator=g, device=device) * scale).to(dtype)


def integer_values(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Small integers as float32: rotations of these are exact, so they land on
    bucket thresholds and zero exactly (tie cases)."""
    return _np_rng(seed, 5).integers(lo, hi + 1, size=shape).astype(np.float32)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy for the oracle: float32 as is, bf16 as its uint16 bit pattern."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def bits_to_torch(a: np.ndarray, dtype) -> torch.Tensor:
    """Inverse of to_numpy_bits (CPU tensor)."""
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32))
