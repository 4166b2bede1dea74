"""Shared helpers for the GPU parity tests (comparison against the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import synth

# Output tolerances: relative Frobenius error of one call's whole output
# against the oracle's binary64 result rounded to the output type.
TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def host(t: torch.Tensor) -> np.ndarray:
    return synth.to_numpy_bits(t)


def as_f64(bits: np.ndarray, dtype) -> np.ndarray:
    return synth.bits_to_torch(bits, dtype).double().numpy()


def rel_err(got: torch.Tensor, ref_bits: np.ndarray) -> float:
    g = got.detach().double().cpu().numpy()
    r = as_f64(ref_bits, got.dtype)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g))


def log(msg: str):
    print(msg, flush=True)
