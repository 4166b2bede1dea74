"""Shared helpers for the GPU parity tests (comparison against the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import synth

# Output tolerances (relative error), the bound the method's target states
# for attention outputs: 2e-3 for bfloat16, 1e-5 for binary32.
TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def host(t: torch.Tensor) -> np.ndarray:
    return synth.to_numpy_bits(t)


def as_f64(bits: np.ndarray, dtype) -> np.ndarray:
    return synth.bits_to_torch(bits, dtype).double().numpy()


def rel_err(got: torch.Tensor, ref_bits: np.ndarray) -> float:
    """Relative Frobenius error of a whole output against the oracle's result
    rounded to the output type."""
    g = got.detach().double().cpu().numpy()
    r = as_f64(ref_bits, got.dtype)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g))


def ulp(x64: np.ndarray, dtype) -> np.ndarray:
    """Spacing of the output type at |x| (bfloat16: 8 significant bits and
    subnormal spacing 2^-133; binary32: 24 bits, subnormal spacing 2^-149)."""
    a = np.abs(np.asarray(x64, np.float64))
    if dtype == torch.float32:
        mant_bits, min_exp = 24, -126
    else:
        mant_bits, min_exp = 8, -126
    _, e = np.frexp(a)                    # a = m * 2^e, m in [0.5, 1)
    # exponent of the leading bit, clamped to the subnormal range (and for 0)
    e = np.where(a == 0, min_exp, np.maximum(e - 1, min_exp))
    return np.ldexp(1.0, e - (mant_bits - 1))


def check_out(ora, got: torch.Tensor, q, k, v, idx, ref_bits: np.ndarray, ref64: np.ndarray,
              what: str = "", scale: float = 0.0) -> float:
    """Compare an attention output with the oracle's, three ways, each within
    the type's tolerance tol (TOL):
      - the whole output: relative Frobenius error <= tol;
      - every (batch, query head) row of d elements: relative error <= tol,
        and a row the oracle leaves zero (nothing selected) is zero;
      - every element: |got - o64| <= ulp(o64) + tol * A, with o64 the
        oracle's binary64 value, ulp the output type's spacing there and
        A = sum_j p_j |v_j| over the same element's terms (the oracle's
        attend_error_scale for the oracle's selection idx): one rounding to the
        output type, plus the binary32 evaluation's error, which scales with
        A and not with |o| (o may cancel).
    Logs the three maxima and how many elements differ from the oracle's
    rounded value; returns the whole-output error."""
    dt = got.dtype
    tol = TOL[dt]
    g = got.detach().double().cpu().numpy()
    r = as_f64(ref_bits, dt)
    o64 = np.asarray(ref64, np.float64)
    A = ora.attend_error_scale(q, k, v, idx, scale)
    d = g.shape[-1]
    frob = rel_err(got, ref_bits)
    gr, rr = g.reshape(-1, d), r.reshape(-1, d)
    num = np.linalg.norm(gr - rr, axis=1)
    den = np.linalg.norm(rr, axis=1)
    zero_rows = den == 0
    assert not np.any(np.abs(gr[zero_rows]) > 0), f"{what}: a head with nothing selected is not zero"
    per_head = np.where(zero_rows, 0.0, num / np.where(zero_rows, 1.0, den))
    bound = ulp(o64, dt) + tol * A
    excess = np.abs(g - o64) - bound
    n_diff = int(np.count_nonzero(g != r))
    n_over_ulp = int(np.count_nonzero(np.abs(g - r) > ulp(r, dt)))
    print(f"  {what} out: rel {frob:.2e}, worst head {per_head.max():.2e}, "
          f"{n_diff}/{g.size} elements differ from the oracle's rounding "
          f"({n_over_ulp} by more than 1 ulp), worst element {np.max(excess):.2e} vs its bound",
          flush=True)
    assert frob <= tol, f"{what}: whole-output relative error {frob:.3e} > {tol}"
    worst = int(np.argmax(per_head))
    assert per_head[worst] <= tol, (
        f"{what}: head row {worst} relative error {per_head[worst]:.3e} > {tol}")
    if np.any(excess > 0):
        i = np.unravel_index(int(np.argmax(excess)), g.shape)
        raise AssertionError(
            f"{what}: element {i} = {g[i]!r}, oracle {o64[i]!r} (bound {bound[i]:.3e}, "
            f"error scale {A[i]:.3e})")
    return frob


def pages_to_rows(pool: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Sequence-major rows of a paged pool [n_pages][Hkv][P][...] through a
    page table [B][max_pages] (entries clamped into the pool, as the library
    clamps them) -> [B][Hkv][max_pages * P][...]."""
    t = np.clip(np.asarray(table), 0, pool.shape[0] - 1)
    return np.ascontiguousarray(np.concatenate([pool[t[:, i]] for i in range(t.shape[1])], axis=2))


def check_out_paged(ora, got, q, k_pool, v_pool, table, idx, ref_bits, ref64, what=""):
    """check_out for a paged step: the error scale is taken over each
    sequence's rows gathered through its page table."""
    return check_out(ora, got, q, pages_to_rows(k_pool, table), pages_to_rows(v_pool, table),
                     idx, ref_bits, ref64, what)


def log(msg: str):
    print(msg, flush=True)
