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


U32 = 2.0 ** -24   # unit roundoff of binary32


def gamma(n) -> np.ndarray:
    """gamma_n = n u / (1 - n u), the usual bound on the relative error of n
    binary32 operations in sequence."""
    n = np.asarray(n, np.float64)
    return n * U32 / (1 - n * U32)


def eval_error_bound(A: np.ndarray, S: np.ndarray, n_sel: np.ndarray, d: int) -> np.ndarray:
    """First-order bound on the error of a binary32 evaluation of softmax
    attention, per output element: each score s_j = scale * q.k_j is off by
    at most gamma_(d+4) * S (a d-term dot product, the scale, the log2(e)
    factor and the subtraction of the running maximum), which moves the
    weight p_j = exp(s_j - m) by that much relatively; weights perturbed by
    at most delta move sum_j p_j v_j / sum_j p_j by at most 2 delta A; the
    weighted sum itself adds gamma_(n + 64) A (n rows, plus the rescalings
    and merges of the partial results), and exp2 another 16 u A."""
    per_row = 2.0 * gamma(d + 4) * S + gamma(n_sel + 64) + 16 * U32     # [B][Hq]
    return per_row[..., None] * A


def check_out(ora, got: torch.Tensor, q, k, v, idx, ref_bits: np.ndarray, ref64: np.ndarray,
              what: str = "", scale: float = 0.0) -> float:
    """Compare an attention output with the oracle's, three ways:
      - the whole output: relative Frobenius error <= tol (TOL);
      - every (batch, query head) row of d elements: relative error <= tol,
        or <= the row's own evaluation bound ||ulp + E|| / ||o|| where that
        is larger (a head whose scores are hundreds of units wide cannot be
        evaluated in binary32 to 1e-5), and a row the oracle leaves zero
        (nothing selected) is zero;
      - every element: |got - o64| <= ulp(o64) + E, with o64 the oracle's
        binary64 value, ulp the output type's spacing there (one rounding to
        the output type) and E the binary32 evaluation's error bound
        (eval_error_bound, from the oracle's error scales for its selection
        idx: A = sum_j p_j |v_j| per element, S = the largest score
        magnitude per head).  E scales with A, not with |o|, which may cancel.
    Logs the maxima and how many elements differ from the oracle's rounded
    value (and by more than one ulp); returns the whole-output error."""
    dt = got.dtype
    tol = TOL[dt]
    g = got.detach().double().cpu().numpy()
    r = as_f64(ref_bits, dt)
    o64 = np.asarray(ref64, np.float64)
    A, S = ora.attend_error_scale(q, k, v, idx, scale)
    n_sel = (np.asarray(idx) >= 0).sum(axis=-1)
    d = g.shape[-1]
    frob = rel_err(got, ref_bits)
    gr, rr = g.reshape(-1, d), r.reshape(-1, d)
    num = np.linalg.norm(gr - rr, axis=1)
    den = np.linalg.norm(rr, axis=1)
    zero_rows = den == 0
    assert not np.any(np.abs(gr[zero_rows]) > 0), f"{what}: a head with nothing selected is not zero"
    per_head = np.where(zero_rows, 0.0, num / np.where(zero_rows, 1.0, den))
    bound = ulp(o64, dt) + eval_error_bound(A, S, n_sel, d)
    head_lim = np.maximum(tol, np.linalg.norm(bound.reshape(-1, d), axis=1)
                          / np.where(zero_rows, 1.0, den))
    err = np.abs(g - o64)
    n_diff = int(np.count_nonzero(g != r))
    n_over_ulp = int(np.count_nonzero(np.abs(g - r) > ulp(r, dt)))
    print(f"  {what} out: rel {frob:.2e}, worst head {per_head.max():.2e}, "
          f"{n_diff}/{g.size} elements differ from the oracle's rounding "
          f"({n_over_ulp} by more than 1 ulp), worst element at "
          f"{np.max(err / np.maximum(bound, 1e-300)):.2f} of its bound", flush=True)
    assert frob <= tol, f"{what}: whole-output relative error {frob:.3e} > {tol}"
    worst = int(np.argmax(per_head / head_lim))
    assert per_head[worst] <= head_lim[worst], (
        f"{what}: head row {worst} relative error {per_head[worst]:.3e} > "
        f"{head_lim[worst]:.3e}")
    if np.any(err > bound):
        i = np.unravel_index(int(np.argmax(err - bound)), g.shape)
        raise AssertionError(
            f"{what}: element {i} = {g[i]!r}, oracle {o64[i]!r} (bound {bound[i]:.3e}, "
            f"A {A[i]:.3e}, S {S[i[:-1]]:.3e})")
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
