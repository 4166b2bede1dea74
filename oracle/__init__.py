"""CPU oracle for the ADAMAS decode path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

The arithmetic lives in ``adamas_oracle.c`` (plain scalar C, built with gcc,
``-O2 -ffp-contract=off``, OpenMP only across independent heads).  This module
is marshalling: numpy arrays in, numpy arrays out.  Citations in the C file
refer to the ADAMAS article (www.lnwmold.com/news/826806) by section:
§2.1 Hadamard rotation, §2.2 bucketing, §2.3 Manhattan distance, §3.1 packing,
§5.2 token budget, §6 final attention.

Parity status per function (what pins it is listed in the test-suite):
  fwht / encode            pinned (closed forms, hand-worked codes)
  manhattan / score        pinned (brute force, closed-form GEMM identity)
  select_topk              pinned (exhaustive brute force on tiny inputs; with a forced
                           set: reduces to the plain selection on the other tokens)
  sparse_attend            pinned (dense attention at budget = n, budget = 1)
  decode_step              pinned by composition of the above
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adamas_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (no GPU toolchain)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.ora_fwht_f32.argtypes = [P, i32]
    lib.ora_hadamard_orthonormal_f64.argtypes = [P, P, i32]
    lib.ora_encode_vec_f32.argtypes = [P, i32, P, P, P]
    lib.ora_encode_keys.argtypes = [P, i32, i32, i32, i64, i32, P, i64, i64]
    lib.ora_manhattan.argtypes = [P, P, i32]
    lib.ora_manhattan.restype = ctypes.c_uint32
    lib.ora_score.argtypes = [P, P, i32, i32, i32, i32, i64, i64, P]
    lib.ora_select_row.argtypes = [P, i64, i32, P]
    lib.ora_select_topk.argtypes = [P, i32, i32, i64, i32, P]
    lib.ora_select_row_keep.argtypes = [P, i64, i32, i64, i64, P]
    lib.ora_select_topk_keep.argtypes = [P, i32, i32, i64, i32, i64, i64, P]
    lib.ora_decode_step_keep.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32, i64,
                                         i64, f64, P, P, P]
    lib.ora_decode_step_ex.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32, i64,
                                       i64, i32, f64, P, P, P]
    lib.ora_encode_vec_f32_rot.argtypes = [P, i32, i32, P, P, P]
    lib.ora_encode_vec_f32_ex.argtypes = [P, i32, i32, ctypes.c_float, P, P, P]
    lib.ora_encode_keys_ex.argtypes = [P, i32, i32, i32, i64, i32, P, i64, i64, i32, P, i32]
    lib.ora_decode_step_alpha.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32,
                                          i64, i64, i32, P, i32, f64, P, P, P]
    lib.ora_encode_keys_rot.argtypes = [P, i32, i32, i32, i64, i32, P, i64, i64, i32]
    lib.ora_sparse_attend.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i64, i32, f64, P, P]
    lib.ora_sparse_attend_ex.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i64, i32, f64, P,
                                         P, P, P]
    lib.ora_decode_step.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32, f64, P, P, P]
    lib.ora_f64_to_f16_value.argtypes = [f64]
    lib.ora_f64_to_f16_value.restype = ctypes.c_float
    lib.ora_f64_to_bf16.argtypes = [f64]
    lib.ora_f64_to_bf16.restype = ctypes.c_uint16
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_tag(a: np.ndarray) -> int:
    """fp32 arrays are float32; bf16 arrays are carried as uint16 bit patterns."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


# ---------------------------------------------------------------- rotation
def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Sylvester-order FWHT of one vector, binary32 (§2.1)."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    _load().ora_fwht_f32(_ptr(y), y.shape[-1])
    return y


def hadamard_orthonormal_f64(x: np.ndarray) -> np.ndarray:
    """H x / sqrt(d) in binary64 (§2.1's orthonormal rotation)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().ora_hadamard_orthonormal_f64(_ptr(x), _ptr(y), x.shape[-1])
    return y


def _alpha_table(alpha):
    """None -> (null, 0); a sequence of per-head-group bucketing fractions -> float32 array."""
    if alpha is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(alpha, np.float32).reshape(-1))
    assert a.size >= 1
    return a, int(a.size)


def encode_vec(x: np.ndarray, rotate: int = True, alpha: float | None = None):
    """One fp32 vector -> (packed bytes, rotated values, codes); rotate=False
    buckets the vector as it is, rotate=2 rotates in binary16; alpha (default
    0.5) places the outer thresholds at -alpha*a and +alpha*a."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    packed = np.empty(d // 4, np.uint8)
    y = np.empty(d, np.float32)
    codes = np.empty(d, np.int32)
    if alpha is not None:
        _load().ora_encode_vec_f32_ex(_ptr(x), d, int(rotate), float(alpha), _ptr(packed), _ptr(y),
                                      _ptr(codes))
    elif rotate is True or rotate == 1:
        _load().ora_encode_vec_f32(_ptr(x), d, _ptr(packed), _ptr(y), _ptr(codes))
    else:
        _load().ora_encode_vec_f32_rot(_ptr(x), d, int(rotate), _ptr(packed), _ptr(y),
                                       _ptr(codes))
    return packed, y, codes


def f64_to_f16_value(x: float) -> float:
    """Correctly rounded binary64 -> binary16, as a float."""
    return float(_load().ora_f64_to_f16_value(float(x)))


def encode_keys(x: np.ndarray, codes: np.ndarray | None = None, cap: int | None = None,
                pos: int = 0, rotate: bool = True, alpha=None) -> np.ndarray:
    """x[batch][heads][n][d] -> codes[batch][heads][cap][d/4], rows [pos, pos+n).
    alpha: per-head bucketing fractions, head h uses alpha[h % len(alpha)]."""
    x = np.ascontiguousarray(x)
    batch, heads, n, d = x.shape
    if cap is None:
        cap = pos + n
    if codes is None:
        codes = np.zeros((batch, heads, cap, d // 4), np.uint8)
    assert codes.shape == (batch, heads, cap, d // 4) and codes.dtype == np.uint8
    if alpha is not None:
        a, na = _alpha_table(alpha)
        _load().ora_encode_keys_ex(_ptr(x), _dtype_tag(x), batch, heads, n, d, _ptr(codes), cap,
                                   pos, int(rotate), _ptr(a), na)
    elif rotate is True or rotate == 1:
        _load().ora_encode_keys(_ptr(x), _dtype_tag(x), batch, heads, n, d, _ptr(codes), cap, pos)
    else:
        _load().ora_encode_keys_rot(_ptr(x), _dtype_tag(x), batch, heads, n, d, _ptr(codes), cap,
                                    pos, int(rotate))
    return codes


# ---------------------------------------------------------------- scoring
def manhattan(qrow: np.ndarray, krow: np.ndarray, d: int) -> int:
    return int(_load().ora_manhattan(_ptr(np.ascontiguousarray(qrow, np.uint8)),
                                     _ptr(np.ascontiguousarray(krow, np.uint8)), d))


def score(q_codes: np.ndarray, k_codes: np.ndarray, n_ctx: int | None = None) -> np.ndarray:
    """q_codes[B][Hq][d/4], k_codes[B][Hkv][cap][d/4] -> dist[B][Hq][n_ctx] (uint16)."""
    B, Hq, rb = q_codes.shape
    _, Hkv, cap, rb2 = k_codes.shape
    assert rb == rb2
    if n_ctx is None:
        n_ctx = cap
    dist = np.empty((B, Hq, n_ctx), np.uint16)
    _load().ora_score(_ptr(np.ascontiguousarray(q_codes)), _ptr(np.ascontiguousarray(k_codes)),
                      B, Hq, Hkv, rb * 4, cap, n_ctx, _ptr(dist))
    return dist


def select_topk(dist: np.ndarray, budget: int, n_sink: int = 0, n_recent: int = 0) -> np.ndarray:
    """dist[B][Hq][n] -> idx[B][Hq][budget] int32, ascending, -1 padded (§5.2);
    the first n_sink and last n_recent tokens rank ahead of all others."""
    dist = np.ascontiguousarray(dist, np.uint16)
    B, Hq, n = dist.shape
    idx = np.empty((B, Hq, budget), np.int32)
    if n_sink == 0 and n_recent == 0:
        _load().ora_select_topk(_ptr(dist), B, Hq, n, budget, _ptr(idx))
    else:
        _load().ora_select_topk_keep(_ptr(dist), B, Hq, n, budget, n_sink, n_recent, _ptr(idx))
    return idx


# ---------------------------------------------------------------- attention
def sparse_attend(q, k, v, idx, scale: float = 0.0):
    """q[B][Hq][d], k/v[B][Hkv][cap][d], idx[B][Hq][budget] -> (out, out64)."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    idx = np.ascontiguousarray(idx, np.int32)
    dt = _dtype_tag(q)
    assert _dtype_tag(k) == dt and _dtype_tag(v) == dt
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    budget = idx.shape[-1]
    out = np.empty((B, Hq, d), q.dtype)
    out64 = np.empty((B, Hq, d), np.float64)
    _load().ora_sparse_attend(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(idx), B, Hq, Hkv, d, cap,
                              budget, float(scale), _ptr(out), _ptr(out64))
    return out, out64


def attend_error_scale(q, k, v, idx, scale: float = 0.0):
    """Error scales of a floating-point evaluation of sparse_attend (test
    tolerances; not part of the result), in binary64 -> (A, S):
    A [B][Hq][d] per output element sum_j p_j |v_j,i|, and S [B][Hq] the
    largest score magnitude |scale| * sum_i |q_i k_j,i| over the selected rows."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    idx = np.ascontiguousarray(idx, np.int32)
    dt = _dtype_tag(q)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    out = np.empty((B, Hq, d), q.dtype)
    out64 = np.empty((B, Hq, d), np.float64)
    am = np.empty((B, Hq, d), np.float64)
    sm = np.empty((B, Hq), np.float64)
    _load().ora_sparse_attend_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(idx), B, Hq, Hkv, d, cap,
                                 idx.shape[-1], float(scale), _ptr(out), _ptr(out64), _ptr(am),
                                 _ptr(sm))
    return am, sm


def decode_step(q, k, v, k_codes, n_ctx: int, budget: int, scale: float = 0.0,
                n_sink: int = 0, n_recent: int = 0, rotate: bool = True, alpha=None):
    """Full step for one layer -> (out, out64, idx).  alpha: the per-KV-head
    bucketing table the keys were encoded with (query head hq uses its KV
    head's entry)."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    k_codes = np.ascontiguousarray(k_codes, np.uint8)
    dt = _dtype_tag(q)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    out = np.empty((B, Hq, d), q.dtype)
    out64 = np.empty((B, Hq, d), np.float64)
    idx = np.empty((B, Hq, budget), np.int32)
    if alpha is not None:
        a, na = _alpha_table(alpha)
        _load().ora_decode_step_alpha(_ptr(q), _ptr(k), _ptr(v), _ptr(k_codes), dt, B, Hq, Hkv, d,
                                      cap, n_ctx, budget, n_sink, n_recent, int(rotate), _ptr(a),
                                      na, float(scale), _ptr(out), _ptr(out64), _ptr(idx))
    elif not (rotate is True or rotate == 1):
        _load().ora_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(k_codes), dt, B, Hq, Hkv, d,
                                   cap, n_ctx, budget, n_sink, n_recent, int(rotate),
                                   float(scale), _ptr(out), _ptr(out64), _ptr(idx))
    elif n_sink == 0 and n_recent == 0:
        _load().ora_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(k_codes), dt, B, Hq, Hkv, d, cap,
                                n_ctx, budget, float(scale), _ptr(out), _ptr(out64), _ptr(idx))
    else:
        _load().ora_decode_step_keep(_ptr(q), _ptr(k), _ptr(v), _ptr(k_codes), dt, B, Hq, Hkv, d,
                                     cap, n_ctx, budget, n_sink, n_recent, float(scale),
                                     _ptr(out), _ptr(out64), _ptr(idx))
    return out, out64, idx


def decode_append_step(q, k, v, k_codes, lens, max_len: int, budget: int, k_new=None,
                       v_new=None, scale: float = 0.0, n_sink: int = 0, n_recent: int = 0,
                       rotate: bool = True, alpha=None):
    """A decode step over sequences of their own lengths, each first taking the
    step's new key and value at its next row (the compressed cache of §3.1
    stores each new token's code at its position; the step itself is §2-§6 on
    that sequence's rows).  Works on copies -> (out, out64, idx, k, v, k_codes)
    with the caches as the step leaves them.

    Sequence b holds L_b = lens[b] rows, clamped to [0, max_len - 1] when a
    token is appended and to [0, max_len] otherwise; it is decoded on its own
    with n_ctx = L_b (+1 with the new token), so its recent window ends at its
    own last row.  No rows: a zero output and an all -1 selection.  alpha: the
    per-KV-head bucketing table (the new key of KV head h buckets with
    alpha[h % len(alpha)], as the cache's codes were made)."""
    k, v, k_codes = (np.array(a, copy=True) for a in (k, v, k_codes))
    B, Hq, d = q.shape
    app = k_new is not None
    out = np.zeros((B, Hq, d), q.dtype)
    out64 = np.zeros((B, Hq, d), np.float64)
    idx = np.full((B, Hq, budget), -1, np.int32)
    for b in range(B):
        L = min(max(int(lens[b]), 0), max_len - (1 if app else 0))
        if app:
            k[b, :, L] = k_new[b]
            v[b, :, L] = v_new[b]
            row = encode_keys(np.ascontiguousarray(k_new[b][None, :, None, :]), rotate=rotate,
                              alpha=alpha)
            k_codes[b, :, L] = row[0, :, 0]
        n = L + (1 if app else 0)
        if n == 0:
            continue
        o, o64, ix = decode_step(q[b:b + 1], k[b:b + 1], v[b:b + 1], k_codes[b:b + 1], n, budget,
                                 scale, n_sink, n_recent, rotate, alpha)
        out[b], out64[b], idx[b] = o[0], o64[0], ix[0]
    return out, out64, idx, k, v, k_codes


def decode_paged_step(q, k_pool, v_pool, code_pool, page_table, lens, max_len: int, budget: int,
                      k_new=None, v_new=None, scale: float = 0.0, n_sink: int = 0,
                      n_recent: int = 0, rotate: bool = True, alpha=None):
    """decode_append_step over paged pools (the §3.1 cache kept in fixed-size
    chunks): pool page p holds tokens of every KV head, k_pool[p][h][j] is
    token j of the page; sequence b's logical page i is pool page
    page_table[b][i].  Each sequence's cache is gathered into one contiguous
    array, stepped as decode_append_step does, and its new row (if any) put
    back into copies of the pools -> (out, out64, idx, k_pool, v_pool, code_pool)."""
    k_pool, v_pool, code_pool = (np.array(a, copy=True) for a in (k_pool, v_pool, code_pool))
    B = q.shape[0]
    n_pages, Hkv, P, d = k_pool.shape
    max_pages = page_table.shape[1]
    outs, out64s, idxs = [], [], []
    for b in range(B):
        pages = [int(x) for x in page_table[b]]
        # only the pages the sequence reaches are looked up
        need = (min(max(int(lens[b]), 0), max_len - (1 if k_new is not None else 0))
                + (1 if k_new is not None else 0) + P - 1) // P
        ids = [pages[i] if i < need else 0 for i in range(max_pages)]
        gather = lambda pool: np.ascontiguousarray(
            np.concatenate([pool[i] for i in ids], axis=1)[None])   # [1][Hkv][max_pages*P][...]
        kb, vb, cb = gather(k_pool), gather(v_pool), gather(code_pool)
        o, o64, ix, k2, v2, c2 = decode_append_step(
            q[b:b + 1], kb, vb, cb, np.asarray(lens)[b:b + 1], max_len, budget,
            None if k_new is None else k_new[b:b + 1], None if v_new is None else v_new[b:b + 1],
            scale, n_sink, n_recent, rotate, alpha)
        if k_new is not None:
            L = min(max(int(lens[b]), 0), max_len - 1)
            pg, off = ids[L // P], L % P
            k_pool[pg][:, off] = k2[0][:, L]
            v_pool[pg][:, off] = v2[0][:, L]
            code_pool[pg][:, off] = c2[0][:, L]
        outs.append(o[0]); out64s.append(o64[0]); idxs.append(ix[0])
    return np.stack(outs), np.stack(out64s), np.stack(idxs), k_pool, v_pool, code_pool


def f64_to_bf16_bits(x: float) -> int:
    return int(_load().ora_f64_to_bf16(float(x)))
