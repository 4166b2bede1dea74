"""Python binding of libadamas.so, the MI355X (gfx950) ADAMAS decode path.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and their device pointers, together with torch's current HIP
stream, are handed to the C ABI declared in include/adamas.h.  Every step of
the path runs in the library's HIP kernels; there is no fallback.  If the
library is not built, every call raises.

Method (ADAMAS article, www.lnwmold.com/news/826806): Hadamard rotation
(§2.1), 2-bit bucketing (§2.2), packed code cache (§3.1), Manhattan scoring
(§2.3), per-head token budget (§5.2), exact attention over the kept rows (§6).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "AdamasError", "load", "library_path", "encode_keys", "encode_query", "score", "select_topk",
    "sparse_attend", "decode_step", "decode_append_step", "decode_paged_step", "workspace_bytes",
    "Workspace",
    "set_decode_mode", "decode_path", "set_rotation", "stream_read", "OP_SELECT_TOPK",
    "OP_SPARSE_ATTEND", "OP_DECODE_STEP", "DECODE_AUTO", "DECODE_LAST_ARRIVAL",
    "DECODE_GROUP_WAIT", "DECODE_SPLIT", "WS_CTRL_BYTES", "WS_STATUS_OFFSET", "ROTATE_OFF",
    "ROTATE_F32", "ROTATE_F16", "GroupWaitGaveUp", "set_wait_polls", "wait_polls",
    "DEFAULT_WAIT_POLLS", "PhaseRecorder", "decode_step_static", "STATIC_SCRATCH_BYTES",
    "set_bucket_alpha", "bucket_alpha", "MAX_ALPHA_GROUPS", "decode_key_bytes",
    "decode_chunk_tokens",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libadamas.so")
# the same library built with the phase timestamps compiled in (measurement only)
_VARIANTS = {None: None, "phases": os.path.join(_HERE, "libadamas_phases.so")}

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = range(5)
F32, BF16 = 0, 1
OP_SELECT_TOPK, OP_SPARSE_ATTEND, OP_DECODE_STEP = 0, 1, 2
WS_CTRL_BYTES = 65792          # ADAMAS_WS_CTRL_BYTES
WS_STATUS_OFFSET = 65536       # ADAMAS_WS_STATUS_OFFSET
DECODE_AUTO, DECODE_LAST_ARRIVAL, DECODE_GROUP_WAIT, DECODE_SPLIT = 0, 1, 2, 3
DEFAULT_WAIT_POLLS = 1 << 20   # the library's initial group-wait bound

_lib = None


class AdamasError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = load().adamas_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


class GroupWaitGaveUp(RuntimeError):
    """A group-wait decode step gave up waiting (workspace status word set):
    the outputs of that call are invalid."""


def library_path() -> str:
    return _LIB_PATH


_variant = None


def load(variant: str | None = None):
    """dlopen libadamas.so (raises if it has not been built).  variant="phases"
    loads the measurement build with phase timestamps instead; it must be the
    first load of the process."""
    global _lib, _variant
    if variant not in _VARIANTS:
        raise ValueError(f"unknown library variant {variant!r}")
    if _lib is not None:
        if variant is not None and variant != _variant:
            raise RuntimeError(f"library already loaded as variant {_variant!r}")
        return _lib
    path = _LIB_PATH if variant is None else _VARIANTS[variant]
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
            "g.build()'` (hipcc --offload-arch=gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    _variant = variant
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.adamas_encode_keys.argtypes = [P, i32, i32, i32, i64, i32, P, i64, i64, P, P]
    lib.adamas_encode_keys_paged.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, i32, i32,
                                             i32, i64, P]
    lib.adamas_score.argtypes = [P, P, i32, i32, i32, i32, i64, i64, P, P]
    lib.adamas_select_topk.argtypes = [P, i32, i32, i64, i32, i32, P, P, sz, P]
    lib.adamas_sparse_attend.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i64, i32, f32, P, P,
                                         sz, P]
    lib.adamas_decode_step.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32, f32, P,
                                       P, P, sz, P]
    lib.adamas_select_topk_keep.argtypes = [P, i32, i32, i64, i32, i32, i32, i32, P, P, sz, P]
    lib.adamas_decode_step_keep.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32,
                                            i32, i32, f32, P, P, P, sz, P]
    lib.adamas_decode_append_step.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i64,
                                              i64, i32, i32, i32, f32, P, P, P, sz, P]
    lib.adamas_decode_paged_step.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                             i32, i32, i64, i32, i32, i32, f32, P, P, P, sz, P]
    lib.adamas_workspace_bytes.argtypes = [i32, i32, i32, i32, i64, i32, i32]
    lib.adamas_workspace_bytes.restype = sz
    lib.adamas_status_string.argtypes = [i32]
    lib.adamas_status_string.restype = ctypes.c_char_p
    lib.adamas_version.restype = i32
    lib.adamas_stream_read.argtypes = [P, sz, P, P]
    lib.adamas_stream_read.restype = i32
    lib.adamas_stream_read_blocks.argtypes = [sz]
    lib.adamas_stream_read_blocks.restype = sz
    lib.adamas_set_decode_mode.argtypes = [i32]
    lib.adamas_set_rotation.argtypes = [i32]
    lib.adamas_set_rotation.restype = i32
    lib.adamas_set_bucket_alpha.argtypes = [P, i32]
    lib.adamas_set_bucket_alpha.restype = i32
    lib.adamas_bucket_alpha.argtypes = [P, i32]
    lib.adamas_bucket_alpha.restype = i32
    lib.adamas_decode_path.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.adamas_decode_key_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.adamas_decode_chunk_tokens.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.adamas_set_wait_polls.argtypes = [ctypes.c_uint32]
    lib.adamas_set_wait_polls.restype = i32
    lib.adamas_decode_step_static.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64, i64, i32,
                                              f32, P, P, P]
    lib.adamas_decode_step_static.restype = i32
    lib.adamas_static_scratch_need.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.adamas_static_scratch_need.restype = sz
    lib.adamas_wait_polls.argtypes = []
    lib.adamas_wait_polls.restype = ctypes.c_uint32
    lib.adamas_phase_stamps_built.restype = i32
    lib.adamas_phase_buffer_bytes.restype = sz
    lib.adamas_set_phase_buffer.argtypes = [P, sz]
    lib.adamas_set_phase_buffer.restype = i32
    lib.adamas_wall_clock_khz.restype = i32
    for fn in ("adamas_set_decode_mode", "adamas_decode_path"):
        getattr(lib, fn).restype = i32
    for fn in ("adamas_encode_keys", "adamas_encode_keys_paged", "adamas_score", "adamas_select_topk", "adamas_sparse_attend",
               "adamas_decode_step", "adamas_select_topk_keep", "adamas_decode_step_keep",
               "adamas_decode_append_step", "adamas_decode_paged_step"):
        getattr(lib, fn).restype = i32
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != OK:
        raise AdamasError(status, what)


def _dev_ptr(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)")


def workspace_bytes(op: int, B: int, Hq: int, Hkv: int, n_ctx: int, budget: int,
                    head_dim: int) -> int:
    n = load().adamas_workspace_bytes(op, B, Hq, Hkv, n_ctx, budget, head_dim)
    if n == 0:
        raise AdamasError(ERR_INVALID, "adamas_workspace_bytes")
    return int(n)


class Workspace:
    """A zero-initialised device workspace reused across calls on one stream.

    The library leaves its control bytes zero after every call, so the buffer
    only grows (re-zeroed on growth) and is never cleared between calls."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = torch.zeros(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, WS_CTRL_BYTES), dtype=torch.uint8,
                                   device=self.device)
        return self.buf

    def status(self) -> int:
        """The workspace status word (ADAMAS_WS_STATUS_OFFSET), read after the work
        enqueued so far on the current stream: nonzero once a group wait gave up
        (that call's outputs are invalid).  The library never clears it."""
        if self.buf.numel() < WS_CTRL_BYTES:
            return 0
        word = self.buf[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 4]
        return int(word.view(torch.int32).item())

    def reset_status(self) -> None:
        """Re-arm the status word (enqueued on the current stream)."""
        if self.buf.numel() >= WS_CTRL_BYTES:
            self.buf[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 4].zero_()

    def check(self) -> None:
        """Raise GroupWaitGaveUp (and re-arm the word) if a call on this
        workspace gave up a group wait since the last check."""
        st = self.status()
        if st != 0:
            self.reset_status()
            raise GroupWaitGaveUp(
                f"a group-wait decode step gave up waiting (status word {st:#x}); "
                "outputs since the last check are invalid")

    def control_bytes_clear(self) -> bool:
        """True when the arrival counters (the control bytes other than the
        status word) are all zero, as every completed call leaves them."""
        if self.buf.numel() < WS_CTRL_BYTES:
            return True
        ctrl = self.buf[:WS_CTRL_BYTES].clone()
        ctrl[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 4] = 0
        return bool((ctrl == 0).all().item())


_default_ws: dict = {}


def _ws_for(device, ws: Workspace | None) -> Workspace:
    if ws is not None:
        return ws
    key = (torch.device(device), torch.cuda.current_stream(device).cuda_stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


# ------------------------------------------------------------------ calls
def encode_keys(x: torch.Tensor, codes: torch.Tensor, pos: int = 0,
                x_copy: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x [batch][heads][n][d] -> codes [batch][heads][cap][d/4] rows [pos, pos+n)."""
    if x.dim() != 4 or codes.dim() != 4 or codes.dtype != torch.uint8:
        raise ValueError("x must be [batch][heads][n][d] and codes uint8 [batch][heads][cap][d/4]")
    batch, heads, n, d = x.shape
    cap = codes.shape[2]
    if tuple(codes.shape) != (batch, heads, cap, d // 4):
        raise ValueError(f"codes shape {tuple(codes.shape)} does not match x {tuple(x.shape)}")
    if x_copy is not None and (tuple(x_copy.shape) != (batch, heads, cap, d) or
                               x_copy.dtype != x.dtype):
        raise ValueError("x_copy must be [batch][heads][cap][d] of x's dtype")
    st = load().adamas_encode_keys(_dev_ptr(x, "x"), _dtype_code(x), batch, heads, n, d,
                                   _dev_ptr(codes, "codes"), cap, pos, _dev_ptr(x_copy, "x_copy"),
                                   _stream(x, stream))
    _check(st, "adamas_encode_keys")
    return codes


def encode_keys_paged(x: torch.Tensor, code_pool: torch.Tensor, page_table: torch.Tensor,
                      pos: int = 0, x_pool: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """x [batch][heads][n][d] (tokens [pos, pos+n) of each sequence) -> the code
    rows in code_pool [n_pages][heads][page][d/4] that page_table [batch][max_pages]
    maps them to (adamas_encode_keys_paged); x_pool: optional raw-row pool."""
    if x.dim() != 4 or code_pool.dim() != 4 or code_pool.dtype != torch.uint8:
        raise ValueError("x must be [batch][heads][n][d] and code_pool uint8 "
                         "[n_pages][heads][page][d/4]")
    batch, heads, n, d = x.shape
    n_pages, page = code_pool.shape[0], code_pool.shape[2]
    if tuple(code_pool.shape) != (n_pages, heads, page, d // 4):
        raise ValueError(f"code_pool shape {tuple(code_pool.shape)} does not match x "
                         f"{tuple(x.shape)}")
    if (page_table.dim() != 2 or page_table.shape[0] != batch or
            page_table.dtype != torch.int32):
        raise ValueError("page_table must be int32 [batch][max_pages]")
    if x_pool is not None and (tuple(x_pool.shape) != (n_pages, heads, page, d) or
                               x_pool.dtype != x.dtype):
        raise ValueError("x_pool must be [n_pages][heads][page][d] of x's dtype")
    st = load().adamas_encode_keys_paged(
        _dev_ptr(x, "x"), _dtype_code(x), batch, heads, n, d, _dev_ptr(code_pool, "code_pool"),
        _dev_ptr(x_pool, "x_pool"), _dev_ptr(page_table, "page_table"), page, n_pages,
        page_table.shape[1], pos, _stream(x, stream))
    _check(st, "adamas_encode_keys_paged")
    return code_pool


def encode_query(q: torch.Tensor, stream=None) -> torch.Tensor:
    """q [B][Hq][d] -> q_codes [B][Hq][d/4] (encode_keys with n = cap = 1)."""
    B, Hq, d = q.shape
    codes = torch.empty((B, Hq, 1, d // 4), dtype=torch.uint8, device=q.device)
    encode_keys(q.reshape(B, Hq, 1, d), codes, 0, None, stream)
    return codes.reshape(B, Hq, d // 4)


def score(q_codes: torch.Tensor, k_codes: torch.Tensor, n_ctx: int | None = None,
          dist: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """-> dist [B][Hq][n_ctx] uint16 (returned as torch.uint16)."""
    B, Hq, rb = q_codes.shape
    _, Hkv, cap, rb2 = k_codes.shape
    if rb != rb2 or q_codes.dtype != torch.uint8 or k_codes.dtype != torch.uint8:
        raise ValueError("q_codes / k_codes must be uint8 with matching row bytes")
    n_ctx = cap if n_ctx is None else n_ctx
    if dist is None:
        dist = torch.empty((B, Hq, n_ctx), dtype=torch.uint16, device=q_codes.device)
    st = load().adamas_score(_dev_ptr(q_codes, "q_codes"), _dev_ptr(k_codes, "k_codes"), B, Hq, Hkv,
                             rb * 4, cap, n_ctx, _dev_ptr(dist, "dist"), _stream(q_codes, stream))
    _check(st, "adamas_score")
    return dist


def select_topk(dist: torch.Tensor, budget: int, head_dim: int, idx: torch.Tensor | None = None,
                ws: Workspace | None = None, stream=None, n_sink: int = 0,
                n_recent: int = 0) -> torch.Tensor:
    """dist [B][Hq][n] uint16 -> idx [B][Hq][budget] int32 (ascending, -1 padded).
    The first n_sink and last n_recent tokens are always kept (adamas_select_topk_keep)."""
    B, Hq, n = dist.shape
    if idx is None:
        idx = torch.empty((B, Hq, budget), dtype=torch.int32, device=dist.device)
    nb = load().adamas_workspace_bytes(OP_SELECT_TOPK, B, Hq, 1, n, budget, head_dim)
    buf = _ws_for(dist.device, ws).get(nb)
    args = (_dev_ptr(dist, "dist"), B, Hq, n, head_dim, budget)
    tail = (_dev_ptr(idx, "idx"), _dev_ptr(buf, "ws"), buf.numel(), _stream(dist, stream))
    if n_sink == 0 and n_recent == 0:
        st = load().adamas_select_topk(*args, *tail)
    else:
        st = load().adamas_select_topk_keep(*args, int(n_sink), int(n_recent), *tail)
    _check(st, "adamas_select_topk")
    return idx


def sparse_attend(q, k, v, idx, scale: float = 0.0, out=None, ws: Workspace | None = None,
                  stream=None) -> torch.Tensor:
    """q [B][Hq][d], k/v [B][Hkv][cap][d], idx [B][Hq][budget] -> out [B][Hq][d]."""
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    budget = idx.shape[-1]
    if k.dtype != q.dtype or v.dtype != q.dtype or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v must share dtype; k and v share shape")
    if out is None:
        out = torch.empty_like(q)
    nb = load().adamas_workspace_bytes(OP_SPARSE_ATTEND, B, Hq, Hkv, 1, budget, d)
    buf = _ws_for(q.device, ws).get(nb)
    st = load().adamas_sparse_attend(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                     _dtype_code(q), _dev_ptr(idx, "idx"), B, Hq, Hkv, d, cap,
                                     budget, float(scale), _dev_ptr(out, "out"),
                                     _dev_ptr(buf, "ws"), buf.numel(), _stream(q, stream))
    _check(st, "adamas_sparse_attend")
    return out


def stream_read(x: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Reference streaming read of x's bytes (adamas_stream_read); returns the sink."""
    nbytes = x.numel() * x.element_size()
    nblk = int(load().adamas_stream_read_blocks(nbytes))
    if sink is None:
        sink = torch.empty(nblk, dtype=torch.int32, device=x.device)
    _check(load().adamas_stream_read(_dev_ptr(x, "x"), nbytes, _dev_ptr(sink, "sink"),
                                     _stream(x, stream)), "adamas_stream_read")
    return sink


ROTATE_OFF, ROTATE_F32, ROTATE_F16 = 0, 1, 2


def set_rotation(on) -> None:
    """Process-wide: rotate vectors before bucketing in binary32 (True / ROTATE_F32, the
    default), not at all (False / ROTATE_OFF) or in binary16 (ROTATE_F16)
    (adamas_set_rotation)."""
    mode = int(on) if not isinstance(on, bool) else (1 if on else 0)
    _check(load().adamas_set_rotation(mode), "adamas_set_rotation")


MAX_ALPHA_GROUPS = 64


def set_bucket_alpha(alpha=None) -> None:
    """Process-wide per-head-group bucketing thresholds (adamas_set_bucket_alpha):
    KV head h (and its query heads) buckets at -alpha[h % n]*a, 0 and
    +alpha[h % n]*a; None or an empty sequence restores the fixed rule
    (alpha 0.5)."""
    if alpha is None:
        _check(load().adamas_set_bucket_alpha(None, 0), "adamas_set_bucket_alpha")
        return
    a = (ctypes.c_float * MAX_ALPHA_GROUPS)()
    vals = [float(x) for x in alpha]
    if len(vals) > MAX_ALPHA_GROUPS:
        raise ValueError(f"at most {MAX_ALPHA_GROUPS} alpha groups")
    for i, x in enumerate(vals):
        a[i] = x
    _check(load().adamas_set_bucket_alpha(a, len(vals)), "adamas_set_bucket_alpha")


def bucket_alpha() -> list:
    """The current table (empty: the fixed rule, alpha 0.5)."""
    a = (ctypes.c_float * MAX_ALPHA_GROUPS)()
    n = load().adamas_bucket_alpha(a, MAX_ALPHA_GROUPS)
    return [a[i] for i in range(n)]


class PhaseRecorder:
    """Phase timestamps of the measurement build (load(variant="phases")):
    a device buffer the kernels write the wall clock into at marked points.
    read() -> numpy int64 [3 regions][8192 workgroups][slots] (0 = not
    reached) after synchronising; clear() zeroes it; ticks_per_us the clock."""

    REGIONS = ("decode", "split", "attend")

    def __init__(self, device="cuda"):
        lib = load()
        if not lib.adamas_phase_stamps_built():
            raise RuntimeError("the loaded library has no phase stamps (load(variant='phases'))")
        n = int(lib.adamas_phase_buffer_bytes())
        self.buf = torch.zeros(n // 8, dtype=torch.int64, device=device)
        _check(lib.adamas_set_phase_buffer(ctypes.c_void_p(self.buf.data_ptr()), n),
               "adamas_set_phase_buffer")
        self.ticks_per_us = lib.adamas_wall_clock_khz() / 1000.0

    def clear(self):
        self.buf.zero_()

    def read(self):
        torch.cuda.synchronize(self.buf.device)
        return self.buf.view(3, 8192, -1).cpu().numpy()

    def close(self):
        load().adamas_set_phase_buffer(None, 0)


def set_wait_polls(polls: int) -> None:
    """Process-wide bound of each group wait, in polls (adamas_set_wait_polls);
    DEFAULT_WAIT_POLLS restores the library's default."""
    if not 0 <= int(polls) < 2 ** 32:
        raise ValueError("polls must fit an unsigned 32-bit integer")
    _check(load().adamas_set_wait_polls(int(polls)), "adamas_set_wait_polls")


def wait_polls() -> int:
    """The current group-wait bound (adamas_wait_polls)."""
    return int(load().adamas_wait_polls())


def decode_key_bytes(B: int, Hq: int, Hkv: int, n_ctx: int, budget: int, head_dim: int) -> int:
    """Bytes per chunk key the fused decode kernel keeps for this shape: 2, or 1
    where grouped heads would otherwise take several rounds of workgroups
    (adamas_decode_key_bytes)."""
    r = load().adamas_decode_key_bytes(B, Hq, Hkv, n_ctx, budget, head_dim)
    if r < 0:
        raise AdamasError(-r, "adamas_decode_key_bytes")
    return r


def decode_chunk_tokens(B: int, Hq: int, Hkv: int, n_ctx: int, budget: int, head_dim: int) -> int:
    """Tokens per chunk the decode step plans for this shape
    (adamas_decode_chunk_tokens)."""
    r = load().adamas_decode_chunk_tokens(B, Hq, Hkv, n_ctx, budget, head_dim)
    if r < 0:
        raise AdamasError(-r, "adamas_decode_chunk_tokens")
    return r


def set_decode_mode(mode: int) -> None:
    """Process-wide schedule of decode_step: DECODE_AUTO, DECODE_LAST_ARRIVAL,
    DECODE_GROUP_WAIT or DECODE_SPLIT (adamas_set_decode_mode)."""
    _check(load().adamas_set_decode_mode(int(mode)), "adamas_set_decode_mode")


def decode_path(B: int, Hq: int, Hkv: int, n_ctx: int, budget: int, head_dim: int) -> int:
    """The schedule decode_step would use for this shape on the current device."""
    r = load().adamas_decode_path(B, Hq, Hkv, n_ctx, budget, head_dim)
    if r < 0:
        raise AdamasError(-r, "adamas_decode_path")
    return r


def decode_step(q, k, v, k_codes, n_ctx: int, budget: int, scale: float = 0.0, out=None,
                idx_out=None, ws: Workspace | None = None, stream=None, n_sink: int = 0,
                n_recent: int = 0, check: bool = False) -> torch.Tensor:
    """One fused decode step of one layer -> out [B][Hq][d] (idx_out optional).
    The first n_sink and last n_recent tokens are always kept (adamas_decode_step_keep).
    With check=True the call waits for the step and raises GroupWaitGaveUp if a
    group wait gave up (Workspace.check); otherwise the caller checks the
    workspace when it synchronises."""
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    if k.dtype != q.dtype or v.dtype != q.dtype or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v must share dtype; k and v share shape")
    if tuple(k_codes.shape) != (B, Hkv, cap, d // 4) or k_codes.dtype != torch.uint8:
        raise ValueError("k_codes must be uint8 [B][Hkv][cap][d/4]")
    if out is None:
        out = torch.empty_like(q)
    nb = load().adamas_workspace_bytes(OP_DECODE_STEP, B, Hq, Hkv, n_ctx, budget, d)
    buf = _ws_for(q.device, ws).get(nb)
    head = (_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(k_codes, "k_codes"),
            _dtype_code(q), B, Hq, Hkv, d, cap, n_ctx, budget)
    tail = (float(scale), _dev_ptr(out, "out"), _dev_ptr(idx_out, "idx_out"), _dev_ptr(buf, "ws"),
            buf.numel(), _stream(q, stream))
    if n_sink == 0 and n_recent == 0:
        st = load().adamas_decode_step(*head, *tail)
    else:
        st = load().adamas_decode_step_keep(*head, int(n_sink), int(n_recent), *tail)
    _check(st, "adamas_decode_step")
    if check:
        (stream if stream is not None else torch.cuda.current_stream(q.device)).synchronize()
        _ws_for(q.device, ws).check()
    return out


STATIC_SCRATCH_BYTES = 16 << 20   # ADAMAS_STATIC_SCRATCH_BYTES


def decode_step_static(q, k, v, k_codes, n_ctx: int, budget: int, scale: float = 0.0,
                       out=None, idx_out=None, stream=None) -> torch.Tensor:
    """decode_step without a workspace (adamas_decode_step_static): the library's
    static per-device scratch, for callers that cannot allocate.  Calls that
    may overlap on one device race.  out / idx_out are the caller's."""
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    if k.dtype != q.dtype or v.dtype != q.dtype or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v must share dtype; k and v share shape")
    if tuple(k_codes.shape) != (B, Hkv, cap, d // 4) or k_codes.dtype != torch.uint8:
        raise ValueError("k_codes must be uint8 [B][Hkv][cap][d/4]")
    if out is None:
        out = torch.empty_like(q)
    st = load().adamas_decode_step_static(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(k_codes, "k_codes"),
        _dtype_code(q), B, Hq, Hkv, d, cap, n_ctx, budget, float(scale), _dev_ptr(out, "out"),
        _dev_ptr(idx_out, "idx_out"), _stream(q, stream))
    _check(st, "adamas_decode_step_static")
    return out


def decode_append_step(q, k, v, k_codes, lens, max_len: int, budget: int, k_new=None,
                       v_new=None, scale: float = 0.0, out=None, idx_out=None,
                       ws: Workspace | None = None, stream=None, n_sink: int = 0,
                       n_recent: int = 0) -> torch.Tensor:
    """One decode step over sequences of lengths lens (int32 [B], on the device),
    appending k_new / v_new [B][Hkv][d] at row lens[b] of the caches when given
    (adamas_decode_append_step).  lens is not advanced."""
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    if k.dtype != q.dtype or v.dtype != q.dtype or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v must share dtype; k and v share shape")
    if tuple(k_codes.shape) != (B, Hkv, cap, d // 4) or k_codes.dtype != torch.uint8:
        raise ValueError("k_codes must be uint8 [B][Hkv][cap][d/4]")
    if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("lens must be int32 [B]")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        for t in (k_new, v_new):
            if t.dtype != q.dtype or tuple(t.shape) != (B, Hkv, d):
                raise ValueError("k_new, v_new must be [B][Hkv][d] of q's dtype")
    if out is None:
        out = torch.empty_like(q)
    nb = load().adamas_workspace_bytes(OP_DECODE_STEP, B, Hq, Hkv, max_len, budget, d)
    buf = _ws_for(q.device, ws).get(nb)
    st = load().adamas_decode_append_step(
        _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), _dev_ptr(k, "k"),
        _dev_ptr(v, "v"), _dev_ptr(k_codes, "k_codes"), _dev_ptr(lens, "lens"), _dtype_code(q), B,
        Hq, Hkv, d, cap, max_len, budget, int(n_sink), int(n_recent), float(scale),
        _dev_ptr(out, "out"), _dev_ptr(idx_out, "idx_out"), _dev_ptr(buf, "ws"), buf.numel(),
        _stream(q, stream))
    _check(st, "adamas_decode_append_step")
    return out


def decode_paged_step(q, k_pool, v_pool, code_pool, page_table, lens, max_len: int, budget: int,
                      k_new=None, v_new=None, scale: float = 0.0, out=None, idx_out=None,
                      ws: Workspace | None = None, stream=None, n_sink: int = 0,
                      n_recent: int = 0) -> torch.Tensor:
    """decode_append_step over paged pools (adamas_decode_paged_step):
    k_pool / v_pool [n_pages][Hkv][page_size][d], code_pool [n_pages][Hkv][page_size][d/4],
    page_table int32 [B][max_pages], lens int32 [B]."""
    B, Hq, d = q.shape
    n_pages, Hkv, page, _ = k_pool.shape
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("q and the pools must share dtype; k and v pools share shape")
    if tuple(code_pool.shape) != (n_pages, Hkv, page, d // 4) or code_pool.dtype != torch.uint8:
        raise ValueError("code_pool must be uint8 [n_pages][Hkv][page_size][d/4]")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be int32 [B][max_pages]")
    if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("lens must be int32 [B]")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        for t in (k_new, v_new):
            if t.dtype != q.dtype or tuple(t.shape) != (B, Hkv, d):
                raise ValueError("k_new, v_new must be [B][Hkv][d] of q's dtype")
    if out is None:
        out = torch.empty_like(q)
    nb = load().adamas_workspace_bytes(OP_DECODE_STEP, B, Hq, Hkv, max_len, budget, d)
    buf = _ws_for(q.device, ws).get(nb)
    st = load().adamas_decode_paged_step(
        _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
        _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), _dev_ptr(code_pool, "code_pool"),
        _dev_ptr(page_table, "page_table"), _dev_ptr(lens, "lens"), _dtype_code(q), B, Hq, Hkv, d,
        page, n_pages, page_table.shape[1], max_len, budget, int(n_sink), int(n_recent),
        float(scale), _dev_ptr(out, "out"), _dev_ptr(idx_out, "idx_out"), _dev_ptr(buf, "ws"),
        buf.numel(), _stream(q, stream))
    _check(st, "adamas_decode_paged_step")
    return out
