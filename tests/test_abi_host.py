"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before anything is enqueued.

No call here reaches a kernel launch: each one fails host-side validation,
which runs before any HIP call (fake, never-dereferenced pointer values)."""
import ctypes
import os
import re

import pytest

import compressed_key_sparse_amd as adamas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adamas.h")

A = 0x10000     # a fake 16-byte-aligned device address (never dereferenced)
MIS = 0x10001   # misaligned
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(adamas.library_path()):
        from compressed_key_sparse_amd import _build
        _build.build(force=False)
    return adamas.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(adamas_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"adamas_encode_keys", "adamas_score", "adamas_select_topk",
                          "adamas_sparse_attend", "adamas_decode_step", "adamas_workspace_bytes",
                          "adamas_status_string", "adamas_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.adamas_version() == 100
    for s in range(5):
        assert lib.adamas_status_string(s)
    assert lib.adamas_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    f = lib.adamas_workspace_bytes
    assert f(2, 1, 32, 32, 131072, 256, 128) > 65536
    assert f(2, 1, 32, 32, 131072, 256, 96) == 0      # head_dim
    assert f(2, 1, 24, 7, 1000, 64, 128) == 0          # Hq % Hkv
    assert f(2, 1, 32, 2, 1000, 64, 128) == 0          # group of 16 > 8
    assert f(0, 1, 32, 1, 1000, 64, 128) > 0           # select ignores Hkv grouping
    assert f(2, 1, 32, 32, 0, 64, 128) == 0
    assert f(2, 1, 32, 32, 1000, 0, 128) == 0
    assert f(7, 1, 32, 32, 1000, 64, 128) == 0         # unknown op
    # never shrinks with the context; grows with the budget
    assert f(2, 1, 32, 32, 262144, 256, 128) >= f(2, 1, 32, 32, 131072, 256, 128)
    assert f(1, 1, 32, 32, 1, 1024, 128) > f(1, 1, 32, 32, 1, 64, 128)


def test_encode_validation(lib):
    f = lib.adamas_encode_keys
    assert f(A, 0, 1, 1, 4, 96, A, 8, 0, None, None) == UNSUPPORTED
    assert f(A, 2, 1, 1, 4, 128, A, 8, 0, None, None) == UNSUPPORTED
    assert f(A, 1, 1, 1, 4, 128, A, 8, 5, None, None) == INVALID     # pos + n > cap
    assert f(A, 1, 1, 1, -1, 128, A, 8, 0, None, None) == INVALID
    assert f(A, 1, 0, 1, 4, 128, A, 8, 0, None, None) == INVALID
    assert f(MIS, 1, 1, 1, 4, 128, A, 8, 0, None, None) == INVALID
    assert f(A, 1, 1, 1, 4, 128, None, 8, 0, None, None) == INVALID
    assert f(A, 1, 1, 1, 4, 128, A, 8, 0, MIS, None) == INVALID
    assert f(A, 1, 1, 1, 0, 128, A, 8, 0, None, None) == OK            # n = 0: no-op


def test_encode_paged_validation(lib):
    f = lib.adamas_encode_keys_paged

    def call(**kw):
        return f(kw.get("x", A), kw.get("dt", 1), kw.get("batch", 2), 4, kw.get("n", 1500),
                 kw.get("d", 128), kw.get("pool", A), kw.get("xpool", None),
                 kw.get("table", A), kw.get("page", 1024), kw.get("n_pages", 8),
                 kw.get("max_pages", 2), kw.get("pos", 100), None)
    assert call(d=96) == UNSUPPORTED
    assert call(dt=2) == UNSUPPORTED
    assert call(page=1000) == UNSUPPORTED           # not a power of two
    assert call(page=512) == UNSUPPORTED
    assert call(page=32768) == UNSUPPORTED
    assert call(pos=600) == INVALID                 # 600 + 1500 > 2 pages of 1024
    assert call(n=-1) == INVALID
    assert call(pos=-1) == INVALID
    assert call(batch=0) == INVALID
    assert call(n_pages=0) == INVALID
    assert call(max_pages=0) == INVALID
    assert call(x=MIS) == INVALID
    assert call(pool=None) == INVALID
    assert call(xpool=MIS) == INVALID
    assert call(table=None) == INVALID
    assert call(table=A + 2) == INVALID
    assert call(n=0) == OK                          # a no-op


def test_score_validation(lib):
    f = lib.adamas_score
    assert f(A, A, 1, 6, 4, 128, 100, 10, A, None) == INVALID          # Hq % Hkv
    assert f(A, A, 1, 4, 4, 128, 100, 101, A, None) == INVALID         # n_ctx > cap
    assert f(A, A, 1, 4, 4, 80, 100, 10, A, None) == UNSUPPORTED
    assert f(A, A, 1, 18, 2, 128, 100, 10, A, None) == UNSUPPORTED     # group of 9
    assert f(A, MIS, 1, 4, 4, 128, 100, 10, A, None) == INVALID
    assert f(A, A, 1, 4, 4, 128, 100, 0, A, None) == OK                # empty: no-op


def test_select_validation(lib):
    f = lib.adamas_select_topk
    need = lib.adamas_workspace_bytes(0, 1, 4, 1, 1000, 64, 128)
    assert f(A, 1, 4, 1000, 128, 0, A, A, need, None) == INVALID       # budget 0
    assert f(A, 1, 4, 0, 128, 64, A, A, need, None) == INVALID         # empty context
    assert f(A, 1, 4, 1000, 64 + 1, 64, A, A, need, None) == UNSUPPORTED
    assert f(A, 1, 4, 1000, 128, 64, A, None, need, None) == WORKSPACE
    assert f(A, 1, 4, 1000, 128, 64, A, A, need - 1, None) == WORKSPACE
    assert f(A, 1, 4, 1000, 128, 64, MIS, A, need, None) == INVALID
    assert f(A, 1, 8193, 1000, 128, 64, A, A, need, None) == UNSUPPORTED  # > 8192 rows


def test_attend_validation(lib):
    f = lib.adamas_sparse_attend
    need = lib.adamas_workspace_bytes(1, 1, 4, 2, 1, 64, 128)
    args = lambda **kw: [kw.get("q", A), A, A, kw.get("dt", 1), A, 1, kw.get("hq", 4), 2, 128,
                         100, kw.get("budget", 64), ctypes.c_float(kw.get("scale", 0.0)), A, A,
                         kw.get("ws", need), None]
    assert f(*args(hq=5)) == INVALID
    assert f(*args(dt=3)) == UNSUPPORTED
    assert f(*args(q=MIS)) == INVALID
    assert f(*args(budget=0)) == INVALID
    assert f(*args(scale=float("nan"))) == INVALID
    assert f(*args(ws=need - 1)) == WORKSPACE


def test_decode_validation(lib):
    f = lib.adamas_decode_step
    need = lib.adamas_workspace_bytes(2, 1, 8, 4, 1000, 64, 128)
    def call(**kw):
        return f(A, A, A, kw.get("codes", A), kw.get("dt", 1), 1, kw.get("hq", 8),
                 kw.get("hkv", 4), kw.get("d", 128), kw.get("cap", 1024), kw.get("n", 1000),
                 kw.get("budget", 64), ctypes.c_float(0.0), A, kw.get("idx", None), A,
                 kw.get("ws", need), None)
    assert call(n=0) == INVALID
    assert call(n=1025) == INVALID
    assert call(hkv=3) == INVALID
    assert call(hq=36, hkv=4) == UNSUPPORTED   # group of 9
    assert call(d=96) == UNSUPPORTED
    assert call(codes=MIS) == INVALID
    assert call(idx=MIS) == INVALID
    assert call(ws=need - 1) == WORKSPACE
    assert call(budget=0) == INVALID


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(adamas, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(adamas, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        adamas.load()


def test_decode_mode_validation(lib):
    assert lib.adamas_set_decode_mode(4) == INVALID
    assert lib.adamas_set_decode_mode(-1) == INVALID
    for m in (3, 2, 1, 0):                  # SPLIT, GROUP_WAIT, LAST_ARRIVAL, back to AUTO
        assert lib.adamas_set_decode_mode(m) == OK
    # shape checks come before any device query
    f = lib.adamas_decode_path
    assert f(1, 32, 32, 0, 256, 128) == -INVALID
    assert f(1, 32, 7, 1000, 256, 128) == -INVALID
    assert f(1, 32, 32, 1000, 256, 96) == -INVALID
    assert f(1, 32, 2, 1000, 256, 128) == -INVALID     # 16 query heads per KV head
    assert f(1, 32, 32, 1000, 0, 128) == -INVALID


def test_status_word_inside_control_bytes():
    assert adamas.WS_STATUS_OFFSET + 4 <= adamas.WS_CTRL_BYTES
    text = open(HEADER).read()
    assert f"#define ADAMAS_WS_CTRL_BYTES {adamas.WS_CTRL_BYTES}" in text
    assert f"#define ADAMAS_WS_STATUS_OFFSET {adamas.WS_STATUS_OFFSET}" in text


def test_stream_read_validation(lib):
    f = lib.adamas_stream_read
    assert f(MIS, 64, A, None) == INVALID
    assert f(A, 0, A, None) == INVALID
    assert f(A, 40, A, None) == INVALID          # not a multiple of 16
    assert f(A, 64, None, None) == INVALID
    assert lib.adamas_stream_read_blocks(16) == 1
    assert lib.adamas_stream_read_blocks(1 << 40) == 1024


def test_keep_validation(lib):
    f = lib.adamas_select_topk_keep
    need = lib.adamas_workspace_bytes(0, 1, 4, 1, 1000, 64, 128)
    assert f(A, 1, 4, 1000, 128, 64, -1, 0, A, A, need, None) == INVALID
    assert f(A, 1, 4, 1000, 128, 64, 0, -5, A, A, need, None) == INVALID
    g = lib.adamas_decode_step_keep
    need = lib.adamas_workspace_bytes(2, 1, 8, 4, 1000, 64, 128)
    args = lambda s, r: [A, A, A, A, 1, 1, 8, 4, 128, 1024, 1000, 64, s, r, ctypes.c_float(0.0),
                         A, None, A, need, None]
    assert g(*args(-1, 0)) == INVALID
    assert g(*args(0, -1)) == INVALID


def test_rotation_switch_validation(lib):
    assert lib.adamas_set_rotation(3) == INVALID
    assert lib.adamas_set_rotation(2) == OK
    assert lib.adamas_set_rotation(-1) == INVALID
    assert lib.adamas_set_rotation(0) == OK
    assert lib.adamas_set_rotation(1) == OK


def test_append_step_validation(lib):
    f = lib.adamas_decode_append_step
    need = lib.adamas_workspace_bytes(2, 2, 8, 4, 1000, 64, 128)

    def call(**kw):
        return f(A, kw.get("kn", A), kw.get("vn", A), A, A, kw.get("codes", A),
                 kw.get("lens", A), kw.get("dt", 1), 2, kw.get("hq", 8), kw.get("hkv", 4),
                 kw.get("d", 128), kw.get("cap", 1024), kw.get("max_len", 1000),
                 kw.get("budget", 64), kw.get("sink", 0), kw.get("recent", 0),
                 ctypes.c_float(0.0), A, kw.get("idx", None), A, kw.get("ws", need), None)
    assert call(max_len=0) == INVALID
    assert call(max_len=1025) == INVALID           # beyond the cache
    assert call(kn=None) == INVALID                # only one of k_new, v_new
    assert call(vn=None) == INVALID
    assert call(lens=None) == INVALID
    assert call(lens=A + 2) == INVALID             # lens needs 4-byte alignment
    assert call(kn=MIS) == INVALID
    assert call(codes=MIS) == INVALID
    assert call(idx=MIS) == INVALID
    assert call(hkv=3) == INVALID
    assert call(hq=36, hkv=4) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED
    assert call(dt=3) == UNSUPPORTED
    assert call(budget=0) == INVALID
    assert call(sink=-1) == INVALID
    assert call(ws=need - 1) == WORKSPACE


def test_paged_step_validation(lib):
    f = lib.adamas_decode_paged_step
    need = lib.adamas_workspace_bytes(2, 2, 8, 4, 4096, 64, 128)

    def call(**kw):
        return f(A, A, A, A, A, A, kw.get("table", A), A, 1, 2, 8, 4, 128,
                 kw.get("page", 1024), kw.get("n_pages", 16), kw.get("max_pages", 4),
                 kw.get("max_len", 4096), 64, 0, 0, ctypes.c_float(0.0), A, None, A,
                 kw.get("ws", need), None)
    assert call(page=1000) == UNSUPPORTED           # not a power of two
    assert call(page=512) == UNSUPPORTED            # below one wavefront load per head
    assert call(page=32768) == UNSUPPORTED
    assert call(n_pages=0) == INVALID
    assert call(max_pages=0) == INVALID
    assert call(table=None) == INVALID
    assert call(table=A + 2) == INVALID
    assert call(max_len=4097) == INVALID            # beyond max_pages * page_size
    assert call(ws=need - 1) == WORKSPACE


def test_head_dim_256_accepted_512_not(lib):
    assert lib.adamas_workspace_bytes(2, 1, 32, 32, 131072, 256, 256) > 0
    assert lib.adamas_workspace_bytes(2, 1, 32, 32, 131072, 256, 512) == 0
    assert lib.adamas_encode_keys(A, 1, 1, 1, 0, 256, A, 8, 0, None, None) == OK
    assert lib.adamas_encode_keys(A, 1, 1, 1, 4, 512, A, 8, 0, None, None) == UNSUPPORTED
    assert lib.adamas_decode_path(1, 32, 32, 1000, 256, 512) == -INVALID


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU: --gpus N > 1 and a multi-rank launch
    exit with a message before any GPU work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    env["WORLD_SIZE"] = "2"
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 2 and "single-GPU" in r.stderr


def test_wait_polls_setter(lib):
    """The group-wait bound is process-wide and round-trips; the binding
    restores the default."""
    lib.adamas_set_wait_polls.argtypes = [ctypes.c_uint32]
    lib.adamas_wait_polls.restype = ctypes.c_uint32
    assert lib.adamas_wait_polls() == adamas.DEFAULT_WAIT_POLLS
    assert lib.adamas_set_wait_polls(0) == OK
    assert lib.adamas_wait_polls() == 0
    adamas.set_wait_polls(12345)
    assert adamas.wait_polls() == 12345
    with pytest.raises(ValueError):
        adamas.set_wait_polls(-1)
    adamas.set_wait_polls(adamas.DEFAULT_WAIT_POLLS)
    assert adamas.wait_polls() == adamas.DEFAULT_WAIT_POLLS


def test_bucket_alpha_setter(lib):
    """The per-head-group bucketing table: validation leaves the table as it
    was; the binding round-trips and restores the fixed rule."""
    F = ctypes.c_float * 70
    good = F(*([0.25, 0.75, 0.0, 1.5] + [0.5] * 66))
    assert lib.adamas_bucket_alpha(None, 0) == 0
    assert lib.adamas_set_bucket_alpha(good, 4) == OK
    assert adamas.bucket_alpha() == [0.25, 0.75, 0.0, 1.5]
    assert lib.adamas_set_bucket_alpha(good, 65) == INVALID
    assert lib.adamas_set_bucket_alpha(good, -1) == INVALID
    assert lib.adamas_set_bucket_alpha(None, 2) == INVALID
    for bad in (-0.25, float("inf"), float("nan")):
        assert lib.adamas_set_bucket_alpha(F(0.5, bad), 2) == INVALID
    assert adamas.bucket_alpha() == [0.25, 0.75, 0.0, 1.5]
    assert lib.adamas_set_bucket_alpha(good, 64) == OK
    assert len(adamas.bucket_alpha()) == 64
    with pytest.raises(ValueError):
        adamas.set_bucket_alpha([0.5] * 65)
    adamas.set_bucket_alpha([0.3])
    assert adamas.bucket_alpha() == [pytest.approx(0.3)]
    adamas.set_bucket_alpha(None)
    assert adamas.bucket_alpha() == []


def test_decode_key_bytes_planning(lib):
    """Grouped heads that would need two rounds of workgroups with 16-bit
    chunk keys plan 8-bit keys; MHA, head_dim 256 and one-round launches keep
    16-bit keys; invalid shapes raise."""
    kb = adamas.decode_key_bytes
    assert kb(1, 24, 8, 1048576, 1024, 128) == 1      # the 1M-token GQA layer
    assert kb(1, 24, 8, 1048576, 1024, 64) == 1
    assert kb(1, 32, 32, 131072, 256, 128) == 2       # MHA
    assert kb(1, 24, 8, 1048576, 1024, 256) == 2      # head_dim 256
    assert kb(1, 24, 8, 32768, 256, 128) == 2         # one round either way
    assert kb(2, 24, 8, 300000, 1024, 128) == 1       # the GPU parity shapes
    assert kb(16, 4, 2, 140000, 256, 128) == 1
    assert kb(16, 4, 2, 140000, 1024, 128) == 1
    with pytest.raises(adamas.AdamasError):
        kb(1, 24, 7, 1000, 64, 128)
    # the workspace covers both key widths of a shape
    ws = lib.adamas_workspace_bytes(2, 2, 24, 8, 300000, 1024, 128)
    assert ws > 0


def test_decode_chunk_planning(lib):
    """Chunk lengths the decode step plans: 16384 tokens at most with 16-bit
    keys, shorter while the launch still fits one round, 32768 with one-byte
    keys and for multi-headed launches of several rounds that keep two
    workgroups per compute unit; invalid shapes raise."""
    ct = adamas.decode_chunk_tokens
    assert ct(1, 32, 32, 131072, 256, 128) == 16384   # the 128K layer: one round
    assert ct(1, 32, 32, 32768, 256, 128) == 4096     # shorter chunks fill the device
    assert ct(1, 1, 1, 1024, 64, 64) == 1024
    assert ct(16, 32, 32, 65536, 512, 128) == 32768   # batch 16: eight rounds become four
    assert ct(8, 32, 32, 40000, 256, 128) == 32768
    assert ct(16, 32, 32, 65536, 512, 256) == 32768
    assert ct(1, 24, 8, 1048576, 1024, 128) == 32768  # one-byte keys
    assert ct(1, 24, 8, 1048576, 1024, 256) == 16384
    # one round of 32768-token chunks would leave one workgroup per compute unit
    assert ct(2, 32, 32, 131072, 256, 128) == 16384
    assert ct(8, 32, 32, 20001, 256, 128) == 16384
    with pytest.raises(adamas.AdamasError):
        ct(1, 24, 7, 1000, 64, 128)
    # the workspace covers the plan of either chunk length
    assert lib.adamas_workspace_bytes(2, 16, 32, 32, 65536, 512, 128) > 0
