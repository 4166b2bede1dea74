"""GPU parity: every entry point of the C ABI against the CPU oracle.

Codes, distances and selected indices must be bit-exact; attention outputs
must be within the relative error bound (2e-3 bf16, 1e-5 fp32) of the
oracle's binary64 result rounded to the output type.  Inputs are seeded
synthetic draws (synth.py); the oracle receives byte-identical host copies.
"""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import check_out, host, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    adamas.load()


def _dt(name):
    return torch.float32 if name == "f32" else torch.bfloat16


# ------------------------------------------------------------------ encode
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_encode_random(ora, d, dt):
    log(f"encode random d={d} dt={dt}")
    x = synth.random_values((2, 3, 777, d), _dt(dt), seed=d, device=DEV, scale=3.0)
    codes = torch.full((2, 3, 1000, d // 4), 0x5A, dtype=torch.uint8, device=DEV)
    copy = torch.zeros((2, 3, 1000, d), dtype=_dt(dt), device=DEV)
    adamas.encode_keys(x, codes, pos=100, x_copy=copy)
    ref = np.full((2, 3, 1000, d // 4), 0x5A, np.uint8)
    ora.encode_keys(host(x), ref, cap=1000, pos=100)
    assert np.array_equal(codes.cpu().numpy(), ref)
    assert torch.equal(copy[:, :, 100:877], x) and not copy[:, :, :100].any()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_encode_edge_values(ora, d):
    log(f"encode edge values d={d}")
    n = 64
    rows = [np.zeros(d, np.float32), -np.zeros(d, np.float32)]
    rows += [np.eye(d, dtype=np.float32)[j] for j in (0, 1, d - 1)]
    rows += list(synth.integer_values((20, d), -3, 3, seed=1))          # exact ties
    rows += list(synth.integer_values((10, d), 0, 1, seed=2))
    rows.append(np.full(d, 1e-42, np.float32))                           # denormals
    rows.append(np.full(d, 3e36, np.float32) * np.sign(np.arange(d) - d / 2 + 0.5))
    rows.append(np.where(np.arange(d) % 3 == 0, 1e-40, -2e-41).astype(np.float32))
    while len(rows) < n:
        rows.append(rows[len(rows) % 7] * np.float32(2.0 ** (len(rows) - 40)))
    x = np.stack(rows[:n]).reshape(1, 1, n, d).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV)
    codes = torch.zeros((1, 1, n, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(xt, codes)
    assert np.array_equal(codes.cpu().numpy(), ora.encode_keys(x))
    xb = xt.to(torch.bfloat16)
    adamas.encode_keys(xb, codes)
    assert np.array_equal(codes.cpu().numpy(), ora.encode_keys(host(xb)))


def test_encode_query_and_large_batch(ora):
    log("encode: queries (n=1) and a 4096-token prefill chunk")
    q = synth.random_values((16, 32, 128), torch.bfloat16, seed=3, device=DEV)
    qc = adamas.encode_query(q)
    assert np.array_equal(qc.cpu().numpy(), ora.encode_keys(host(q)[:, :, None, :])[:, :, 0])
    w = synth.BATCH16_64K
    chunk = synth.make_chunk(w, 0, DEV)
    codes = torch.zeros((1, 32, 4096 + 16, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(chunk, codes, pos=16)
    ref = ora.encode_keys(host(chunk), np.zeros((1, 32, 4096 + 16, 32), np.uint8), 4096 + 16, 16)
    assert np.array_equal(codes.cpu().numpy(), ref)


# ------------------------------------------------------------------- score
@pytest.mark.parametrize("d,hq,hkv,n", [(128, 4, 4, 9000), (64, 6, 2, 4097), (128, 24, 8, 300),
                                        (128, 8, 1, 5000), (64, 3, 3, 1), (128, 2, 1, 255),
                                        (256, 4, 2, 5000), (256, 8, 1, 3000)])
def test_score(ora, d, hq, hkv, n):
    log(f"score d={d} hq={hq} hkv={hkv} n={n}")
    g = torch.Generator(device=DEV).manual_seed(n + hq)
    cap = n + 37
    kc = torch.randint(0, 256, (2, hkv, cap, d // 4), generator=g, device=DEV,
                       dtype=torch.int32).to(torch.uint8)
    qc = torch.randint(0, 256, (2, hq, d // 4), generator=g, device=DEV,
                       dtype=torch.int32).to(torch.uint8)
    dist = adamas.score(qc, kc, n_ctx=n)
    ref = ora.score(qc.cpu().numpy(), kc.cpu().numpy(), n_ctx=n)
    assert np.array_equal(dist.cpu().numpy(), ref)


# ------------------------------------------------------------------ select
@pytest.mark.parametrize("n,budget,hi", [(1, 1, 5), (100, 64, 3), (100, 200, 3), (4097, 64, 384),
                                         (20000, 256, 40), (20000, 1000, 2), (70000, 256, 384),
                                         (9000, 4096, 10), (33, 32, 0)])
def test_select(ora, n, budget, hi):
    log(f"select n={n} budget={budget} values<={hi}")
    g = torch.Generator(device=DEV).manual_seed(n * 7 + budget)
    dist = torch.randint(0, hi + 1, (2, 3, n), generator=g, device=DEV,
                         dtype=torch.int32).to(torch.uint16)
    idx = adamas.select_topk(dist, budget, head_dim=128)
    ref = ora.select_topk(dist.cpu().numpy(), budget)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("n,budget", [(5000, 128), (70000, 1024)])
def test_select_d256_distances(ora, n, budget):
    log(f"select with head_dim 256 distances (0..768) n={n} budget={budget}")
    g = torch.Generator(device=DEV).manual_seed(n + 256)
    dist = torch.randint(0, 769, (1, 4, n), generator=g, device=DEV,
                         dtype=torch.int32).to(torch.uint16)
    idx = adamas.select_topk(dist, budget, head_dim=256)
    assert np.array_equal(idx.cpu().numpy(), ora.select_topk(dist.cpu().numpy(), budget))


# ------------------------------------------------------------------ attend
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("budget", [1, 31, 256, 1000])
def test_sparse_attend(ora, d, dt, budget):
    log(f"attend d={d} dt={dt} budget={budget}")
    B, Hq, Hkv, cap = 2, 6, 3, 3000
    dtype = _dt(dt)
    q = synth.random_values((B, Hq, d), dtype, seed=1, device=DEV)
    k = synth.random_values((B, Hkv, cap, d), dtype, seed=2, device=DEV)
    v = synth.random_values((B, Hkv, cap, d), dtype, seed=3, device=DEV, scale=2.0)
    rng = np.random.default_rng(budget)
    idx = np.full((B, Hq, budget), -1, np.int32)
    for b in range(B):
        for h in range(Hq):
            m = int(rng.integers(1, budget + 1)) if h else budget
            idx[b, h, :m] = np.sort(rng.choice(cap, size=m, replace=False))
    idx[0, 1, :] = -1                      # a head with nothing selected -> zeros
    it = torch.from_numpy(idx).to(DEV)
    out = adamas.sparse_attend(q, k, v, it)
    ref, ref64 = ora.sparse_attend(host(q), host(k), host(v), idx)
    check_out(ora, out, host(q), host(k), host(v), idx, ref, ref64, f"attend d={d} {dt}")
    assert not out[0, 1].any()


def test_sparse_attend_single_row_exact(ora):
    q = synth.random_values((1, 4, 128), torch.bfloat16, seed=4, device=DEV)
    k = synth.random_values((1, 4, 50, 128), torch.bfloat16, seed=5, device=DEV)
    v = synth.random_values((1, 4, 50, 128), torch.bfloat16, seed=6, device=DEV)
    idx = torch.tensor([[[7], [0], [49], [23]]], dtype=torch.int32, device=DEV)
    out = adamas.sparse_attend(q, k, v, idx)
    for h, t in enumerate((7, 0, 49, 23)):
        assert torch.equal(out[0, h], v[0, h, t])


# ------------------------------------------------------------- decode step
def _decode_case(ora, w, n_ctx=None, budget=None, layer=0):
    n_ctx = w.n_ctx if n_ctx is None else n_ctx
    budget = w.budget if budget is None else budget
    lay = synth.make_layer(w, layer, DEV, n_ctx=n_ctx)
    cap = lay["cap"]
    codes = torch.zeros((w.batch, w.hkv, cap, w.head_dim // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((w.batch, w.hq, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n_ctx, budget, idx_out=idx)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k)
    assert np.array_equal(codes.cpu().numpy(), ocodes), "code cache differs"
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, n_ctx, budget)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, f"{w.name} n={n_ctx} budget={budget}")
    return lay, out, idx


def test_decode_tiny_config(ora):
    log("decode: tiny single-head fp32 config (full size)")
    lay, out, idx = _decode_case(ora, synth.TINY)
    p = int(lay["needles"][0, 0, 0, 0])
    assert p in idx[0, 0].tolist()       # the planted key is selected


@pytest.mark.parametrize("n,budget", [(1, 64), (63, 64), (64, 64), (700, 64), (5000, 256),
                                      (20000, 1024), (4096, 2048), (30000, 20000),
                                      (70000, 512), (1000, 100000)])
def test_decode_small_mha(ora, n, budget):
    log(f"decode small MHA n={n} budget={budget}")
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=n, cap=n + 100, budget=budget)
    _decode_case(ora, w)


@pytest.mark.parametrize("hq,hkv", [(6, 2), (24, 8), (8, 1), (5, 5)])
def test_decode_small_gqa(ora, hq, hkv):
    log(f"decode small GQA hq={hq} hkv={hkv}")
    w = synth.LLAMA32_GQA_1M.replace(hq=hq, hkv=hkv, n_ctx=9001, cap=9001, budget=128)
    _decode_case(ora, w)


def test_decode_fp32_d64_batch(ora):
    log("decode fp32 d=64 batch 3")
    w = synth.TINY.replace(batch=3, hq=4, hkv=2, n_ctx=3000, cap=3000, budget=100)
    _decode_case(ora, w)


def test_decode_full_budget_equals_dense(ora):
    log("decode: budget >= n equals dense attention over all n rows")
    w = synth.LLAMA2_32K.replace(hq=2, hkv=2, n_ctx=500, cap=500, budget=512)
    lay, out, idx = _decode_case(ora, w)
    assert idx[..., :500].equal(torch.arange(500, device=DEV, dtype=torch.int32).expand(1, 2, 500))
    assert (idx[..., 500:] == -1).all()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    dense_idx = np.tile(np.arange(500, dtype=np.int32), (1, 2, 1))
    ref, ref64 = ora.sparse_attend(q, k, v, dense_idx)
    check_out(ora, out, q, k, v, dense_idx, ref, ref64, "dense")


def test_decode_deterministic_and_workspace_reuse(ora):
    log("decode: run-twice bit determinism; one workspace across shapes")
    ws = adamas.Workspace(DEV)
    w = synth.LLAMA2_32K.replace(hq=8, hkv=8, n_ctx=12000, cap=12000, budget=256)
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((1, 8, 12000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    outs = []
    for n, bud in ((12000, 256), (5000, 64), (12000, 256), (777, 1024), (12000, 256)):
        idx = torch.empty((1, 8, bud), dtype=torch.int32, device=DEV)
        o = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, bud, idx_out=idx, ws=ws)
        outs.append((n, bud, o.clone(), idx.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][2], outs[2][2]) and torch.equal(outs[0][2], outs[4][2])
    assert torch.equal(outs[0][3], outs[2][3]) and torch.equal(outs[0][3], outs[4][3])
    # control bytes back to zero after every call
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k)
    for n, bud, o, idx in outs[:4]:
        _, _, oidx = ora.decode_step(q, k, v, oc, n, bud)
        assert np.array_equal(idx.cpu().numpy(), oidx)


# ------------------------------------------- decode schedules, both forced
_SCHED_CASES = {
    "mha-5000-b256": synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=5000, cap=5100, budget=256),
    "mha-70000-b512": synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=70000, cap=70000, budget=512),
    "mha-30000-b20000": synth.LLAMA2_32K.replace(hq=2, hkv=2, n_ctx=30000, cap=30000,
                                                 budget=20000),
    "mha-1-b64": synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=1, cap=16, budget=64),
    "gqa-24-8-9001": synth.LLAMA32_GQA_1M.replace(hq=24, hkv=8, n_ctx=9001, cap=9001, budget=128),
    "gqa-8-1-9001": synth.LLAMA32_GQA_1M.replace(hq=8, hkv=1, n_ctx=9001, cap=9001, budget=300),
    "f32-d64-batch3": synth.TINY.replace(batch=3, hq=4, hkv=2, n_ctx=3000, cap=3000, budget=100),
    "gqa-6-2-300000-b1024": synth.LLAMA32_GQA_1M.replace(hq=6, hkv=2, n_ctx=300000, cap=300000,
                                                         budget=1024),
}


@pytest.fixture
def restore_mode():
    yield
    adamas.set_decode_mode(adamas.DECODE_AUTO)


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
                                  adamas.DECODE_SPLIT])
@pytest.mark.parametrize("case", sorted(_SCHED_CASES))
def test_decode_schedules(ora, restore_mode, mode, case):
    _check_schedule(ora, _SCHED_CASES[case], mode, case)


# split schedule only: more chunks (74 of 4096 tokens) than the selection
# kernel's register path takes, so its general count passes run at d = 128
_SPLIT_CASES = {
    "gqa-16-2-300000-b512": synth.LLAMA32_GQA_1M.replace(hq=16, hkv=2, n_ctx=300000,
                                                         cap=300000, budget=512),
}


@pytest.mark.parametrize("case", sorted(_SPLIT_CASES))
def test_decode_split_many_chunks(ora, restore_mode, case):
    _check_schedule(ora, _SPLIT_CASES[case], adamas.DECODE_SPLIT, case)


def _check_schedule(ora, w, mode, case):
    log(f"decode schedule {mode} {case}")
    adamas.set_decode_mode(mode)
    assert adamas.decode_path(w.batch, w.hq, w.hkv, w.n_ctx, w.budget, w.head_dim) == mode
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    ws = adamas.Workspace(DEV)
    idx = torch.empty((w.batch, w.hq, w.budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                             idx_out=idx, ws=ws)
    out_noidx = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget, ws=ws)
    torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any(), "control bytes or status word left set"
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), w.n_ctx, w.budget)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, case)
    assert torch.equal(out, out_noidx)


def test_decode_schedule_choice(restore_mode):
    adamas.set_decode_mode(adamas.DECODE_AUTO)
    # one 256-row batch per head: the last workgroup attends alone
    assert adamas.decode_path(1, 32, 32, 131072, 256, 128) == adamas.DECODE_LAST_ARRIVAL
    # 1024 rows per head would need a second launch; 256 workgroups fit the device
    assert adamas.decode_path(1, 32, 32, 131072, 1024, 128) == adamas.DECODE_GROUP_WAIT
    # 512 KV heads of chunks do not fit: the last-arrival schedule takes them
    assert adamas.decode_path(16, 32, 32, 65536, 512, 128) == adamas.DECODE_LAST_ARRIVAL
    # 128 chunks of 1024 candidates per head at 1M tokens: selection on its own
    assert adamas.decode_path(1, 24, 8, 1048576, 1024, 128) == adamas.DECODE_SPLIT
    assert adamas.decode_path(1, 32, 32, 1048576, 256, 128) == adamas.DECODE_SPLIT
    adamas.set_decode_mode(adamas.DECODE_GROUP_WAIT)
    assert adamas.decode_path(1, 32, 32, 131072, 256, 128) == adamas.DECODE_GROUP_WAIT
    adamas.set_decode_mode(adamas.DECODE_GROUP_WAIT)
    with pytest.raises(adamas.AdamasError):
        adamas.decode_path(16, 32, 32, 65536, 512, 128)


def test_stream_read_reads_every_byte():
    # the reference read's sink words XOR to the XOR of the whole buffer
    g = torch.Generator(device=DEV).manual_seed(7)
    for n in (4, 1000, (1 << 22) + 12):
        x = torch.randint(-2**31, 2**31 - 1, (n,), generator=g, device=DEV, dtype=torch.int32)
        sink = adamas.stream_read(x)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(x.cpu().numpy().view(np.uint32))
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, n


# -------------------------------------------- always-kept sinks and window
@pytest.mark.parametrize("n,budget,n_sink,n_recent,hi", [
    (3000, 64, 4, 60, 6), (3000, 64, 64, 0, 6), (3000, 64, 0, 100, 6), (3000, 50, 40, 40, 2),
    (20000, 256, 1, 32, 384), (777, 1000, 5, 5, 3), (70000, 512, 16, 256, 40)])
def test_select_keep(ora, n, budget, n_sink, n_recent, hi):
    log(f"select keep n={n} budget={budget} sink={n_sink} recent={n_recent}")
    g = torch.Generator(device=DEV).manual_seed(n + budget + n_sink)
    dist = torch.randint(0, hi + 1, (2, 3, n), generator=g, device=DEV,
                         dtype=torch.int32).to(torch.uint16)
    idx = adamas.select_topk(dist, budget, head_dim=128, n_sink=n_sink, n_recent=n_recent)
    ref = ora.select_topk(dist.cpu().numpy(), budget, n_sink, n_recent)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
                                  adamas.DECODE_SPLIT])
@pytest.mark.parametrize("n,budget,n_sink,n_recent", [
    (5000, 256, 4, 64), (70000, 512, 1, 128), (9001, 128, 128, 0), (30000, 1024, 8, 1000)])
def test_decode_keep(ora, restore_mode, mode, n, budget, n_sink, n_recent):
    log(f"decode keep mode {mode} n={n} budget={budget} sink={n_sink} recent={n_recent}")
    adamas.set_decode_mode(mode)
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=n, cap=n, budget=budget)
    lay = synth.make_layer(w, 1, DEV)
    codes = torch.zeros((1, 4, n, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((1, 4, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, budget, idx_out=idx,
                             n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), n, budget, 0.0, n_sink,
                                      n_recent)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, "keep")


# ------------------------- 32768-token chunks (multi-round MHA launches)
# Launches of several rounds of one-query-per-KV-head workgroups run two per
# compute unit with chunks of 32768 tokens, each selected a half at a time;
# the second chunk here is a 7232-token tail.
_LONG_CASES = {
    "bf16-d128-b256": (synth.LLAMA2_32K.replace(batch=8, hq=32, hkv=32, n_ctx=40000, cap=40000,
                                                budget=256), 0, 0),
    "bf16-d128-b512-keep": (synth.LLAMA2_32K.replace(batch=8, hq=32, hkv=32, n_ctx=40000,
                                                     cap=40010, budget=512), 3, 200),
    "f32-d64-b100": (synth.TINY.replace(batch=8, hq=32, hkv=32, n_ctx=40000, cap=40000,
                                        budget=100), 0, 0),
}


@pytest.mark.parametrize("mode", [adamas.DECODE_AUTO, adamas.DECODE_SPLIT])
@pytest.mark.parametrize("case", sorted(_LONG_CASES))
def test_decode_long_chunks(ora, restore_mode, mode, case):
    w, n_sink, n_recent = _LONG_CASES[case]
    log(f"decode 32768-token chunks mode {mode} {case}")
    adamas.set_decode_mode(mode)
    assert adamas.decode_chunk_tokens(w.batch, w.hq, w.hkv, w.n_ctx, w.budget,
                                      w.head_dim) == 32768
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    ws = adamas.Workspace(DEV)
    idx = torch.empty((w.batch, w.hq, w.budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                             idx_out=idx, ws=ws, n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any(), "control bytes or status word left set"
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), w.n_ctx, w.budget, 0.0,
                                      n_sink, n_recent)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, case)


# ------------------------- one chunk per KV head (selection = its candidates)
# Contexts of at most one chunk: the chunk workgroup's candidates are the
# selection, so it attends over them directly (fused attention) or writes the
# index rows for the attention launch.  Heads of one, two, three and eight
# query rows, budgets at the fused limit and beyond the context, a single
# row, always-kept tokens, a batch.
_SOLO_CASES = {
    "mha-f32-d64-777-b512": (synth.TINY.replace(hq=2, hkv=2, n_ctx=777, cap=800,
                                                budget=512), 0, 0),
    "gqa2-bf16-1000-b256": (synth.LLAMA32_GQA_1M.replace(hq=2, hkv=1, n_ctx=1000, cap=1000,
                                                         budget=256), 0, 0),
    "gqa2-bf16-1-b64": (synth.LLAMA32_GQA_1M.replace(hq=4, hkv=2, n_ctx=1, cap=8, budget=64),
                        0, 0),
    "gqa2-f32-d64-keep": (synth.TINY.replace(hq=6, hkv=3, n_ctx=1024, cap=1024, budget=100),
                          4, 16),
    "mha-bf16-batch2-keep": (synth.LLAMA2_32K.replace(batch=2, hq=3, hkv=3, n_ctx=1023,
                                                      cap=1030, budget=64), 1, 100),
    "gqa2-d256-bf16-1024-b200": (synth.LLAMA2_32K.replace(hq=4, hkv=2, head_dim=256, n_ctx=1024,
                                                          cap=1024, budget=200), 0, 0),
    # selections attended in a second launch (more than two 256-row batches
    # per KV head): the chunk workgroup writes the index rows itself
    "mha-bf16-1024-b700": (synth.LLAMA2_32K.replace(hq=2, hkv=2, n_ctx=1024, cap=1024,
                                                    budget=700), 0, 0),
    "gqa3-bf16-999-b256-keep": (synth.LLAMA32_GQA_1M.replace(hq=6, hkv=2, n_ctx=999, cap=1000,
                                                             budget=256), 2, 30),
    "gqa8-f32-d64-1000-b64": (synth.TINY.replace(hq=8, hkv=1, n_ctx=1000, cap=1000, budget=64),
                              0, 0),
    "gqa8-bf16-600-b2048": (synth.LLAMA32_GQA_1M.replace(hq=8, hkv=1, n_ctx=600, cap=600,
                                                         budget=2048), 0, 0),
}


@pytest.mark.parametrize("mode", [adamas.DECODE_AUTO, adamas.DECODE_LAST_ARRIVAL,
                                  adamas.DECODE_GROUP_WAIT, adamas.DECODE_SPLIT])
@pytest.mark.parametrize("case", sorted(_SOLO_CASES))
def test_decode_single_chunk(ora, restore_mode, mode, case):
    w, n_sink, n_recent = _SOLO_CASES[case]
    log(f"decode single chunk mode {mode} {case}")
    adamas.set_decode_mode(mode)
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    ws = adamas.Workspace(DEV)
    idx = torch.empty((w.batch, w.hq, w.budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                             idx_out=idx, ws=ws, n_sink=n_sink, n_recent=n_recent)
    out_noidx = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                                   ws=ws, n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any(), "control bytes or status word left set"
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), w.n_ctx, w.budget, 0.0,
                                      n_sink, n_recent)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, case)
    assert torch.equal(out, out_noidx)


# --------------------------------------- rotation switched off (ablation)
@pytest.fixture
def restore_rotation():
    yield
    adamas.set_rotation(True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_encode_without_rotation(ora, restore_rotation, d, dt):
    adamas.set_rotation(False)
    x = synth.random_values((2, 3, 777, d), _dt(dt), seed=31, device=DEV)
    codes = torch.zeros((2, 3, 777, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(x, codes)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ora.encode_keys(host(x), rotate=False))


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
                                  adamas.DECODE_SPLIT])
def test_decode_without_rotation(ora, restore_rotation, restore_mode, mode):
    adamas.set_rotation(False)
    adamas.set_decode_mode(mode)
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=20000, cap=20000, budget=256)
    lay = synth.make_layer(w, 2, DEV)
    codes = torch.zeros((1, 4, 20000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((1, 4, 256), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 20000, 256, idx_out=idx)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k, rotate=False)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 20000, 256, rotate=False)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, "no rotation")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_encode_f16_rotation(ora, restore_rotation, d, dt):
    adamas.set_rotation(adamas.ROTATE_F16)
    rows = [synth.random_values((1, 2, 500, d), _dt(dt), seed=41, device=DEV, scale=4.0)]
    # exact ties and sums that round in binary16
    ints = synth.integer_values((1, 2, 100, d), -9, 9, seed=3)
    rows.append(torch.from_numpy(ints.astype(np.float32) * np.float32(7.0)).to(DEV).to(_dt(dt)))
    x = torch.cat(rows, dim=2).contiguous()
    codes = torch.zeros((1, 2, 600, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(x, codes)
    torch.cuda.synchronize()
    ref = ora.encode_keys(host(x), rotate=2)
    assert np.array_equal(codes.cpu().numpy(), ref)
    # and the binary16 codes do differ from the binary32 ones somewhere
    assert not np.array_equal(ref, ora.encode_keys(host(x)))


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
                                  adamas.DECODE_SPLIT])
def test_decode_f16_rotation(ora, restore_rotation, restore_mode, mode):
    adamas.set_rotation(adamas.ROTATE_F16)
    adamas.set_decode_mode(mode)
    w = synth.LLAMA2_32K.replace(hq=8, hkv=4, n_ctx=20000, cap=20000, budget=256)
    lay = synth.make_layer(w, 3, DEV)
    codes = torch.zeros((1, 4, 20000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((1, 8, 256), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 20000, 256, idx_out=idx)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k, rotate=2)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 20000, 256, rotate=2)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, "f16 rotation")


def test_quality_dense_reference_matches_oracle(ora):
    # the sweep's dense reference is exact attention over every row
    from quality import dense_attention
    w = synth.LLAMA32_GQA_1M.replace(hq=6, hkv=2, n_ctx=2000, cap=2000)
    lay = synth.make_layer(w, 0, DEV)
    got = dense_attention(lay["q"], lay["k"], lay["v"])
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    idx = np.tile(np.arange(2000, dtype=np.int32), (1, 6, 1))
    _, ref64 = ora.sparse_attend(q, k, v, idx)
    e = float(np.linalg.norm(got.cpu().double().numpy() - ref64) / np.linalg.norm(ref64))
    assert e < 1e-5


# ------------------------------------------------ group-wait give-up path
def test_group_wait_give_up_is_reported(ora, restore_mode):
    """A group wait bounded at 0 polls gives up at once wherever its group is
    not complete yet.  Forced from the host this way, every workgroup still
    runs to its end: the call's status word is set, its arrival counters are
    left zero, and after re-arming the word the next call (default bound) is
    correct and reports nothing."""
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=20000, cap=20000, budget=256)
    adamas.set_decode_mode(adamas.DECODE_GROUP_WAIT)
    assert adamas.decode_path(1, 4, 4, w.n_ctx, w.budget, 128) == adamas.DECODE_GROUP_WAIT
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((1, 4, w.cap, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    ws = adamas.Workspace(DEV)
    try:
        adamas.set_wait_polls(0)
        log("group wait with a bound of 0 polls")
        adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget, ws=ws)
        torch.cuda.synchronize()
    finally:
        adamas.set_wait_polls(adamas.DEFAULT_WAIT_POLLS)
    assert ws.status() != 0, "no give-up reported"
    assert ws.control_bytes_clear(), "arrival counters left set after a give-up"
    with pytest.raises(adamas.GroupWaitGaveUp):
        ws.check()                                   # raises and re-arms
    assert ws.status() == 0
    idx = torch.empty((1, 4, w.budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget, idx_out=idx,
                             ws=ws, check=True)
    assert ws.status() == 0 and ws.control_bytes_clear()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), w.n_ctx, w.budget)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, "after a give-up")


@pytest.mark.parametrize("hq,hkv,n,budget,key_bytes", [(6, 2, 20000, 256, 2),
                                                       (24, 8, 300000, 1024, 1)])
def test_group_wait_give_up_grouped_heads(restore_mode, hq, hkv, n, budget, key_bytes):
    """The same give-up for grouped heads (16-bit and one-byte keys): the
    status word is set, the control bytes are left zero, and a re-armed
    workspace then gives the same result as a fresh one."""
    w = synth.LLAMA32_GQA_1M.replace(hq=hq, hkv=hkv, n_ctx=n, cap=n, budget=budget)
    adamas.set_decode_mode(adamas.DECODE_GROUP_WAIT)
    assert adamas.decode_path(1, hq, hkv, n, budget, 128) == adamas.DECODE_GROUP_WAIT
    assert adamas.decode_key_bytes(1, hq, hkv, n, budget, 128) == key_bytes
    log(f"group wait give-up, {hq}/{hkv} heads x {n} tokens, {key_bytes}-byte keys")
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((1, hkv, n, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    ws = adamas.Workspace(DEV)
    try:
        adamas.set_wait_polls(0)
        adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, budget, ws=ws)
        torch.cuda.synchronize()
    finally:
        adamas.set_wait_polls(adamas.DEFAULT_WAIT_POLLS)
    assert ws.status() != 0, "no give-up reported"
    assert ws.control_bytes_clear(), "arrival counters left set after a give-up"
    with pytest.raises(adamas.GroupWaitGaveUp):
        ws.check()
    idx = torch.empty((1, hq, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, budget, idx_out=idx, ws=ws,
                             check=True)
    idx2 = torch.empty_like(idx)
    out2 = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, budget, idx_out=idx2,
                              ws=adamas.Workspace(DEV), check=True)
    torch.cuda.synchronize()
    assert ws.status() == 0 and ws.control_bytes_clear()
    assert torch.equal(idx, idx2) and torch.equal(out, out2)

