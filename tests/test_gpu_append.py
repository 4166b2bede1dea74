"""GPU parity of adamas_decode_append_step against the oracle: ragged batches
(per-sequence lengths read from device memory), the new token appended to the
K, V and code caches inside the step, GQA, large budgets (separate attention
launch), the always-kept set, clamped lengths, and replay from a HIP graph
with the lengths advanced between replays.

Every case checks the selection and the three caches bit for bit and the
output against the oracle's binary64 result within the dtype's tolerance."""
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
    adamas.load()


def _inputs(w, seed, near_query=True):
    """Caches filled to cap, their codes, and a new key/value per (b, KV head).
    With near_query, even-numbered sequences get a new key close to their first
    query head, so the appended row tends to be selected."""
    lay = synth.make_layer(w, 0, DEV, n_ctx=w.cap)
    B, Hkv, d, G = w.batch, w.hkv, w.head_dim, w.hq // w.hkv
    codes = torch.zeros((B, Hkv, w.cap, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    kn = synth.random_values((B, Hkv, d), w.torch_dtype, seed, device=DEV)
    vn = synth.random_values((B, Hkv, d), w.torch_dtype, seed + 1, device=DEV)
    if near_query:
        for b in range(0, B, 2):
            kn[b] = (lay["q"][b, ::G].float() + 0.05 * kn[b].float()).to(w.torch_dtype)
    return lay, codes, kn, vn


def _run(ora, w, lens, max_len, budget, append=True, n_sink=0, n_recent=0, seed=500, alpha=None):
    adamas.set_bucket_alpha(alpha)
    try:
        return _run_rule(ora, w, lens, max_len, budget, append, n_sink, n_recent, seed, alpha)
    finally:
        adamas.set_bucket_alpha(None)


def _run_rule(ora, w, lens, max_len, budget, append, n_sink, n_recent, seed, alpha):
    lay, codes, kn, vn = _inputs(w, seed)
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k, alpha=alpha)
    assert np.array_equal(codes.cpu().numpy(), oc), "code cache differs before the step"
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = torch.full((w.batch, w.hq, budget), -7, dtype=torch.int32, device=DEV)
    out = adamas.decode_append_step(lay["q"], lay["k"], lay["v"], codes, lens_d, max_len, budget,
                                    k_new=kn if append else None, v_new=vn if append else None,
                                    idx_out=idx, n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    kn_h, vn_h = (host(t) for t in (kn, vn))
    oout, o64, oidx, ok, ov, ocd = ora.decode_append_step(
        q, k, v, oc, np.array(lens), max_len, budget, kn_h if append else None,
        vn_h if append else None, n_sink=n_sink, n_recent=n_recent, alpha=alpha)
    assert torch.equal(lens_d.cpu(), torch.tensor(lens, dtype=torch.int32)), "lens written"
    assert np.array_equal(host(lay["k"]), ok), "K cache differs"
    assert np.array_equal(host(lay["v"]), ov), "V cache differs"
    assert np.array_equal(codes.cpu().numpy(), ocd), "code cache differs"
    got = idx.cpu().numpy()
    for b in range(w.batch):
        assert np.array_equal(got[b], oidx[b]), f"selection of sequence {b} differs"
    check_out(ora, out, q, ok, ov, oidx, oout, o64,
              f"append={append} lens={lens} max_len={max_len} budget={budget} alpha={alpha}")
    return got, lay, kn


@pytest.mark.parametrize("append", [True, False])
def test_ragged_mha(ora, append):
    log(f"ragged MHA batch, append={append}")
    w = synth.LLAMA2_32K.replace(batch=6, hq=4, hkv=4, n_ctx=9001, cap=9001, budget=256)
    _run(ora, w, [1, 700, 0, 4097, 9000, 4096], 9001, 256, append)


def test_append_at_chunk_boundaries(ora):
    log("append at and around power-of-two boundaries")
    w = synth.LLAMA2_32K.replace(batch=12, hq=2, hkv=2, n_ctx=4098, cap=4098, budget=64)
    lens = [63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 4095, 4096, 4097]
    idx, _, _ = _run(ora, w, lens, 4098, 64)
    for b in range(0, 12, 2):
        assert (idx[b, 0] == lens[b]).any(), "the near-query new key was not selected"


@pytest.mark.parametrize("hq,hkv,dt,d", [(24, 8, "bf16", 128), (6, 2, "f32", 64), (8, 1, "bf16", 128)])
def test_append_gqa(ora, hq, hkv, dt, d):
    log(f"append GQA hq={hq} hkv={hkv} {dt} d={d}")
    w = synth.LLAMA32_GQA_1M.replace(batch=3, hq=hq, hkv=hkv, head_dim=d, dtype=dt, n_ctx=5000,
                                     cap=5000, budget=128)
    _run(ora, w, [4999, 17, 2500], 5000, 128)


def test_append_bucket_alpha(ora):
    log("append with per-head-group bucketing thresholds")
    w = synth.LLAMA32_GQA_1M.replace(batch=3, hq=8, hkv=4, n_ctx=5000, cap=5000, budget=128)
    _run(ora, w, [4999, 17, 2500], 5000, 128, alpha=[0.25, 0.75, 0.4])


@pytest.mark.parametrize("budget", [2048, 20000])
def test_append_large_budget(ora, budget):
    log(f"append with budget {budget} (attention in its own launch)")
    w = synth.LLAMA2_32K.replace(batch=3, hq=4, hkv=4, n_ctx=6001, cap=6001, budget=budget)
    _run(ora, w, [100, 3000, 6000], 6001, budget)


def test_append_keep_set(ora):
    log("append with sinks and a recent window")
    w = synth.LLAMA2_32K.replace(batch=4, hq=4, hkv=4, n_ctx=7000, cap=7000, budget=128)
    idx, _, _ = _run(ora, w, [6999, 40, 3000, 0], 7000, 128, n_sink=4, n_recent=64)
    for b, L in enumerate([6999, 40, 3000, 0]):
        assert (idx[b] == L).any(axis=-1).all(), "the new token is in the recent window"


def test_lengths_clamped(ora):
    log("lengths beyond max_len or negative are clamped")
    w = synth.LLAMA2_32K.replace(batch=3, hq=2, hkv=2, n_ctx=3000, cap=3500, budget=64)
    _run(ora, w, [-5, 100000, 2999], 3000, 64)
    _run(ora, w, [-5, 100000, 2999], 3000, 64, append=False)


def test_mode_setting_ignored(ora):
    log("the append step takes the last-arrival schedule whatever the mode")
    w = synth.LLAMA2_32K.replace(batch=2, hq=4, hkv=4, n_ctx=5000, cap=5000, budget=256)
    try:
        adamas.set_decode_mode(adamas.DECODE_GROUP_WAIT)
        _run(ora, w, [4999, 1234], 5000, 256)
    finally:
        adamas.set_decode_mode(adamas.DECODE_AUTO)


def test_graph_replay_advances_lengths(ora):
    log("HIP graph: one captured append step replayed 4 times, lens advanced between replays")
    w = synth.LLAMA2_32K.replace(batch=3, hq=4, hkv=4, n_ctx=3000, cap=3000, budget=64)
    B, Hq, Hkv, d, dt = w.batch, w.hq, w.hkv, w.head_dim, w.torch_dtype
    lay, codes, _, _ = _inputs(w, 700)
    q_s = lay["q"].clone()
    kn_s = torch.empty((B, Hkv, d), dtype=dt, device=DEV)
    vn_s = torch.empty_like(kn_s)
    lens0 = [1000, 2500, 0]
    lens_d = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q_s)
    idx = torch.empty((B, Hq, 64), dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream(DEV)
    ws = adamas.Workspace(DEV)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, 3000, 64, d))
    k_h, v_h, c_h = host(lay["k"]), host(lay["v"]), codes.cpu().numpy()
    assert np.array_equal(c_h, ora.encode_keys(k_h))

    def step():
        adamas.decode_append_step(q_s, lay["k"], lay["v"], codes, lens_d, 3000, 64, k_new=kn_s,
                                  v_new=vn_s, out=out, idx_out=idx, ws=ws, stream=s)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        q_new = synth.random_values((B, Hq, d), dt, 800 + rep, device=DEV)
        kn = synth.random_values((B, Hkv, d), dt, 900 + rep, device=DEV)
        vn = synth.random_values((B, Hkv, d), dt, 950 + rep, device=DEV)
        q_s.copy_(q_new)
        kn_s.copy_(kn)
        vn_s.copy_(vn)
        out.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lens = [L + rep for L in lens0]
        oout, o64, oidx, k_h, v_h, c_h = ora.decode_append_step(
            host(q_new), k_h, v_h, c_h, np.array(lens), 3000, 64, host(kn), host(vn))
        assert np.array_equal(idx.cpu().numpy(), oidx), f"replay {rep}: selection differs"
        check_out(ora, out, host(q_new), k_h, v_h, oidx, oout, o64, f"replay {rep}")
        assert np.array_equal(host(lay["k"]), k_h) and np.array_equal(codes.cpu().numpy(), c_h)
        with torch.cuda.stream(s):
            lens_d.add_(1)
        torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any()


def test_append_many_rounds(ora):
    log("append step over 256 KV heads x 2 chunks (two workgroups per compute unit)")
    w = synth.LLAMA2_32K.replace(batch=8, hq=32, hkv=32, n_ctx=20001, cap=20001, budget=256)
    _run(ora, w, [20000, 9000, 16384, 1, 0, 12345, 16383, 19999], 20001, 256)


def test_append_long_chunks(ora):
    log("append step over 256 KV heads x 2 chunks of up to 32768 tokens (two per compute unit)")
    w = synth.LLAMA2_32K.replace(batch=8, hq=32, hkv=32, n_ctx=40001, cap=40001, budget=256)
    assert adamas.decode_chunk_tokens(8, 32, 32, 40001, 256, 128) == 32768
    _run(ora, w, [40000, 9000, 32768, 1, 0, 32767, 16384, 39999], 40001, 256)
