"""GPU parity of adamas_decode_paged_step against the oracle: K, V and code
caches kept as pools of fixed-size pages shared by the sequences of a batch,
each sequence's logical pages mapped to pool pages by a page table (shuffled
here), with ragged lengths, the new token appended into its page, GQA, fp32,
large budgets (paged attention launch), larger pages, two workgroups per
compute unit, and replay from a HIP graph across a page boundary.

The pools are filled the documented way: adamas_encode_keys on each pool page
(batch 1, heads Hkv, cap page_size), copying the K rows with x_copy.  Every
case checks the selection and the three pools bit for bit and the output
against the oracle's binary64 result within the dtype's tolerance."""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import check_out_paged, host, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    adamas.load()


def _pools(w, P, pages_per_seq, spare, seed):
    """Pools holding every sequence's pages_per_seq pages in shuffled pool
    order (plus `spare` unused pool pages), and the page table; table entries
    past a sequence's pages are -1 or out of range (never looked up)."""
    B, Hkv, d, dt = w.batch, w.hkv, w.head_dim, w.torch_dtype
    cap = pages_per_seq * P
    lay = synth.make_layer(w.replace(n_ctx=cap, cap=cap), 0, DEV)
    n_pages = B * pages_per_seq + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)[:B * pages_per_seq].reshape(B, pages_per_seq)
    k_pool = torch.zeros((n_pages, Hkv, P, d), dtype=dt, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    c_pool = torch.zeros((n_pages, Hkv, P, d // 4), dtype=torch.uint8, device=DEV)
    for b in range(B):
        for i in range(pages_per_seq):
            pg = int(perm[b, i])
            src = lay["k"][b:b + 1, :, i * P:(i + 1) * P].contiguous()
            adamas.encode_keys(src, c_pool[pg:pg + 1], x_copy=k_pool[pg:pg + 1])
            v_pool[pg] = lay["v"][b, :, i * P:(i + 1) * P]
    max_pages = pages_per_seq + 2
    table = np.full((B, max_pages), -1, np.int32)
    table[:, :pages_per_seq] = perm
    table[:, -1] = 10 ** 6                           # out of range, never reached
    return lay, k_pool, v_pool, c_pool, table


def _run(ora, w, P, pages_per_seq, lens, budget, append=True, n_sink=0, n_recent=0, seed=11,
         alpha=None):
    adamas.set_bucket_alpha(alpha)
    try:
        return _run_rule(ora, w, P, pages_per_seq, lens, budget, append, n_sink, n_recent, seed,
                         alpha)
    finally:
        adamas.set_bucket_alpha(None)


def _run_rule(ora, w, P, pages_per_seq, lens, budget, append, n_sink, n_recent, seed, alpha):
    lay, kp, vp, cp, table = _pools(w, P, pages_per_seq, 3, seed)
    B, Hkv, d, dt = w.batch, w.hkv, w.head_dim, w.torch_dtype
    max_len = pages_per_seq * P
    kn = synth.random_values((B, Hkv, d), dt, seed + 1, device=DEV)
    vn = synth.random_values((B, Hkv, d), dt, seed + 2, device=DEV)
    for b in range(0, B, 2):                          # some new keys near a query head
        kn[b] = (lay["q"][b, ::w.hq // w.hkv].float() + 0.05 * kn[b].float()).to(dt)
    q = host(lay["q"])
    kp_h, vp_h = host(kp), host(vp)
    # the oracle's own codes of the pages in use (spare pages stay zero)
    cp_h = np.zeros(tuple(cp.shape), np.uint8)
    used = np.unique(table[(table >= 0) & (table < cp.shape[0])])
    cp_h[used] = ora.encode_keys(kp_h[used], alpha=alpha)
    assert np.array_equal(cp.cpu().numpy(), cp_h), "code pool differs before the step"
    table_d = torch.from_numpy(table).to(DEV)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = torch.full((B, w.hq, budget), -7, dtype=torch.int32, device=DEV)
    out = adamas.decode_paged_step(lay["q"], kp, vp, cp, table_d, lens_d, max_len, budget,
                                   k_new=kn if append else None, v_new=vn if append else None,
                                   idx_out=idx, n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    oout, o64, oidx, okp, ovp, ocp = ora.decode_paged_step(
        q, kp_h, vp_h, cp_h, table, np.array(lens), max_len, budget,
        host(kn) if append else None, host(vn) if append else None, n_sink=n_sink,
        n_recent=n_recent, alpha=alpha)
    assert np.array_equal(host(kp), okp), "K pool differs"
    assert np.array_equal(host(vp), ovp), "V pool differs"
    assert np.array_equal(cp.cpu().numpy(), ocp), "code pool differs"
    got = idx.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], oidx[b]), f"selection of sequence {b} differs"
    check_out_paged(ora, out, q, okp, ovp, table, oidx, oout, o64,
                    f"P={P} lens={lens} budget={budget} append={append}")
    return got


@pytest.mark.parametrize("append", [True, False])
def test_paged_ragged_mha(ora, append):
    log(f"paged MHA, append={append}")
    w = synth.LLAMA2_32K.replace(batch=5, hq=4, hkv=4)
    _run(ora, w, 1024, 5, [5119, 1023, 1024, 0, 3000], 256, append)


def test_paged_gqa_fp32_d64(ora):
    log("paged GQA 6/2 heads, fp32, d=64")
    w = synth.LLAMA32_GQA_1M.replace(batch=3, hq=6, hkv=2, head_dim=64, dtype="f32")
    _run(ora, w, 1024, 4, [4095, 2047, 100], 128)


def test_paged_bucket_alpha(ora):
    log("paged GQA with per-head-group bucketing thresholds")
    w = synth.LLAMA32_GQA_1M.replace(batch=3, hq=6, hkv=2, head_dim=128, dtype="bf16")
    _run(ora, w, 1024, 3, [3071, 1000, 5], 128, alpha=[0.3, 0.65])


def test_paged_large_budget(ora):
    log("paged, budget 2048 (attention in its own launch)")
    w = synth.LLAMA2_32K.replace(batch=3, hq=4, hkv=4)
    _run(ora, w, 1024, 4, [4000, 1024, 3071], 2048)


def test_paged_page_4096_keep(ora):
    log("paged with 4096-token pages, sinks and a recent window")
    w = synth.LLAMA2_32K.replace(batch=3, hq=4, hkv=4)
    idx = _run(ora, w, 4096, 3, [12287, 4095, 5000], 128, n_sink=4, n_recent=32)
    for b, L in enumerate([12287, 4095, 5000]):
        assert (idx[b] == L).any(axis=-1).all()


def test_paged_many_rounds(ora):
    log("paged over 256 KV heads x 2 chunks (two workgroups per compute unit)")
    w = synth.LLAMA2_32K.replace(batch=8, hq=32, hkv=32)
    _run(ora, w, 1024, 20, [20479, 9000, 16384, 1, 0, 12345, 16383, 20000], 256)


def test_paged_graph_replay_across_page_boundary(ora):
    log("HIP graph: paged append step replayed 4 times, lens advancing across a page boundary")
    w = synth.LLAMA2_32K.replace(batch=2, hq=4, hkv=4)
    B, Hq, Hkv, d, dt, P = w.batch, w.hq, w.hkv, w.head_dim, w.torch_dtype, 1024
    lay, kp, vp, cp, table = _pools(w, P, 3, 1, 21)
    table_d = torch.from_numpy(table).to(DEV)
    lens0 = [1022, 2000]
    lens_d = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    q_s = lay["q"].clone()
    kn_s = torch.empty((B, Hkv, d), dtype=dt, device=DEV)
    vn_s = torch.empty_like(kn_s)
    out = torch.empty_like(q_s)
    idx = torch.empty((B, Hq, 64), dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream(DEV)
    ws = adamas.Workspace(DEV)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, B, Hq, Hkv, 3 * P, 64, d))
    kp_h, vp_h = host(kp), host(vp)
    cp_h = np.zeros(tuple(cp.shape), np.uint8)
    used = np.unique(table[(table >= 0) & (table < cp.shape[0])])
    cp_h[used] = ora.encode_keys(kp_h[used])
    assert np.array_equal(cp.cpu().numpy(), cp_h), "code pool differs before the steps"

    def step():
        adamas.decode_paged_step(q_s, kp, vp, cp, table_d, lens_d, 3 * P, 64, k_new=kn_s,
                                 v_new=vn_s, out=out, idx_out=idx, ws=ws, stream=s)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        q_new = synth.random_values((B, Hq, d), dt, 300 + rep, device=DEV)
        kn = synth.random_values((B, Hkv, d), dt, 400 + rep, device=DEV)
        vn = synth.random_values((B, Hkv, d), dt, 500 + rep, device=DEV)
        q_s.copy_(q_new)
        kn_s.copy_(kn)
        vn_s.copy_(vn)
        out.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lens = [L + rep for L in lens0]
        oout, o64, oidx, kp_h, vp_h, cp_h = ora.decode_paged_step(
            host(q_new), kp_h, vp_h, cp_h, table, np.array(lens), 3 * P, 64, host(kn), host(vn))
        assert np.array_equal(idx.cpu().numpy(), oidx), f"replay {rep}: selection differs"
        check_out_paged(ora, out, host(q_new), kp_h, vp_h, table, oidx, oout, o64,
                        f"replay {rep}")
        assert np.array_equal(host(kp), kp_h) and np.array_equal(cp.cpu().numpy(), cp_h)
        with torch.cuda.stream(s):
            lens_d.add_(1)
        torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any()
