"""GPU parity of adamas_encode_keys_paged: a block of keys encoded straight
into pools of pages (shuffled pool order, a start inside a page, several
pages per sequence, every head_dim and element type) must put the oracle's
code row of every token, and its raw row, at the pool row its page table
names, bit for bit, and touch no other byte of the pools; a token whose table
entry is out of range is not stored.  Also: a decode over pools filled this
way selects exactly what it selects over pools filled page by page with
adamas_encode_keys."""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import host, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FILL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    adamas.load()


def _expected(pool_bits, rows, table, pos, n, P, fill_bad):
    """pool_bits [n_pages][H][P][w] with rows [B][H][n][w] placed per table."""
    B = rows.shape[0]
    for b in range(B):
        t = pos
        while t < pos + n:
            i, off = divmod(t, P)
            m = min(P - off, pos + n - t)
            pg = int(table[b, i])
            if 0 <= pg < pool_bits.shape[0]:
                pool_bits[pg, :, off:off + m] = rows[b, :, t - pos:t - pos + m]
            else:
                fill_bad.append((b, i))
            t += m
    return pool_bits


@pytest.mark.parametrize("dtype,d,pos,n,P,B,H", [
    (torch.bfloat16, 128, 500, 3000, 1024, 2, 4),
    (torch.float32, 64, 0, 2048, 1024, 3, 2),
    (torch.bfloat16, 256, 1000, 5000, 2048, 2, 2),
    (torch.bfloat16, 128, 4095, 1, 1024, 1, 8),     # one token, last row of a page
    (torch.float32, 128, 1024, 4096, 4096, 2, 3),   # page-aligned start, one page
])
def test_encode_paged_matches_oracle(ora, dtype, d, pos, n, P, B, H):
    log(f"encode_paged dtype={dtype} d={d} pos={pos} n={n} P={P} B={B} H={H}")
    x = synth.random_values((B, H, n, d), dtype, seed=pos + n + d, device=DEV)
    per = (pos + n + P - 1) // P
    n_pages = B * per + 3
    rng = np.random.default_rng(n + P)
    table = np.full((B, per + 1), -1, np.int32)
    table[:, :per] = rng.permutation(n_pages)[:B * per].reshape(B, per)
    if B > 1 and per > 1:
        table[1, per - 1] = n_pages + 7               # out of range: those tokens not stored
    code_pool = torch.full((n_pages, H, P, d // 4), FILL, dtype=torch.uint8, device=DEV)
    x_pool = torch.full((n_pages, H, P, d), 3.0, dtype=dtype, device=DEV)
    x_pool_bits0 = host(x_pool)
    adamas.encode_keys_paged(x, code_pool, torch.from_numpy(table).to(DEV), pos=pos,
                             x_pool=x_pool)
    torch.cuda.synchronize()
    codes_ref = ora.encode_keys(host(x))               # [B][H][n][d/4]
    skipped = []
    want_codes = _expected(np.full((n_pages, H, P, d // 4), FILL, np.uint8), codes_ref, table,
                           pos, n, P, skipped)
    want_x = _expected(x_pool_bits0.copy(), host(x), table, pos, n, P, [])
    assert np.array_equal(code_pool.cpu().numpy(), want_codes)
    assert np.array_equal(host(x_pool), want_x)
    assert (B > 1 and per > 1) == bool(skipped)


def test_paged_pools_from_one_call_decode_alike(ora):
    """A 16-bit-key MHA decode over pools filled by one paged encode call
    gives the same indices and output as over pools filled page by page."""
    w = synth.BATCH16_64K.replace(batch=2, hq=4, hkv=4, n_ctx=5000, cap=6144, budget=64)
    P, per = 1024, 6
    lay = synth.make_layer(w, 3, DEV)
    n_pages = w.batch * per + 2
    table = np.random.default_rng(9).permutation(n_pages)[:w.batch * per].reshape(
        w.batch, per).astype(np.int32)
    t_dev = torch.from_numpy(table).to(DEV)
    pools = []
    for mode in ("one call", "page by page"):
        kp = torch.zeros((n_pages, w.hkv, P, w.head_dim), dtype=w.torch_dtype, device=DEV)
        vp = torch.zeros_like(kp)
        cp = torch.zeros((n_pages, w.hkv, P, w.head_dim // 4), dtype=torch.uint8, device=DEV)
        if mode == "one call":
            adamas.encode_keys_paged(lay["k"][:, :, :per * P].contiguous(), cp, t_dev, x_pool=kp)
        else:
            for b in range(w.batch):
                for i in range(per):
                    pg = int(table[b, i])
                    adamas.encode_keys(lay["k"][b:b + 1, :, i * P:(i + 1) * P].contiguous(),
                                       cp[pg:pg + 1], x_copy=kp[pg:pg + 1])
        for b in range(w.batch):
            for i in range(per):
                vp[int(table[b, i])] = lay["v"][b, :, i * P:(i + 1) * P]
        pools.append((kp, vp, cp))
    assert torch.equal(pools[0][0], pools[1][0]) and torch.equal(pools[0][2], pools[1][2])
    outs = []
    lens = torch.full((w.batch,), w.n_ctx, dtype=torch.int32, device=DEV)
    for kp, vp, cp in pools:
        idx = torch.empty((w.batch, w.hq, w.budget), dtype=torch.int32, device=DEV)
        out = adamas.decode_paged_step(lay["q"], kp, vp, cp, t_dev, lens, w.n_ctx, w.budget,
                                       idx_out=idx)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), out.cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_encode_paged_graph_replay(ora):
    """Captured once in a HIP graph and replayed over new key values (the same
    buffers refilled between replays, with eager work in between): every
    replay leaves the oracle's rows in the pages."""
    B, H, n, d, P, pos = 2, 4, 1500, 128, 1024, 700
    per = (pos + n + P - 1) // P
    n_pages = B * per + 1
    table = torch.from_numpy(
        np.random.default_rng(4).permutation(n_pages)[:B * per].reshape(B, per).astype(np.int32)
    ).to(DEV)
    x = torch.empty((B, H, n, d), dtype=torch.bfloat16, device=DEV)
    code_pool = torch.zeros((n_pages, H, P, d // 4), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream(DEV)
    x.copy_(synth.random_values(x.shape, x.dtype, seed=1, device=DEV))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        adamas.encode_keys_paged(x, code_pool, table, pos=pos, stream=s)
    tab = table.cpu().numpy()
    for rep in range(3):
        log(f"encode_paged graph replay {rep}")
        x.copy_(synth.random_values(x.shape, x.dtype, seed=10 + rep, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = _expected(np.zeros((n_pages, H, P, d // 4), np.uint8), ora.encode_keys(host(x)),
                         tab, pos, n, P, [])
        assert np.array_equal(code_pool.cpu().numpy(), want)
