"""GPU parity of the per-head-group bucketing thresholds (the §3.2 tuning
list of the ADAMAS article: groups of attention heads bucket with their own
thresholds, here -alpha*a, 0, +alpha*a with alpha taken per KV head from a
table): the key codes bit for bit, the selection bit for bit and the output
within the dtype's bound, under every decode schedule."""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import check_out, host, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _restore():
    adamas.load()
    yield
    adamas.set_bucket_alpha(None)
    adamas.set_decode_mode(adamas.DECODE_AUTO)
    adamas.set_rotation(True)


def _dt(s):
    return torch.bfloat16 if s == "bf16" else torch.float32


@pytest.mark.parametrize("rotate", [1, 2])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_encode_bucket_alpha(ora, d, dt, rotate):
    table = [0.25, 0.75, 0.5, 0.3, 0.0, 1.2]
    log(f"encode d={d} {dt} rotate={rotate} alpha={table}")
    adamas.set_bucket_alpha(table)
    adamas.set_rotation(rotate)
    x = synth.random_values((2, 7, 611, d), _dt(dt), seed=61, device=DEV)
    codes = torch.zeros((2, 7, 611, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(x, codes)
    torch.cuda.synchronize()
    ref = ora.encode_keys(host(x), rotate=rotate, alpha=table)
    assert np.array_equal(codes.cpu().numpy(), ref)
    # and the table changes the codes of every head whose alpha is not 0.5
    base = ora.encode_keys(host(x), rotate=rotate)
    for h in range(7):
        same = np.array_equal(ref[:, h], base[:, h])
        assert same == (table[h % 6] == 0.5), f"head {h}"


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
                                  adamas.DECODE_SPLIT])
@pytest.mark.parametrize("rotate", [1, 0])
def test_decode_bucket_alpha_gqa(ora, mode, rotate):
    table = [0.3, 0.7, 0.25]        # 3 entries over 4 KV heads: head 3 takes alpha[0]
    log(f"decode GQA 8/4 mode={mode} rotate={rotate} alpha={table}")
    adamas.set_bucket_alpha(table)
    adamas.set_rotation(rotate)
    adamas.set_decode_mode(mode)
    w = synth.LLAMA32_GQA_1M.replace(hq=8, hkv=4, n_ctx=30001, cap=30001, budget=256)
    lay = synth.make_layer(w, 4, DEV)
    codes = torch.zeros((1, 4, 30001, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((1, 8, 256), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 30001, 256, idx_out=idx)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k, rotate=rotate, alpha=table)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 30001, 256, rotate=rotate, alpha=table)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, f"alpha GQA mode {mode}")


@pytest.mark.parametrize("mode", [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_SPLIT])
def test_decode_bucket_alpha_mha_keep(ora, mode):
    table = [0.0, 0.35, 0.5, 1.0, 0.6, 0.45]
    log(f"decode MHA 6 heads mode={mode} alpha={table} with sinks and a recent window")
    adamas.set_bucket_alpha(table)
    adamas.set_decode_mode(mode)
    w = synth.LLAMA2_32K.replace(batch=2, hq=6, hkv=6, n_ctx=40000, cap=40000, budget=512)
    lay = synth.make_layer(w, 5, DEV)
    codes = torch.zeros((2, 6, 40000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((2, 6, 512), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 40000, 512, idx_out=idx,
                             n_sink=4, n_recent=64)
    torch.cuda.synchronize()
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k, alpha=table)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 40000, 512, n_sink=4, n_recent=64,
                                      alpha=table)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, f"alpha MHA keep mode {mode}")


def test_alpha_half_table_is_the_fixed_rule(ora):
    log("a table of 0.5s gives the fixed rule's codes and selection")
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=9000, cap=9000, budget=128)
    lay = synth.make_layer(w, 6, DEV)
    res = []
    for table in (None, [0.5, 0.5]):
        adamas.set_bucket_alpha(table)
        codes = torch.zeros((1, 4, 9000, 32), dtype=torch.uint8, device=DEV)
        adamas.encode_keys(lay["k"], codes)
        idx = torch.empty((1, 4, 128), dtype=torch.int32, device=DEV)
        out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 9000, 128, idx_out=idx)
        torch.cuda.synchronize()
        res.append((codes.cpu(), idx.cpu(), out.cpu()))
    assert all(torch.equal(a, b) for a, b in zip(*res))


def test_captured_graph_keeps_its_table(ora):
    """A launch takes the bucketing table by value: a graph captured under one
    table replays with it after the process-wide table has changed."""
    log("graph captured under one alpha table, replayed under another")
    w = synth.LLAMA32_GQA_1M.replace(hq=6, hkv=2, n_ctx=12000, cap=12000, budget=128)
    lay = synth.make_layer(w, 8, DEV)
    table = [0.3, 0.65]
    adamas.set_bucket_alpha(table)
    codes = torch.zeros((1, 2, 12000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    s = torch.cuda.Stream(DEV)
    ws = adamas.Workspace(DEV)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, 1, 6, 2, 12000, 128, 128))
    idx = torch.empty((1, 6, 128), dtype=torch.int32, device=DEV)
    out = torch.empty_like(lay["q"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 12000, 128, out=out, idx_out=idx,
                           ws=ws, stream=s)   # warm-up outside the capture
        with torch.cuda.graph(g, stream=s):
            adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 12000, 128, out=out,
                               idx_out=idx, ws=ws, stream=s)
    torch.cuda.synchronize()
    adamas.set_bucket_alpha([0.9, 0.1])
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k, alpha=table)
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 12000, 128, alpha=table)
    for rep in range(3):
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), oidx), f"replay {rep}"
        check_out(ora, out, q, k, v, oidx, oout, o64, f"graph replay {rep}")
