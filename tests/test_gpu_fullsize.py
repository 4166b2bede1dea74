"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (fused decode step, one call per layer).

The GPU always runs the whole workload; the oracle checks every head of the
layers it is given (MHA workloads) or a sampled subset of sequences (the
batch-16 workload: the oracle's per-sequence computations are independent,
so slicing the batch is exact).  Codes and selected indices must be
bit-exact; outputs within the relative error bound of the output type.
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


def _run_layer(w, layer, budget):
    lay = synth.make_layer(w, layer, DEV)
    codes = torch.zeros((w.batch, w.hkv, lay["cap"], w.head_dim // 4), dtype=torch.uint8,
                        device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.empty((w.batch, w.hq, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, budget, idx_out=idx)
    torch.cuda.synchronize()
    return lay, codes, idx, out


def _check(ora, w, lay, codes, idx, out, budget, batch_rows=None):
    sl = slice(None) if batch_rows is None else batch_rows
    q, k, v = (host(lay[x][sl]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k)
    assert np.array_equal(codes[sl].cpu().numpy(), ocodes), "code cache differs"
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, w.n_ctx, budget)
    assert np.array_equal(idx[sl].cpu().numpy(), oidx), "selection differs"
    check_out(ora, out[sl], q, k, v, oidx, oout, o64, f"{w.name} budget {budget}")


def test_llama2_32k_full(ora):
    log("full size: Llama-2-7B-shaped layer, 32 heads x 32768 tokens, budget 256")
    w = synth.LLAMA2_32K
    _check(ora, w, *_run_layer(w, 0, w.budget), w.budget)


@pytest.mark.parametrize("budget", [64, 128, 256, 1024])
def test_llama2_128k_layer_budgets(ora, budget):
    layer = {64: 0, 128: 7, 256: 31, 1024: 16}[budget]
    log(f"full size: 128K-token layer {layer} of the 32-layer stack, budget {budget}")
    w = synth.LLAMA2_128K_32L
    _check(ora, w, *_run_layer(w, layer, budget), budget)


@pytest.mark.parametrize("extra", [0, 1000])
def test_llama2_128k_layer_dense_budget(ora, extra):
    """The article's accuracy policy of dense attention in the last layers
    (§3.2) is a call with a budget >= the context: every row is selected (in
    order, -1 padded beyond the context) and the output is exact attention
    over all 131072 rows."""
    w = synth.LLAMA2_128K_32L
    budget = w.n_ctx + extra
    log(f"full size: 128K-token layer 29 with budget {budget} (dense)")
    lay, codes, idx, out = _run_layer(w, 29, budget)
    want = torch.arange(w.n_ctx, dtype=torch.int32, device=DEV)
    assert torch.equal(idx[..., :w.n_ctx], want.expand(1, w.hq, w.n_ctx))
    assert (idx[..., w.n_ctx:] == -1).all()
    _check(ora, w, lay, codes, idx, out, budget)


def test_llama32_gqa_1m(ora):
    log("full size: GQA 24 q / 8 kv heads x 1,048,576 tokens, budget 1024")
    w = synth.LLAMA32_GQA_1M
    _check(ora, w, *_run_layer(w, 0, w.budget), w.budget)


def test_batch16_64k_sampled(ora):
    log("full size: batch 16 x 32 heads x 65536 tokens, budget 512 (oracle on 3 sequences)")
    w = synth.BATCH16_64K
    lay, codes, idx, out = _run_layer(w, 0, w.budget)
    for b in (0, 7, 15):
        _check(ora, w, lay, codes, idx, out, w.budget, batch_rows=slice(b, b + 1))


def test_batch16_append_on_second_stream(ora):
    log("batched decode on stream 1 while a 4096-token prefill chunk is encoded on stream 2")
    w = synth.BATCH16_64K
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((16, 32, w.cap, 32), dtype=torch.uint8, device=DEV)
    for b in range(16):
        adamas.encode_keys(lay["k"][b:b + 1], codes[b:b + 1])
    torch.cuda.synchronize()
    ref_idx = torch.empty((16, 32, w.budget), dtype=torch.int32, device=DEV)
    ref = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                             idx_out=ref_idx)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    ws1, ws2 = adamas.Workspace(DEV), adamas.Workspace(DEV)
    outs = []
    for step in range(3):
        b = step % 16
        chunk = synth.make_chunk(w, step, DEV)
        kdst = lay["k"][b:b + 1]
        cdst = codes[b:b + 1]
        torch.cuda.synchronize()
        with torch.cuda.stream(s2):
            adamas.encode_keys(chunk, cdst, pos=w.n_ctx, x_copy=kdst, stream=s2)
        with torch.cuda.stream(s1):
            idx = torch.empty_like(ref_idx)
            o = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                                   idx_out=idx, ws=ws1, stream=s1)
        torch.cuda.synchronize()
        outs.append((o, idx))
        # the appended rows landed where they should, bit-exactly
        got = codes[b, :, w.n_ctx:].cpu().numpy()
        want = ora.encode_keys(host(chunk))[0]
        assert np.array_equal(got, want)
        assert torch.equal(lay["k"][b, :, w.n_ctx:], chunk[0])
    for o, idx in outs:   # the decode reads rows [0, n_ctx) only: unaffected by the appends
        assert torch.equal(o, ref) and torch.equal(idx, ref_idx)
    del ws2


def test_graph_replay_of_layer_stack(ora):
    log("HIP graph: 4 layers of the 128K stack captured once, replayed 3 times")
    w = synth.LLAMA2_128K_32L.replace(n_ctx=40000, cap=40000)
    layers = []
    for l in range(4):
        lay = synth.make_layer(w, l, DEV)
        codes = torch.empty((1, 32, w.cap, 32), dtype=torch.uint8, device=DEV)
        adamas.encode_keys(lay["k"], codes)
        layers.append((lay, codes, torch.empty_like(lay["q"]),
                       torch.empty((1, 32, 256), dtype=torch.int32, device=DEV)))
    s = torch.cuda.Stream(DEV)
    ws = adamas.Workspace(DEV)
    ws.get(adamas.workspace_bytes(adamas.OP_DECODE_STEP, 1, 32, 32, w.n_ctx, 256, 128))

    def step():
        for lay, codes, out, idx in layers:
            adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, 256, out=out,
                               idx_out=idx, ws=ws, stream=s)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = [(o.clone(), i.clone()) for _, _, o, i in layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for _, _, o, i in layers:
            o.zero_()
            i.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, i), (_, _, og, ig) in zip(eager, layers):
            assert torch.equal(o, og) and torch.equal(i, ig), f"replay {rep} differs"
        # eager work between replays, as a real loop would interleave it
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any()
    lay, codes, o, i = layers[2]
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    _, _, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), w.n_ctx, 256)
    assert np.array_equal(i.cpu().numpy(), oidx)
