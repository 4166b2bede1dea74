"""The allocation-free decode step (adamas_decode_step_static) against the
workspace one (adamas_decode_step), through the C ABI: two calls in a row,
the second on a smaller input, each bit-identical to the workspace call of
the same schedule (last arrival) and its selection equal to the oracle's."""
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
    yield
    adamas.set_decode_mode(adamas.DECODE_AUTO)


def _pair(ora, w, budget, n_ctx, layer):
    lay = synth.make_layer(w, layer, DEV)
    codes = torch.zeros((w.batch, w.hkv, w.cap, w.head_dim // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx_s = torch.full((w.batch, w.hq, budget), -7, dtype=torch.int32, device=DEV)
    out_s = adamas.decode_step_static(lay["q"], lay["k"], lay["v"], codes, n_ctx, budget,
                                      idx_out=idx_s)
    # the workspace entry point in the same (last-arrival) schedule
    adamas.set_decode_mode(adamas.DECODE_LAST_ARRIVAL)
    idx_w = torch.full_like(idx_s, -7)
    out_w = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n_ctx, budget, idx_out=idx_w,
                               ws=adamas.Workspace(DEV))
    adamas.set_decode_mode(adamas.DECODE_AUTO)
    torch.cuda.synchronize()
    assert torch.equal(idx_s, idx_w), "selection differs from the workspace entry point"
    assert torch.equal(out_s, out_w), "output differs from the workspace entry point"
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oout, o64, oidx = ora.decode_step(q, k, v, ora.encode_keys(k), n_ctx, budget)
    assert np.array_equal(idx_s.cpu().numpy(), oidx)
    check_out(ora, out_s, q, k, v, oidx, oout, o64, f"static n={n_ctx} budget={budget}")


def test_static_scratch_two_calls_second_smaller(ora):
    log("static scratch: 32 heads x 40000 tokens, budget 1024 (attention in its own launch)")
    big = synth.LLAMA2_32K.replace(hq=32, hkv=32, n_ctx=40000, cap=40000, budget=1024)
    assert adamas.load().adamas_static_scratch_need(1, 32, 32, 40000, 1024, 128) <= \
        adamas.STATIC_SCRATCH_BYTES
    _pair(ora, big, 1024, 40000, 0)
    log("static scratch: then 8 q / 4 kv heads x 3000 tokens, budget 64")
    small = synth.LLAMA32_GQA_1M.replace(hq=8, hkv=4, n_ctx=3000, cap=3000, budget=64)
    _pair(ora, small, 64, 3000, 1)


def test_static_scratch_rejects_a_shape_beyond_it():
    # 32 heads x 131072 tokens with every row selected needs ~40 MiB: rejected on the host
    need = adamas.load().adamas_static_scratch_need(1, 32, 32, 131072, 131072, 128)
    assert need > adamas.STATIC_SCRATCH_BYTES
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 32, 16, 128), dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros((1, 32, 16, 32), dtype=torch.uint8, device=DEV)
    big_cap = torch.zeros((1, 32, 131072, 128), dtype=torch.bfloat16, device=DEV)
    big_codes = torch.zeros((1, 32, 131072, 32), dtype=torch.uint8, device=DEV)
    with pytest.raises(adamas.AdamasError) as e:
        adamas.decode_step_static(q, big_cap, big_cap, big_codes, 131072, 131072)
    assert e.value.status == 3          # ADAMAS_ERR_WORKSPACE
    del kv, codes


def test_static_scratch_single_chunk(ora):
    # contexts of one chunk: the chunk workgroup's candidates are the selection
    log("static scratch: 8 q / 2 kv heads x 900 tokens, budget 300 (attention in its own launch)")
    w = synth.LLAMA32_GQA_1M.replace(hq=8, hkv=2, n_ctx=900, cap=900, budget=300)
    _pair(ora, w, 300, 900, 2)
    log("static scratch: then 2 heads x 1000 tokens, budget 128 (fused attention)")
    w = synth.LLAMA2_32K.replace(hq=2, hkv=2, n_ctx=1000, cap=1000, budget=128)
    _pair(ora, w, 128, 1000, 3)
