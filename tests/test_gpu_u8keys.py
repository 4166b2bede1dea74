"""GPU parity of the one-byte key variant of the fused decode kernel.

Grouped heads whose 16-bit chunk keys would make a launch take two rounds of
workgroups keep min(key, 255) in LDS instead, in chunks twice as long.
Selection must not change: keys below a chunk threshold under 255 are
exact, and a chunk where some head's threshold reaches 255 is re-scanned
with exact keys, half a chunk at a time.  The first test runs the common
case (every chunk threshold far below 255); the second builds caches whose
keys are far from every query (codes near the complement of the query's,
distances around 290 for head_dim 128), so whole sequences are selected
from re-scanned chunks, with ties at the threshold split across halves.
The group-wait kernel takes one-byte keys where 16-bit ones would need
more chunks than the device holds at once, with the same exact re-scan.
Selection bit for bit, output within the dtype's bound, under every
schedule."""
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
    adamas.set_decode_mode(adamas.DECODE_AUTO)
    adamas.set_rotation(True)


@pytest.fixture(scope="module")
def gqa_case(ora):
    w = synth.LLAMA32_GQA_1M.replace(batch=2, n_ctx=300000, cap=300000)
    log("building the 2 x 8 x 300000-token GQA caches and the oracle's codes")
    lay = synth.make_layer(w, 7, DEV)
    codes = torch.zeros((2, 8, 300000, 32), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    ocodes = ora.encode_keys(k)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    return lay, codes, q, k, v, ocodes


MODES = [adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_SPLIT, adamas.DECODE_GROUP_WAIT]


@pytest.mark.parametrize("budget", [256, 1024])
@pytest.mark.parametrize("mode", MODES)
def test_u8_keys_gqa(ora, gqa_case, mode, budget):
    lay, codes, q, k, v, ocodes = gqa_case
    log(f"GQA 24/8, 2 x 300000 tokens, budget {budget}, mode {mode}")
    adamas.set_decode_mode(mode)
    assert adamas.decode_path(2, 24, 8, 300000, budget, 128) == mode
    assert adamas.decode_key_bytes(2, 24, 8, 300000, budget, 128) == 1
    idx = torch.empty((2, 24, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 300000, budget, idx_out=idx)
    torch.cuda.synchronize()
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 300000, budget)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, k, v, oidx, oout, o64, f"u8 keys GQA budget {budget} mode {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_u8_keys_gqa_keep_set(ora, gqa_case, mode):
    """Always-kept sinks and recent window (key 0) through the one-byte keys."""
    lay, codes, q, k, v, ocodes = gqa_case
    log(f"GQA 24/8, 2 x 300000 tokens, budget 512 with 4 sinks and a 64-token window, mode {mode}")
    adamas.set_decode_mode(mode)
    assert adamas.decode_key_bytes(2, 24, 8, 300000, 512, 128) == 1
    idx = torch.empty((2, 24, 512), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, 300000, 512, idx_out=idx,
                             n_sink=4, n_recent=64)
    torch.cuda.synchronize()
    oout, o64, oidx = ora.decode_step(q, k, v, ocodes, 300000, 512, n_sink=4, n_recent=64)
    got = idx.cpu().numpy()
    assert np.array_equal(got, oidx)
    assert np.isin(np.arange(4), got[0, 0]).all() and np.isin(np.arange(299936, 300000), got[1, 5]).all()
    check_out(ora, out, q, k, v, oidx, oout, o64, f"u8 keys keep set mode {mode}")


def _far_caches(B, Hkv, G, n, d, n_far, seed):
    """q: per (sequence, KV head) a +-1 pattern shared by its G query heads
    (codes 0 and 3 with the rotation off); keys of sequence b's tokens below
    n_far[b] are minus that pattern plus N(0, 0.6^2) noise, the rest N(0, 1)."""
    signs = synth.integer_values((B, Hkv, d), 0, 1, seed) * 2 - 1
    s = torch.from_numpy(signs).to(DEV)
    q = s.repeat_interleave(G, dim=1).to(torch.bfloat16).contiguous()
    noise = synth.random_values((B, Hkv, n, d), torch.float32, seed + 1, device=DEV)
    rnd = synth.random_values((B, Hkv, n, d), torch.float32, seed + 2, device=DEV)
    far = -s[:, :, None, :] + 0.6 * noise
    tok = torch.arange(n, device=DEV)[None, None, :, None]
    lim = torch.tensor(n_far, device=DEV)[:, None, None, None]
    k = torch.where(tok < lim, far, rnd).to(torch.bfloat16).contiguous()
    del noise, rnd, far
    v = synth.random_values((B, Hkv, n, d), torch.bfloat16, seed + 3, device=DEV)
    return q, k, v


@pytest.mark.parametrize("shape", [(2, 2, 256), (2, 2, 1024), (1, 8, 256)],
                         ids=lambda s: f"hkv{s[0]}-g{s[1]}-b{s[2]}")
@pytest.mark.parametrize("mode", MODES)
def test_u8_keys_exact_rescan(ora, mode, shape):
    Hkv, G, budget = shape
    B, n, d = 16, 140000, 128
    log(f"far keys: {B} x {Hkv * G}/{Hkv} heads x {n} tokens, budget {budget}, mode {mode}")
    adamas.set_rotation(False)
    adamas.set_decode_mode(mode)
    assert adamas.decode_path(B, Hkv * G, Hkv, n, budget, d) == mode
    assert adamas.decode_key_bytes(B, Hkv * G, Hkv, n, budget, d) == 1
    n_far = [n] * 7 + [70000] + [0] * 8    # 7 sequences all far, one half, 8 none
    q, k, v = _far_caches(B, Hkv, G, n, d, n_far, seed=81)
    codes = torch.zeros((B, Hkv, n, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(k, codes)
    idx = torch.empty((B, Hkv * G, budget), dtype=torch.int32, device=DEV)
    out = adamas.decode_step(q, k, v, codes, n, budget, idx_out=idx)
    torch.cuda.synchronize()
    qh, kh, vh = host(q), host(k), host(v)
    ocodes = ora.encode_keys(kh, rotate=False)
    assert np.array_equal(codes.cpu().numpy(), ocodes)
    oout, o64, oidx = ora.decode_step(qh, kh, vh, ocodes, n, budget, rotate=False)
    # every chunk of a far sequence (16384 or 32768 tokens as planned) has
    # its kc-th smallest key (distance + 1) at 255 or above: the kernel must
    # re-scan it
    qc = ora.encode_keys(qh[:, :, None, :], rotate=False)[:, :, 0]
    dist = ora.score(qc[:1], ocodes[:1], n_ctx=n)[0]
    for c0 in range(0, n, 16384):
        part = np.sort(dist[:, c0:c0 + 16384], axis=-1)
        kc = min(budget, part.shape[-1])
        assert part[:, kc - 1].min() + 1 >= 255, f"chunk at {c0} would not re-scan"
    got = idx.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], oidx[b]), f"selection of sequence {b} differs"
    check_out(ora, out, qh, kh, vh, oidx, oout, o64, f"u8 keys rescan budget {budget} mode {mode}")
