"""GPU parity over a seeded sweep of decode-step shapes: head_dim, dtype,
grouped heads, batch, context length, budget, always-kept tokens and the
schedule are drawn at random (a fixed seed per case), and every case checks
the selection bit for bit and the output within the dtype's tolerance
against the oracle.  Forced schedules that do not apply to a drawn shape
fall back to the automatic choice."""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import TOL, host, log, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_MODES = [adamas.DECODE_AUTO, adamas.DECODE_LAST_ARRIVAL, adamas.DECODE_GROUP_WAIT,
          adamas.DECODE_SPLIT]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    adamas.load()


@pytest.fixture
def restore_mode():
    yield
    adamas.set_decode_mode(adamas.DECODE_AUTO)


def _draw(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128, 256]))
    dt = "f32" if r.random() < 0.3 else "bf16"
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 3, 4, 8]))
    b = int(r.integers(1, 4))
    n = int(r.choice([1, 2, 63, 64, 65, 1000, 4097, 9000, 20000]))
    n = max(1, min(n, int(r.integers(n // 2 + 1, n + 1))))
    budget = int(r.choice([1, 5, 64, 100, 256, 1000, 3000]))
    keep = r.random() < 0.3
    n_sink = int(r.integers(0, 8)) if keep else 0
    n_recent = int(r.integers(0, 64)) if keep else 0
    mode = _MODES[int(r.integers(0, len(_MODES)))]
    return d, dt, hkv, g, b, n, budget, n_sink, n_recent, mode


@pytest.mark.parametrize("seed", list(range(24)))
def test_decode_random_shape(ora, restore_mode, seed):
    d, dt, hkv, g, b, n, budget, n_sink, n_recent, mode = _draw(7000 + seed)
    hq = hkv * g
    w = synth.TINY.replace(batch=b, hq=hq, hkv=hkv, head_dim=d, dtype=dt, n_ctx=n, cap=n + 3,
                           budget=budget)
    adamas.set_decode_mode(mode)
    try:
        path = adamas.decode_path(b, hq, hkv, n, budget, d)
    except adamas.AdamasError:  # the forced schedule does not fit this shape
        mode = adamas.DECODE_AUTO
        adamas.set_decode_mode(mode)
        path = adamas.decode_path(b, hq, hkv, n, budget, d)
    log(f"seed {seed}: d={d} {dt} B={b} Hq={hq} Hkv={hkv} n={n} budget={budget} "
        f"sink={n_sink} recent={n_recent} mode={mode} path={path}")
    lay = synth.make_layer(w, seed % 3, DEV)
    codes = torch.zeros((b, hkv, n + 3, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    idx = torch.full((b, hq, budget), -7, dtype=torch.int32, device=DEV)
    ws = adamas.Workspace(DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, n, budget, idx_out=idx, ws=ws,
                             n_sink=n_sink, n_recent=n_recent)
    torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any(), "control bytes left set"
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k)
    assert np.array_equal(codes.cpu().numpy(), oc), "code cache differs"
    oout, _, oidx = ora.decode_step(q, k, v, oc, n, budget, 0.0, n_sink, n_recent)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    e = rel_err(out, oout)
    log(f"  rel err {e:.3e}")
    assert e <= TOL[w.torch_dtype]
