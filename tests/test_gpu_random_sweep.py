"""GPU parity over seeded sweeps of shapes (the decode step, the ragged append
step and the paged step): head_dim, dtype,
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
from gpu_helpers import check_out, check_out_paged, host, log

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
    oout, o64, oidx = ora.decode_step(q, k, v, oc, n, budget, 0.0, n_sink, n_recent)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, f"seed {seed}")


def _append_draw(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128, 256]))
    dt = "f32" if r.random() < 0.3 else "bf16"
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 3, 4]))
    b = int(r.integers(1, 6))
    max_len = int(r.choice([64, 1000, 4097, 9000]))
    lens = [int(x) for x in r.integers(0, max_len, size=b)]
    lens[0] = max_len - 1                      # one sequence at the bound
    budget = int(r.choice([1, 16, 100, 256, 700]))
    append = r.random() < 0.8
    keep = r.random() < 0.3
    return (d, dt, hkv, g, b, max_len, lens, budget, append,
            int(r.integers(0, 6)) if keep else 0, int(r.integers(0, 40)) if keep else 0)


@pytest.mark.parametrize("seed", list(range(12)))
def test_append_random_shape(ora, seed):
    d, dt, hkv, g, b, max_len, lens, budget, append, n_sink, n_recent = _append_draw(8000 + seed)
    hq = hkv * g
    log(f"append seed {seed}: d={d} {dt} B={b} Hq={hq} Hkv={hkv} max_len={max_len} lens={lens} "
        f"budget={budget} append={append} sink={n_sink} recent={n_recent}")
    w = synth.TINY.replace(batch=b, hq=hq, hkv=hkv, head_dim=d, dtype=dt, n_ctx=max_len,
                           cap=max_len, budget=budget)
    lay = synth.make_layer(w, seed % 3, DEV)
    codes = torch.zeros((b, hkv, max_len, d // 4), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    kn = synth.random_values((b, hkv, d), w.torch_dtype, 50 + seed, device=DEV)
    vn = synth.random_values((b, hkv, d), w.torch_dtype, 90 + seed, device=DEV)
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k)
    idx = torch.full((b, hq, budget), -7, dtype=torch.int32, device=DEV)
    out = adamas.decode_append_step(lay["q"], lay["k"], lay["v"], codes,
                                    torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
                                    budget, k_new=kn if append else None,
                                    v_new=vn if append else None, idx_out=idx, n_sink=n_sink,
                                    n_recent=n_recent)
    torch.cuda.synchronize()
    oout, o64, oidx, ok, ov, ocd = ora.decode_append_step(
        q, k, v, oc, np.array(lens), max_len, budget, host(kn) if append else None,
        host(vn) if append else None, n_sink=n_sink, n_recent=n_recent)
    assert np.array_equal(host(lay["k"]), ok) and np.array_equal(host(lay["v"]), ov)
    assert np.array_equal(codes.cpu().numpy(), ocd), "code cache differs"
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, ok, ov, oidx, oout, o64, f"append seed {seed}")


@pytest.mark.parametrize("seed", list(range(8)))
def test_paged_random_shape(ora, seed):
    r = np.random.default_rng(9000 + seed)
    d = int(r.choice([64, 128]))
    dt = "f32" if r.random() < 0.3 else "bf16"
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 3]))
    b = int(r.integers(1, 5))
    P = int(r.choice([1024, 2048]))
    per = int(r.integers(1, 4))
    budget = int(r.choice([1, 64, 256, 600]))
    append = r.random() < 0.8
    hq = hkv * g
    max_len = per * P
    lens = [int(x) for x in r.integers(0, max_len, size=b)]
    log(f"paged seed {seed}: d={d} {dt} B={b} Hq={hq} Hkv={hkv} P={P} pages={per} lens={lens} "
        f"budget={budget} append={append}")
    w = synth.TINY.replace(batch=b, hq=hq, hkv=hkv, head_dim=d, dtype=dt, n_ctx=max_len,
                           cap=max_len, budget=budget)
    lay = synth.make_layer(w, seed % 3, DEV)
    n_pages = b * per + 2
    perm = r.permutation(n_pages)[:b * per].reshape(b, per)
    kp = torch.zeros((n_pages, hkv, P, d), dtype=w.torch_dtype, device=DEV)
    vp = torch.zeros_like(kp)
    cp = torch.zeros((n_pages, hkv, P, d // 4), dtype=torch.uint8, device=DEV)
    for s in range(b):
        for i in range(per):
            pg = int(perm[s, i])
            adamas.encode_keys(lay["k"][s:s + 1, :, i * P:(i + 1) * P].contiguous(),
                               cp[pg:pg + 1], x_copy=kp[pg:pg + 1])
            vp[pg] = lay["v"][s, :, i * P:(i + 1) * P]
    table = perm.astype(np.int32)
    kn = synth.random_values((b, hkv, d), w.torch_dtype, 130 + seed, device=DEV)
    vn = synth.random_values((b, hkv, d), w.torch_dtype, 170 + seed, device=DEV)
    kp_h, vp_h, cp_h = host(kp), host(vp), cp.cpu().numpy()
    idx = torch.full((b, hq, budget), -7, dtype=torch.int32, device=DEV)
    out = adamas.decode_paged_step(lay["q"], kp, vp, cp, torch.from_numpy(table).to(DEV),
                                   torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
                                   budget, k_new=kn if append else None,
                                   v_new=vn if append else None, idx_out=idx)
    torch.cuda.synchronize()
    oout, o64, oidx, okp, ovp, ocp = ora.decode_paged_step(
        host(lay["q"]), kp_h, vp_h, cp_h, table, np.array(lens), max_len, budget,
        host(kn) if append else None, host(vn) if append else None)
    assert np.array_equal(host(kp), okp) and np.array_equal(host(vp), ovp)
    assert np.array_equal(cp.cpu().numpy(), ocp), "code pool differs"
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out_paged(ora, out, host(lay["q"]), okp, ovp, table, oidx, oout, o64,
                    f"paged seed {seed}")
