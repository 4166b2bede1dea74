"""GPU parity at head_dim 256 (two 128-dimension absmax groups per vector):
the fused decode step under each schedule, the ragged append step and the
paged step, against the oracle (codes and selections bit for bit, outputs
within the dtype's tolerance)."""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import check_out, check_out_paged, host, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    adamas.load()


@pytest.fixture
def restore_mode():
    yield
    adamas.set_decode_mode(adamas.DECODE_AUTO)


_CASES = {
    "gqa-8-4-20000-b256": synth.LLAMA2_32K.replace(head_dim=256, hq=8, hkv=4, n_ctx=20000,
                                                   cap=20000, budget=256),
    "mha-4-70000-b1024": synth.LLAMA2_32K.replace(head_dim=256, hq=4, hkv=4, n_ctx=70000,
                                                  cap=70000, budget=1024),
    "f32-3-1-3000-b100": synth.TINY.replace(head_dim=256, batch=2, hq=3, hkv=1, n_ctx=3000,
                                            cap=3000, budget=100),
}


@pytest.mark.parametrize("mode", [adamas.DECODE_AUTO, adamas.DECODE_LAST_ARRIVAL,
                                  adamas.DECODE_GROUP_WAIT, adamas.DECODE_SPLIT])
@pytest.mark.parametrize("case", sorted(_CASES))
def test_decode_d256(ora, restore_mode, mode, case):
    w = _CASES[case]
    log(f"decode d=256 {case} mode {mode}")
    adamas.set_decode_mode(mode)
    path = adamas.decode_path(w.batch, w.hq, w.hkv, w.n_ctx, w.budget, 256)
    if mode != adamas.DECODE_AUTO:
        assert path == mode
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((w.batch, w.hkv, w.cap, 64), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k)
    assert np.array_equal(codes.cpu().numpy(), oc), "code cache differs"
    idx = torch.empty((w.batch, w.hq, w.budget), dtype=torch.int32, device=DEV)
    ws = adamas.Workspace(DEV)
    out = adamas.decode_step(lay["q"], lay["k"], lay["v"], codes, w.n_ctx, w.budget,
                             idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    assert not ws.buf[:adamas.WS_CTRL_BYTES].any()
    oout, o64, oidx = ora.decode_step(q, k, v, oc, w.n_ctx, w.budget)
    assert np.array_equal(idx.cpu().numpy(), oidx), "selection differs"
    check_out(ora, out, q, k, v, oidx, oout, o64, f"path {path}")


def test_append_d256(ora):
    log("ragged append step at d=256")
    w = synth.LLAMA2_32K.replace(head_dim=256, batch=3, hq=4, hkv=2, n_ctx=5000, cap=5000,
                                 budget=128)
    lay = synth.make_layer(w, 0, DEV)
    codes = torch.zeros((3, 2, 5000, 64), dtype=torch.uint8, device=DEV)
    adamas.encode_keys(lay["k"], codes)
    kn = synth.random_values((3, 2, 256), torch.bfloat16, 5, device=DEV)
    vn = synth.random_values((3, 2, 256), torch.bfloat16, 6, device=DEV)
    kn[0] = lay["q"][0, ::2]
    lens = [4999, 1024, 0]
    q, k, v = (host(lay[x]) for x in ("q", "k", "v"))
    oc = ora.encode_keys(k)
    idx = torch.empty((3, 4, 128), dtype=torch.int32, device=DEV)
    out = adamas.decode_append_step(lay["q"], lay["k"], lay["v"], codes,
                                    torch.tensor(lens, dtype=torch.int32, device=DEV), 5000, 128,
                                    k_new=kn, v_new=vn, idx_out=idx)
    torch.cuda.synchronize()
    oout, o64, oidx, ok, ov, ocd = ora.decode_append_step(q, k, v, oc, np.array(lens), 5000,
                                                          128, host(kn), host(vn))
    assert np.array_equal(codes.cpu().numpy(), ocd) and np.array_equal(host(lay["k"]), ok)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out(ora, out, q, ok, ov, oidx, oout, o64, "append d256")
    assert (idx[0, 0].cpu().numpy() == 4999).any()      # the near-query key is kept


def test_paged_d256(ora):
    log("paged step at d=256 (1024-token pages)")
    B, Hq, Hkv, d, P, per = 2, 4, 4, 256, 1024, 3
    w = synth.LLAMA2_32K.replace(head_dim=d, batch=B, hq=Hq, hkv=Hkv, n_ctx=per * P,
                                 cap=per * P)
    lay = synth.make_layer(w, 0, DEV)
    n_pages = B * per + 1
    perm = np.random.default_rng(8).permutation(n_pages)[:B * per].reshape(B, per)
    kp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    cp = torch.zeros((n_pages, Hkv, P, d // 4), dtype=torch.uint8, device=DEV)
    for b in range(B):
        for i in range(per):
            pg = int(perm[b, i])
            adamas.encode_keys(lay["k"][b:b + 1, :, i * P:(i + 1) * P].contiguous(),
                               cp[pg:pg + 1], x_copy=kp[pg:pg + 1])
            vp[pg] = lay["v"][b, :, i * P:(i + 1) * P]
    table = perm.astype(np.int32)
    kn = synth.random_values((B, Hkv, d), torch.bfloat16, 9, device=DEV)
    vn = synth.random_values((B, Hkv, d), torch.bfloat16, 10, device=DEV)
    lens = [2047, 3000]
    kp_h, vp_h, cp_h = host(kp), host(vp), cp.cpu().numpy()
    idx = torch.empty((B, Hq, 256), dtype=torch.int32, device=DEV)
    out = adamas.decode_paged_step(lay["q"], kp, vp, cp, torch.from_numpy(table).to(DEV),
                                   torch.tensor(lens, dtype=torch.int32, device=DEV), per * P,
                                   256, k_new=kn, v_new=vn, idx_out=idx)
    torch.cuda.synchronize()
    oout, o64, oidx, okp, ovp, ocp = ora.decode_paged_step(host(lay["q"]), kp_h, vp_h, cp_h,
                                                           table, np.array(lens), per * P, 256,
                                                           host(kn), host(vn))
    assert np.array_equal(host(kp), okp) and np.array_equal(cp.cpu().numpy(), ocp)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    check_out_paged(ora, out, host(lay["q"]), okp, ovp, table, oidx, oout, o64, "paged d256")
