"""Full-size parity of the batch-16 calls the benchmark times.

bench.py's batch16-mha-64k-append4k workload (BatchAppendState) runs
adamas_decode_append_step -- or, with --paged, adamas_decode_paged_step --
over 16 sequences x 32 heads x 65536 rows with budget 512, each sequence
appending its new token at row 65535, while a 4096-token prefill chunk is
encoded on a second stream.  These tests build that same state, run the same
steps (the chunk beside each), and check three sequences against the oracle's
append step: the code, K and V rows the step writes and the selection
bit-exact, the output element-wise within tolerance; the chunk's code rows
bit-exact.  The oracle's per-sequence steps are independent, so checking a
subset of the batch is exact for those sequences.
"""
import numpy as np
import pytest
import torch

import compressed_key_sparse_amd as adamas
import synth
from gpu_helpers import check_out, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"
SEQS = (0, 9, 15)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    adamas.load()


def _sequence_caches(st, b):
    """Host copies of sequence b's K, V and code rows [0, n) as the step left them."""
    n, P = st.w.n_ctx, st.PAGE
    if not st.paged:
        return (host(st.k[b:b + 1, :, :n]), host(st.v[b:b + 1, :, :n]),
                st.codes[b:b + 1, :, :n].cpu().numpy())
    pages = [int(x) for x in st.table[b].tolist()]
    assert len(pages) * P == n
    gather = lambda pool: torch.cat([pool[pg] for pg in pages], dim=1)[None]
    return host(gather(st.kp)), host(gather(st.vp)), gather(st.cp).cpu().numpy()


def _run_and_check(ora, paged):
    import bench
    w = synth.BATCH16_64K
    n, bud = w.n_ctx, w.budget
    log(f"bench call at full size: {'paged' if paged else 'contiguous'} append step, "
        f"16 x 32 heads x {n} rows, budget {bud}, chunk on a second stream")
    st = bench.BatchAppendState(w, torch.device(DEV), bud, paged=paged)
    for i in range(3):                      # as the benchmark's steps, the chunk beside each
        st.step(i)
    torch.cuda.synchronize()
    out_bench = st.out.clone()
    idx = torch.empty((w.batch, w.hq, bud), dtype=torch.int32, device=DEV)
    st.step(3, idx_out=idx)                 # the same call, also returning the selection
    torch.cuda.synchronize()
    assert torch.equal(st.out, out_bench), "the step is not deterministic"
    assert st.ws.control_bytes_clear() and st.ws.status() == 0
    # the last chunk (step 3) landed bit-exactly where it should
    ch = st.chunks[3 % len(st.chunks)]
    want = ora.encode_keys(host(ch))[0]
    if paged:
        got = np.concatenate([st.cp[pg].cpu().numpy() for pg in st.spare], axis=1)
    else:
        got = st.codes[3 % w.batch, :, n:].cpu().numpy()
    assert np.array_equal(got, want), "prefill chunk codes differ"
    for b in SEQS:
        log(f"  sequence {b}")
        k, v, c = _sequence_caches(st, b)
        q = host(st.q[b:b + 1])
        kn, vn = host(st.kn[b:b + 1]), host(st.vn[b:b + 1])
        oout, o64, oidx, k2, v2, c2 = ora.decode_append_step(
            q, k, v, ora.encode_keys(k), np.array([n - 1]), n, bud, kn, vn)
        assert np.array_equal(c, c2), "code cache differs (setup rows or the appended row)"
        assert np.array_equal(k, k2) and np.array_equal(v, v2), "appended K/V row differs"
        assert np.array_equal(idx[b:b + 1].cpu().numpy(), oidx), "selection differs"
        check_out(ora, out_bench[b:b + 1], q, k2, v2, oidx, oout, o64, f"sequence {b}")


def test_bench_append_step_full_size(ora):
    _run_and_check(ora, paged=False)


def test_bench_paged_step_full_size(ora):
    _run_and_check(ora, paged=True)
