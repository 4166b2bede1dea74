"""Host checks of the test helpers the GPU parity tests rely on: the output
type's spacing used in the element-wise bound, and the oracle's error scale
sum_j p_j |v_j| (equal to the output itself when every value is >= 0)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import ulp


def test_ulp_bf16_and_f32():
    x = np.array([1.0, 1.5, 2.0, -3.0, 0.0, 2.0 ** -126, 2.0 ** -130, 1e30])
    got = ulp(x, torch.bfloat16)
    want = [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133,
            2.0 ** (int(np.floor(np.log2(1e30))) - 7)]
    assert np.array_equal(got, np.array(want))
    g32 = ulp(x, torch.float32)
    assert np.array_equal(g32[:5], [2.0 ** -23, 2.0 ** -23, 2.0 ** -22, 2.0 ** -22, 2.0 ** -149])
    # agrees with numpy's float32 spacing on normal numbers
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32) * 100
    assert np.array_equal(ulp(r.astype(np.float64), torch.float32),
                          np.spacing(np.abs(r)).astype(np.float64))


def test_error_scale_equals_output_for_nonnegative_values(ora):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 3, 64)).astype(np.float32)
    k = rng.standard_normal((2, 3, 50, 64)).astype(np.float32)
    v = np.abs(rng.standard_normal((2, 3, 50, 64))).astype(np.float32)
    idx = np.sort(rng.choice(50, size=(2, 3, 20)), axis=-1).astype(np.int32)
    _, o64 = ora.sparse_attend(q, k, v, idx)
    a, s = ora.attend_error_scale(q, k, v, idx)
    assert np.array_equal(a, o64)
    # the score magnitude: the largest |scale| * sum_i |q_i k_j,i| over the selection
    for b in range(2):
        for h in range(3):
            rows = k[b, h, idx[b, h]].astype(np.float64)
            want = np.max(np.abs(rows) @ np.abs(q[b, h].astype(np.float64))) / 8.0
            assert s[b, h] == pytest.approx(want, rel=1e-14)
    # with signed values it bounds |o| from above
    v2 = (v * np.where(rng.random(v.shape) < 0.5, -1, 1)).astype(np.float32)
    _, o64b = ora.sparse_attend(q, k, v2, idx)
    a, s2 = ora.attend_error_scale(q, k, v2, idx)
    assert np.all(a >= np.abs(o64b)) and np.array_equal(a, o64) and np.array_equal(s2, s)


def _counter_csv(path, counter, rows):
    """A rocprofv3 counter_collection.csv with (kernel, grid, value) rows."""
    import csv
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for name, grid, val in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": val})


def test_bench_traffic_from_counter_runs(tmp_path):
    """bench.py --traffic-from: per-dispatch means of the decode kernel's
    FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for the
    1 GiB fp32 -> bf16 calibration conversion (grid 2^25), in bytes."""
    import json
    import bench
    dec = "void adm::k_decode<128, 1, true, 0, false, false>(void const*, ...)"
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda"
    _counter_csv(tmp_path / "f", "FETCH_SIZE",
                 [(dec, "262144", 1000.0), (dec, "262144", 1200.0), (cal, str(1 << 25), 524288.0),
                  (cal, "256", 3.0), ("void adm::k_encode<128>", "2097152", 9.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE",
                 [(dec, "262144", 10.0), (cal, str(1 << 25), 262144.0)])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out))
    t = json.load(open(out))
    # fetch: mean 1100 KiB x (1048576 / 524288); write: 10 KiB x (524288 / 262144)
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 2.0
    assert t["traffic_bytes_per_launch"] == (1100 * 2 + 10 * 2) * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    assert t["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(1, 32, 32, 128, 131072,
                                                                        256, 2)
