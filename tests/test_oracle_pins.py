"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a hand-worked example, an
invariant the ADAMAS article (www.lnwmold.com/news/826806) states, or brute
force on tiny inputs -- never against a retyped copy of its own formula.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent helpers (not the oracle's code paths)
def sylvester(d: int) -> np.ndarray:
    """H_d from the recursion [[H, H], [H, -H]] (§2.1 recursive construction)."""
    h = np.ones((1, 1), np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Bytes -> 2-bit codes, first code in the top bits, via np.unpackbits."""
    bits = np.unpackbits(np.asarray(packed, np.uint8).reshape(-1, 1), axis=1)  # MSB first
    pairs = bits.reshape(-1, 4, 2)
    return (pairs[..., 0] * 2 + pairs[..., 1]).reshape(np.asarray(packed).shape[:-1] + (-1,))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8).reshape(-1, 4)
    bits = np.stack([c >> 1 & 1, c & 1], axis=-1).reshape(-1, 8)
    return np.packbits(bits, axis=1).reshape(-1)


def thermometer(codes: np.ndarray) -> np.ndarray:
    """U(c) in {0,1}^3 with <U(a), U(b)> = min(a, b)."""
    c = np.asarray(codes)[..., None]
    return (c >= np.array([1, 2, 3])).astype(np.int64).reshape(c.shape[:-2] + (-1,))


# --------------------------------------------------------------------------
# §2.1 rotation
@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_columns_are_sylvester_hadamard(ora, d):
    H = sylvester(d)
    cols = np.stack([ora.fwht_f32(np.eye(d, dtype=np.float32)[j]) for j in range(d)], axis=1)
    assert np.array_equal(cols.astype(np.int64), H)
    i = np.arange(d)
    popc = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(H, (-1) ** popc)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [4, 64, 128, 256])
def test_fwht_exact_on_integers(ora, d):
    # |x| * d < 2^24 keeps every partial sum exact in binary32
    x = synth.integer_values((50, d), -1000, 1000, seed=d)
    H = sylvester(d)
    for row in x:
        y = ora.fwht_f32(row)
        assert np.array_equal(y.astype(np.int64), H @ row.astype(np.int64))


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_f32_within_rounding_bound(ora, d):
    rng = np.random.default_rng(3)
    H = sylvester(d).astype(np.float64)
    for _ in range(20):
        x = (rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float32)
        y = ora.fwht_f32(x).astype(np.float64)
        exact = H @ x.astype(np.float64)
        # log2(d) rounded adds, each with relative error <= 2^-24 of a partial sum
        bound = math.log2(d) * 2.0 ** -24 * np.abs(H) @ np.abs(x.astype(np.float64)) * 1.01
        assert np.all(np.abs(y - exact) <= bound)


@pytest.mark.parametrize("d", [64, 128])
def test_orthonormal_rotation_preserves_dot_and_norm(ora, d):
    rng = np.random.default_rng(d)
    H = sylvester(d) / math.sqrt(d)
    assert np.allclose(H @ H.T, np.eye(d), atol=1e-15 * d)
    for _ in range(20):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        hq, hk = ora.hadamard_orthonormal_f64(q), ora.hadamard_orthonormal_f64(k)
        assert abs(hq @ hk - q @ k) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(np.linalg.norm(hq) - np.linalg.norm(q)) <= 1e-12 * np.linalg.norm(q)
        assert np.max(np.abs(hq)) >= np.linalg.norm(q) / math.sqrt(d) * (1 - 1e-12)


# --------------------------------------------------------------------------
# §2.2 bucketing + §3.1 packing
def _golden_encode_cases():
    cases = []
    with open(os.path.join(GOLDEN, "encode_hand_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            d, x, y, c, hexes = (s.strip() for s in line.split("|"))
            cases.append((int(d), [float(t) for t in x.split(",")], [float(t) for t in y.split(",")],
                          [int(t) for t in c.split(",")], bytes.fromhex(hexes.replace(" ", ""))))
    return cases


@pytest.mark.parametrize("case", _golden_encode_cases(), ids=lambda c: f"d{c[0]}-{c[4].hex()}")
def test_encode_hand_worked(ora, case):
    d, x, y, codes, packed = case
    p, yy, cc = ora.encode_vec(np.array(x, np.float32))
    assert yy.tolist() == y
    assert cc.tolist() == codes
    assert bytes(p) == packed
    assert unpack_codes(p).tolist() == codes


@pytest.mark.parametrize("d", [64, 128, 256])
def test_encode_unit_vectors_closed_form(ora, d):
    # H e_j is column j of H (entries +-1, absmax 1): +1 -> code 3, -1 -> code 0
    H = sylvester(d)
    for j in range(d):
        p, _, c = ora.encode_vec(np.eye(d, dtype=np.float32)[j])
        want = np.where(H[:, j] > 0, 3, 0)
        assert np.array_equal(c, want)
        assert np.array_equal(p, pack_codes(want))


def test_encode_scale_and_sign_properties(ora):
    rng = np.random.default_rng(11)
    for d in (64, 128):
        for _ in range(200):
            x = rng.standard_normal(d).astype(np.float32)
            p, y, c = ora.encode_vec(x)
            # power-of-two scaling is exact in binary32 -> identical codes
            for s in (2.0 ** -20, 0.5, 4.0, 2.0 ** 30):
                assert np.array_equal(ora.encode_vec(x * np.float32(s))[0], p)
            # negation mirrors the codes when no rotated value sits on a threshold
            a = np.max(np.abs(y))
            if not np.any(np.isin(y, [0.0, a / 2, -a / 2])):
                assert np.array_equal(ora.encode_vec(-x)[2], 3 - c)
            # the definition, by brute force over the rotated values
            want = np.select([y < -0.5 * a, y < 0, y < 0.5 * a], [0, 1, 2], 3)
            assert np.array_equal(c, want)


def test_encode_keys_layout(ora):
    # codes land at rows [pos, pos+n) of a [batch][heads][cap][d/4] cache
    x = synth.integer_values((2, 3, 5, 64), -9, 9, seed=1)
    codes = np.full((2, 3, 9, 16), 0x5A, np.uint8)
    ora.encode_keys(x, codes, cap=9, pos=3)
    for b, h, t in itertools.product(range(2), range(3), range(9)):
        if 3 <= t < 8:
            assert np.array_equal(codes[b, h, t], ora.encode_vec(x[b, h, t - 3])[0])
        else:
            assert np.all(codes[b, h, t] == 0x5A)


def test_encode_keys_bf16_widening_exact(ora):
    import torch
    x = synth.random_values((1, 2, 40, 128), torch.bfloat16, seed=4)
    xb = synth.to_numpy_bits(x)
    c1 = ora.encode_keys(xb)
    c2 = ora.encode_keys(x.float().numpy())
    assert np.array_equal(c1, c2)


# --------------------------------------------------------------------------
# §2.3 Manhattan distance
def test_manhattan_exhaustive_small(ora):
    # every pair of 2-bit code vectors of length 4 (one byte each)
    allc = np.array(list(itertools.product(range(4), repeat=4)))
    for a in allc:
        for b in allc[::7]:
            got = ora.manhattan(pack_codes(a), pack_codes(b), 4)
            assert got == int(np.abs(a - b).sum())


@pytest.mark.parametrize("d", [64, 128])
def test_score_gemm_identity_and_metric(ora, d):
    rng = np.random.default_rng(d)
    B, Hq, Hkv, n = 2, 6, 3, 300
    qc = rng.integers(0, 4, size=(B, Hq, d))
    kc = rng.integers(0, 4, size=(B, Hkv, n, d))
    qp = pack_codes(qc.reshape(-1, d).reshape(-1)).reshape(B, Hq, d // 4)
    kp = pack_codes(kc.reshape(-1)).reshape(B, Hkv, n, d // 4)
    dist = ora.score(qp, kp)
    G = Hq // Hkv
    # D = sum(q) + sum(k) - 2 <U(q), U(k)> with the thermometer expansion U
    for b in range(B):
        for h in range(Hq):
            uq = thermometer(qc[b, h])
            uk = thermometer(kc[b, h // G])
            want = qc[b, h].sum() + kc[b, h // G].sum(axis=1) - 2 * (uk @ uq)
            assert np.array_equal(dist[b, h].astype(np.int64), want)
    # metric facts on packed rows
    zeros, threes = pack_codes(np.zeros(d, int)), pack_codes(np.full(d, 3))
    assert ora.manhattan(zeros, threes, d) == 3 * d
    assert ora.manhattan(threes, threes, d) == 0
    e0 = ora.encode_vec(np.eye(d, dtype=np.float32)[0])[0]
    e1 = ora.encode_vec(np.eye(d, dtype=np.float32)[1])[0]
    assert ora.manhattan(e0, e1, d) == 3 * d // 2
    for _ in range(50):
        a, b, c = (pack_codes(rng.integers(0, 4, d)) for _ in range(3))
        ab, ba = ora.manhattan(a, b, d), ora.manhattan(b, a, d)
        assert ab == ba and 0 <= ab <= 3 * d
        assert ab <= ora.manhattan(a, c, d) + ora.manhattan(c, b, d)


def test_score_respects_n_ctx_and_gqa_mapping(ora):
    rng = np.random.default_rng(5)
    d, n, cap = 64, 37, 50
    kc = rng.integers(0, 4, size=(1, 2, cap, d))
    qc = rng.integers(0, 4, size=(1, 4, d))
    kp = pack_codes(kc.reshape(-1)).reshape(1, 2, cap, d // 4)
    qp = pack_codes(qc.reshape(-1)).reshape(1, 4, d // 4)
    dist = ora.score(qp, kp, n_ctx=n)
    assert dist.shape == (1, 4, n)
    for h in range(4):
        want = np.abs(qc[0, h][None, :] - kc[0, h // 2, :n]).sum(axis=1)
        assert np.array_equal(dist[0, h], want)


# --------------------------------------------------------------------------
# §5.2 budget selection
def brute_select(dvec, budget):
    """Rank counting: token t is kept iff fewer than `budget` tokens precede
    it in (distance, index) order.  No sorting involved."""
    n = len(dvec)
    keep = [t for t in range(n)
            if sum(1 for u in range(n) if (dvec[u], u) < (dvec[t], t)) < budget]
    return keep + [-1] * (budget - len(keep))


def test_select_exhaustive_tiny(ora):
    for n in range(1, 7):
        vecs = np.array(list(itertools.product(range(4), repeat=n)), np.uint16)
        for budget in range(1, n + 3):
            got = ora.select_topk(vecs.reshape(1, -1, n), budget)[0]
            for row, dv in zip(got, vecs):
                assert row.tolist() == brute_select(dv.tolist(), budget)


def test_select_ties_lowest_index(ora):
    d = np.full((1, 1, 1000), 77, np.uint16)
    assert ora.select_topk(d, 64)[0, 0].tolist() == list(range(64))
    d[0, 0, 500:] = 76   # the 500 smaller ones win, ties fill from index 0
    got = ora.select_topk(d, 600)[0, 0]
    assert got.tolist() == list(range(100)) + list(range(500, 1000))


def test_select_random_against_brute(ora):
    rng = np.random.default_rng(9)
    for n in (5, 17, 40):
        for budget in (1, 3, 16, 50):
            d = rng.integers(0, 8, size=(3, 2, n)).astype(np.uint16)
            got = ora.select_topk(d, budget)
            for b in range(3):
                for h in range(2):
                    assert got[b, h].tolist() == brute_select(d[b, h].tolist(), budget)


def test_select_forced_set_reduces_to_plain_selection(ora):
    """A forced set F (first n_sink, last n_recent tokens) ranks first inside
    the budget.  Characterised against the plain selection, pinned above: if
    |F| >= budget the budget's lowest-index members of F are kept; otherwise
    all of F plus the plain selection of budget - |F| among the other tokens."""
    for n in range(1, 6):
        vecs = np.array(list(itertools.product(range(4), repeat=n)), np.uint16)
        for n_sink in range(0, n + 1):
            for n_recent in range(0, n + 1):
                forced = [t for t in range(n) if t < n_sink or t >= n - n_recent]
                others = [t for t in range(n) if t not in forced]
                for budget in range(1, n + 2):
                    got = ora.select_topk(vecs.reshape(1, -1, n), budget, n_sink, n_recent)[0]
                    if len(forced) >= budget:
                        want_one = forced[:budget]
                    for row, dv in zip(got, vecs):
                        if len(forced) < budget:
                            rest = []
                            if others:
                                sub = dv[others].reshape(1, 1, -1)
                                pick = ora.select_topk(sub, budget - len(forced))[0, 0]
                                rest = [others[i] for i in pick if i >= 0]
                            want_one = sorted(forced + rest)
                        want = want_one + [-1] * (budget - len(want_one))
                        assert row.tolist() == want, (n, n_sink, n_recent, budget, dv)


def test_select_forced_set_special_cases(ora):
    rng = np.random.default_rng(4)
    d = rng.integers(0, 385, size=(1, 2, 3000)).astype(np.uint16)
    # no forced tokens: the plain selection
    assert np.array_equal(ora.select_topk(d, 256, 0, 0), ora.select_topk(d, 256))
    # sink and window cover everything: the first budget tokens
    assert ora.select_topk(d, 100, 2000, 1000)[0, 0].tolist() == list(range(100))
    # budget exactly the window: the last tokens, whatever their distances
    assert ora.select_topk(d, 64, 0, 64)[0, 1].tolist() == list(range(2936, 3000))
    # a sink of 4 and a window of 60 inside a budget of 256: all 64 kept
    got = ora.select_topk(d, 256, 4, 60)[0, 0].tolist()
    assert set(range(4)) <= set(got) and set(range(2940, 3000)) <= set(got)
    assert got == sorted(got) and len(set(got)) == 256


def test_decode_step_with_forced_set_composes(ora):
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    k = rng.standard_normal((1, 2, 700, 64)).astype(np.float32)
    v = rng.standard_normal((1, 2, 700, 64)).astype(np.float32)
    codes = ora.encode_keys(k)
    out, out64, idx = ora.decode_step(q, k, v, codes, 650, 40, 0.0, 3, 20)
    qc = np.ascontiguousarray(ora.encode_keys(q.reshape(1, 2, 1, 64))[:, :, 0, :])
    dist = ora.score(qc, codes, 650)
    assert np.array_equal(idx, ora.select_topk(dist, 40, 3, 20))
    ref, ref64 = ora.sparse_attend(q, k, v, idx)
    assert np.array_equal(out64, ref64)


def _golden_no_rotation_cases():
    out = []
    with open(os.path.join(GOLDEN, "encode_no_rotation_hand_worked.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            d, x, codes, packed = (p.strip() for p in line.split("|"))
            out.append((int(d), [float(v) for v in x.split(",")],
                        [int(c) for c in codes.split(",")], bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("case", _golden_no_rotation_cases(), ids=lambda c: c[3].hex())
def test_encode_without_rotation_hand_worked(ora, case):
    d, x, codes, packed = case
    got_packed, y, got_codes = ora.encode_vec(np.array(x, np.float32), rotate=False)
    assert got_codes.tolist() == codes
    assert bytes(got_packed) == packed
    assert np.array_equal(y, np.array(x, np.float32))   # nothing rotated


def _golden_alpha_cases():
    out = []
    with open(os.path.join(GOLDEN, "encode_alpha_hand_worked.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            d, rot, alpha, x, y, codes, packed = (p.strip() for p in line.split("|"))
            out.append((int(d), int(rot), float(alpha), [float(v) for v in x.split(",")],
                        [float(v) for v in y.split(",")], [int(c) for c in codes.split(",")],
                        bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("case", _golden_alpha_cases(),
                         ids=lambda c: f"rot{c[1]}-a{c[2]}-{c[6].hex()}")
def test_encode_alpha_hand_worked(ora, case):
    d, rot, alpha, x, y, codes, packed = case
    got_packed, got_y, got_codes = ora.encode_vec(np.array(x, np.float32), rotate=rot, alpha=alpha)
    assert got_y.tolist() == y
    assert got_codes.tolist() == codes
    assert bytes(got_packed) == packed


def test_encode_alpha_half_is_the_fixed_rule(ora):
    # 0.5 * a is exact in binary32, so alpha = 0.5 gives the §2.2 codes bit for bit
    rng = np.random.default_rng(21)
    for d in (64, 128, 256):
        for _ in range(50):
            x = rng.standard_normal(d).astype(np.float32)
            for rot in (0, 1):
                assert np.array_equal(ora.encode_vec(x, rotate=rot, alpha=0.5)[0],
                                      ora.encode_vec(x, rotate=rot)[0])


def test_encode_alpha_definition_and_limits(ora):
    rng = np.random.default_rng(22)
    for d in (64, 256):
        for alpha in (0.0, 0.1, 0.3, 0.7, 1.0, 1.5):
            x = rng.standard_normal(d).astype(np.float32)
            _, y, c = ora.encode_vec(x, rotate=1, alpha=alpha)
            g = 128 if d > 128 else d
            for g0 in range(0, d, g):
                yy, cc = y[g0:g0 + g], c[g0:g0 + g]
                t2 = np.float32(np.float32(alpha) * np.max(np.abs(yy)))
                want = np.select([yy < -t2, yy < 0, yy < t2], [0, 1, 2], 3)
                assert np.array_equal(cc, want)
                if alpha == 0.0:       # sign codes: 3 for y >= 0, 0 below
                    assert np.array_equal(cc, np.where(yy >= 0, 3, 0))
                if alpha >= 1.0:       # only the maximum can reach code 3, nothing code 0
                    assert not np.any(cc == 0)
                    assert np.all((cc != 3) | (yy == np.max(np.abs(yy))))


def test_encode_keys_alpha_per_head(ora):
    x = synth.integer_values((2, 5, 7, 64), -9, 9, seed=3)
    table = [0.25, 0.75, 0.4]
    codes = ora.encode_keys(x, alpha=table)
    for b, h, t in itertools.product(range(2), range(5), range(7)):
        want = ora.encode_vec(x[b, h, t], alpha=table[h % 3])[0]
        assert np.array_equal(codes[b, h, t], want)
    assert np.array_equal(ora.encode_keys(x, alpha=[0.5]), ora.encode_keys(x))


def test_decode_step_alpha_is_composition(ora):
    # query head hq buckets with its KV head's alpha (hq // G)
    w = synth.LLAMA2_32K.replace(hq=8, hkv=2, n_ctx=2000, cap=2100, budget=48)
    lay = synth.make_layer(w, 0, "cpu")
    q, k, v = (synth.to_numpy_bits(lay[x]) for x in ("q", "k", "v"))
    table = [0.3, 0.7]
    codes = ora.encode_keys(k, alpha=table)
    out, out64, idx = ora.decode_step(q, k, v, codes, n_ctx=2000, budget=48, alpha=table)
    qc = np.concatenate([ora.encode_keys(q[:, h:h + 1, None, :], alpha=[table[h // 4]])[:, :, 0]
                         for h in range(8)], axis=1)
    dist = ora.score(qc, codes, n_ctx=2000)
    idx2 = ora.select_topk(dist, 48)
    assert np.array_equal(idx, idx2)
    o2, o64 = ora.sparse_attend(q, k, v, idx2)
    assert np.array_equal(out, o2) and np.array_equal(out64, o64)
    # a table of 0.5s is the fixed rule
    c05 = ora.encode_keys(k, alpha=[0.5, 0.5])
    assert np.array_equal(c05, ora.encode_keys(k))
    r = ora.decode_step(q, k, v, c05, n_ctx=2000, budget=48, alpha=[0.5, 0.5])
    r0 = ora.decode_step(q, k, v, c05, n_ctx=2000, budget=48)
    assert all(np.array_equal(a, b) for a, b in zip(r, r0))


def test_encode_rotation_off_is_rotation_of_rotated_input(ora):
    # H (H x) = d x for the unnormalised Sylvester H, and codes are invariant
    # to a positive scale: encoding H x without the rotation equals encoding x
    # with it, whenever H x is exact in fp32 (integer inputs here)
    rng = np.random.default_rng(21)
    for d in (64, 128):
        x = rng.integers(-50, 50, size=(5, d)).astype(np.float32)
        for row in x:
            _, y, _ = ora.encode_vec(row)                 # y = H x, exact
            with_rot, _, _ = ora.encode_vec(row)
            without, _, _ = ora.encode_vec(y, rotate=False)
            assert bytes(with_rot) == bytes(without)
        k = x.reshape(1, 1, 5, d)
        yk = np.stack([ora.encode_vec(r)[1] for r in x]).reshape(1, 1, 5, d)
        assert np.array_equal(ora.encode_keys(k), ora.encode_keys(yk, rotate=False))


# --------------------------------------------------------------------------
# §6 attention over the selected rows
def dense_attention(q, k, v, scale):
    s = (k @ q) * scale
    w = np.exp(s - s.max())
    return (w / w.sum()) @ v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attend_full_budget_equals_dense(ora, dtype):
    import torch
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    B, Hq, Hkv, n, d = 2, 4, 2, 33, 64
    q = synth.random_values((B, Hq, d), dt, 1)
    k = synth.random_values((B, Hkv, n, d), dt, 2)
    v = synth.random_values((B, Hkv, n, d), dt, 3)
    idx = np.tile(np.arange(n, dtype=np.int32), (B, Hq, 1))
    out, out64 = ora.sparse_attend(*(synth.to_numpy_bits(t) for t in (q, k, v)), idx)
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    for b in range(B):
        for h in range(Hq):
            want = dense_attention(qd[b, h], kd[b, h // 2], vd[b, h // 2], 1 / math.sqrt(d))
            assert np.allclose(out64[b, h], want, rtol=1e-13, atol=1e-13)


def test_attend_single_row_is_exact_v(ora):
    import torch
    for dt in (torch.float32, torch.bfloat16):
        q = synth.random_values((1, 2, 128), dt, 5)
        k = synth.random_values((1, 2, 10, 128), dt, 6)
        v = synth.random_values((1, 2, 10, 128), dt, 7)
        idx = np.array([[[3, -1, -1]], [[7, -1, -1]]], np.int32).reshape(1, 2, 3)
        out, _ = ora.sparse_attend(*(synth.to_numpy_bits(t) for t in (q, k, v)), idx)
        vb = synth.to_numpy_bits(v)
        assert np.array_equal(out[0, 0], vb[0, 0, 3]) and np.array_equal(out[0, 1], vb[0, 1, 7])


def test_attend_two_rows_closed_form(ora):
    q = np.array([[[1.0, 0, 0, 0]]], np.float32)
    k = np.array([[[[2.0, 0, 0, 0], [0.0, 0, 0, 0]]]], np.float32)
    v = np.array([[[[1.0, 2, 3, 4], [5.0, 6, 7, 8]]]], np.float32)
    idx = np.array([[[0, 1]]], np.int32)
    _, o = ora.sparse_attend(q, k, v, idx, scale=1.0)
    p0 = 1 / (1 + math.exp(-2.0))   # logistic of s0 - s1 = 2
    vd = v.astype(np.float64)
    assert np.allclose(o[0, 0], p0 * vd[0, 0, 0] + (1 - p0) * vd[0, 0, 1], rtol=1e-14, atol=0)


def test_attend_order_and_padding_invariance(ora):
    import torch
    q = synth.random_values((1, 1, 64), torch.float32, 8)
    k = synth.random_values((1, 1, 50, 64), torch.float32, 9)
    v = synth.random_values((1, 1, 50, 64), torch.float32, 10)
    a = np.array([[[4, 9, 13, 40]]], np.int32)
    b = np.array([[[40, -1, 13, 4, -1, 9]]], np.int32)
    _, oa = ora.sparse_attend(q.numpy(), k.numpy(), v.numpy(), a)
    _, ob = ora.sparse_attend(q.numpy(), k.numpy(), v.numpy(), b)
    assert np.allclose(oa, ob, rtol=1e-14, atol=1e-15)
    vs = v.numpy()[0, 0, [4, 9, 13, 40]]
    assert np.all(oa[0, 0] <= vs.max(axis=0) + 1e-12) and np.all(oa[0, 0] >= vs.min(axis=0) - 1e-12)


def test_f64_to_bf16_correct_rounding(ora):
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000)))
    # halfway cases between adjacent bf16 values: ties go to the even pattern
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -133 * 1.5]
    for x in xs:
        bits = ora.f64_to_bf16_bits(x)
        val = np.array([bits << 16], np.uint32).view(np.float32)[0]
        # neighbours in bf16: step the pattern by one
        def as_f(b):
            return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))
        fx, fv = Fraction(x), Fraction(float(val))
        for nb in (bits - 1, bits + 1):
            if 0 <= nb < 1 << 16 and (nb & 0x7F80) != 0x7F80:
                err_v, err_n = abs(fx - fv), abs(fx - as_f(nb))
                assert err_v < err_n or (err_v == err_n and bits % 2 == 0)


def _bf16_bits_exact(x: float) -> int:
    """bfloat16 round-to-nearest-even of x by exact rational arithmetic, from
    the format's definition: sign, 8 exponent bits (bias 127), 7 fraction
    bits; normal values (1 + f/128) * 2^(e-127), subnormal f/128 * 2^-126;
    a result of 2^128 or more is an infinity."""
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x))
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                             # subnormals share the spacing of 2^-126
    spacing = Fraction(2) ** (e - 7)
    q = a / spacing
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * spacing                              # the rounded magnitude
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    if v < Fraction(2) ** -126:                  # subnormal: fraction bits only
        return sign | int(v / Fraction(2) ** -133)
    ev = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** ev > v:
        ev -= 1
    frac = (v / Fraction(2) ** ev - 1) * 128
    assert frac.denominator == 1 and 0 <= frac < 128
    return sign | ((ev + 127) << 7) | int(frac)


def test_f64_to_bf16_extremes_exact(ora):
    """The binary64 -> bfloat16 rounding at the edges of the format, against
    exact rational rounding: the overflow boundary (the largest finite value,
    the tie above it, which rounds to infinity because its pattern is odd, and
    the values just below that tie), the normal/subnormal boundary, the whole
    subnormal range including ties at half the smallest subnormal, and
    log-uniform draws over the entire binary64 range."""
    maxf = (2 - 2.0 ** -7) * 2.0 ** 127                 # largest finite bfloat16
    tie_inf = (2 - 2.0 ** -8) * 2.0 ** 127              # halfway to 2^128
    edge = [maxf, np.nextafter(maxf, np.inf), np.nextafter(tie_inf, 0), tie_inf,
            np.nextafter(tie_inf, np.inf), 2.0 ** 128, 1e300, float(np.finfo(np.float64).max),
            (2 - 2.0 ** -7) * 2.0 ** 126 + 2.0 ** 118,    # a tie below the top binade
            2.0 ** -126, np.nextafter(2.0 ** -126, 0), 2.0 ** -126 - 2.0 ** -134,
            2.0 ** -133, 2.0 ** -134, np.nextafter(2.0 ** -134, 1), np.nextafter(2.0 ** -134, 0),
            3 * 2.0 ** -134, 5 * 2.0 ** -134, 2.0 ** -140, 5e-324, 0.0, -0.0]
    edge += [-x for x in edge]
    rng = np.random.default_rng(17)
    sub = list(rng.integers(0, 2 ** 20, 1500) * 2.0 ** -147)           # across the subnormals
    sub += list((rng.integers(0, 2 ** 8, 500) * 2 + 1) * 2.0 ** -134)  # exact subnormal ties
    wide = list(np.ldexp(rng.uniform(1, 2, 3000), rng.integers(-1074, 1024, 3000)))
    wide = [x * (1 if s else -1) for x, s in zip(wide, rng.integers(0, 2, 3000))]
    top = list(np.ldexp(rng.uniform(1, 2, 1000), 127))                 # the top binade
    for x in edge + sub + wide + top:
        x = float(x)
        assert ora.f64_to_bf16_bits(x) == _bf16_bits_exact(x), x
    assert _bf16_bits_exact(maxf) == 0x7F7F and _bf16_bits_exact(tie_inf) == 0x7F80
    assert _bf16_bits_exact(np.nextafter(tie_inf, 0)) == 0x7F7F
    assert _bf16_bits_exact(2.0 ** -134) == 0 and _bf16_bits_exact(3 * 2.0 ** -134) == 2


# --------------------------------------------------------------------------
# the composed step
def test_decode_step_is_composition(ora):
    w = synth.LLAMA2_32K.replace(hq=4, hkv=2, n_ctx=3000, cap=3100, budget=64)
    lay = synth.make_layer(w, 0, "cpu")
    q, k, v = (synth.to_numpy_bits(lay[x]) for x in ("q", "k", "v"))
    codes = ora.encode_keys(k)
    out, out64, idx = ora.decode_step(q, k, v, codes, n_ctx=3000, budget=64)
    qc = ora.encode_keys(q[:, :, None, :])[:, :, 0]
    dist = ora.score(qc, codes, n_ctx=3000)
    idx2 = ora.select_topk(dist, 64)
    assert np.array_equal(idx, idx2)
    o2, o64 = ora.sparse_attend(q, k, v, idx2)
    assert np.array_equal(out, o2) and np.array_equal(out64, o64)


def test_decode_step_finds_planted_needles(ora):
    # sanity signal (not a parity bar): most planted needles survive selection
    w = synth.LLAMA2_32K.replace(hq=4, hkv=4, n_ctx=8192, cap=8192)
    lay = synth.make_layer(w, 0, "cpu")
    q, k, v = (synth.to_numpy_bits(lay[x]) for x in ("q", "k", "v"))
    codes = ora.encode_keys(k)
    _, _, idx = ora.decode_step(q, k, v, codes, n_ctx=8192, budget=256)
    found = sum(len(set(lay["needles"][0, h, 0]) & set(idx[0, h].tolist())) for h in range(4))
    assert found >= 0.75 * 4 * w.needles


# --------------------------------------------------------------------------
# ragged decode step with the new token appended (§3.1 cache, §2-§6 per sequence)
def _append_case(dtype, seed, B=4, Hq=4, Hkv=2, cap=40, d=64):
    import torch
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = synth.random_values((B, Hq, d), dt, seed)
    k = synth.random_values((B, Hkv, cap, d), dt, seed + 1)
    v = synth.random_values((B, Hkv, cap, d), dt, seed + 2)
    kn = synth.random_values((B, Hkv, d), dt, seed + 3)
    vn = synth.random_values((B, Hkv, d), dt, seed + 4)
    return [synth.to_numpy_bits(t) for t in (q, k, v, kn, vn)], dt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_step_full_budget_is_dense_attention(ora, dtype):
    # budget >= every sequence's rows: the step is exact softmax attention over
    # the sequence's first L_b cached rows plus the appended one, whatever the codes
    (q, k, v, kn, vn), dt = _append_case(dtype, 40)
    codes = ora.encode_keys(k)
    lens = np.array([0, 7, 39, 25], np.int32)
    out, out64, idx, k2, v2, c2 = ora.decode_append_step(q, k, v, codes, lens, 40, 64, kn, vn)
    f64 = lambda a: synth.bits_to_torch(a, dt).double().numpy()
    qd, kd, vd, knd, vnd = (f64(a) for a in (q, k, v, kn, vn))
    for b in range(4):
        L = int(lens[b])
        for h in range(4):
            kk = np.concatenate([kd[b, h // 2, :L], knd[b, h // 2][None]])
            vv = np.concatenate([vd[b, h // 2, :L], vnd[b, h // 2][None]])
            want = dense_attention(qd[b, h], kk, vv, 1 / math.sqrt(64))
            assert np.allclose(out64[b, h], want, rtol=1e-12, atol=1e-12)
            assert list(idx[b, h, :L + 1]) == list(range(L + 1))
            assert (idx[b, h, L + 1:] == -1).all()


def test_append_step_writes_only_the_next_row(ora):
    (q, k, v, kn, vn), _ = _append_case("bf16", 50)
    codes = ora.encode_keys(k)
    lens = np.array([3, 0, 39, 100], np.int32)   # the last one clamps to max_len - 1 = 39
    _, _, _, k2, v2, c2 = ora.decode_append_step(q, k, v, codes, lens, 40, 8, kn, vn)
    want_codes = ora.encode_keys(kn[:, :, None, :])[:, :, 0]
    for b, L in enumerate([3, 0, 39, 39]):
        assert np.array_equal(k2[b, :, L], kn[b]) and np.array_equal(v2[b, :, L], vn[b])
        assert np.array_equal(c2[b, :, L], want_codes[b])
        others = [t for t in range(40) if t != L]
        assert np.array_equal(k2[b][:, others], k[b][:, others])
        assert np.array_equal(v2[b][:, others], v[b][:, others])
        assert np.array_equal(c2[b][:, others], codes[b][:, others])


def test_append_step_alpha_encodes_the_new_key_per_head(ora):
    (q, k, v, kn, vn), _ = _append_case("f32", 70, Hkv=2)
    table = [0.2, 0.8]
    codes = ora.encode_keys(k, alpha=table)
    lens = np.array([5, 0, 39, 17], np.int32)
    r = ora.decode_append_step(q, k, v, codes, lens, 40, 8, kn, vn, alpha=table)
    c2 = r[5]
    for b, L in enumerate(lens):
        for h in range(2):
            assert np.array_equal(c2[b, h, L], ora.encode_vec(kn[b, h], alpha=table[h])[0])
        # the sequence's step is the alpha decode step over its own rows
        o, o64, ix = ora.decode_step(q[b:b + 1], r[3][b:b + 1], r[4][b:b + 1], c2[b:b + 1],
                                     int(L) + 1, 8, alpha=table)
        assert np.array_equal(r[2][b], ix[0]) and np.array_equal(r[1][b], o64[0])


def test_append_step_recent_window_and_empty_sequences(ora):
    (q, k, v, kn, vn), _ = _append_case("f32", 60)
    codes = ora.encode_keys(k)
    lens = np.array([30, 12, 0, 5], np.int32)
    # a recent window of one always keeps the appended token
    _, _, idx, *_ = ora.decode_append_step(q, k, v, codes, lens, 40, 4, kn, vn, n_recent=1)
    for b, L in enumerate(lens):
        assert (idx[b] == L).any(axis=-1).all()
    # nothing appended: an empty sequence gives zeros and no selection, the
    # others match the plain step over their own rows
    out, out64, idx, k2, _, _ = ora.decode_append_step(q, k, v, codes, lens, 40, 4)
    assert np.array_equal(k2, k)
    assert not out64[2].any() and (idx[2] == -1).all()
    for b, L in enumerate(lens):
        if L == 0:
            continue
        o, o64, ix = ora.decode_step(q[b:b + 1], k[b:b + 1], v[b:b + 1], codes[b:b + 1], int(L), 4)
        assert np.array_equal(ix[0], idx[b]) and np.array_equal(o64[0], out64[b])


def test_paged_step_matches_contiguous_layout(ora):
    # the paged oracle over a shuffled pool equals the contiguous append step
    # on the caches the page tables describe, and writes the new row into the
    # pool page the table names
    import torch
    B, Hq, Hkv, d, P = 2, 4, 2, 64, 1024
    pages_per_seq = 3
    rng = np.random.default_rng(3)
    q = synth.to_numpy_bits(synth.random_values((B, Hq, d), torch.bfloat16, 70))
    kc = synth.to_numpy_bits(synth.random_values((B, Hkv, pages_per_seq * P, d), torch.bfloat16, 71))
    vc = synth.to_numpy_bits(synth.random_values((B, Hkv, pages_per_seq * P, d), torch.bfloat16, 72))
    kn = synth.to_numpy_bits(synth.random_values((B, Hkv, d), torch.bfloat16, 73))
    vn = synth.to_numpy_bits(synth.random_values((B, Hkv, d), torch.bfloat16, 74))
    cc = ora.encode_keys(kc)
    n_pages = B * pages_per_seq + 2
    perm = rng.permutation(n_pages)[:B * pages_per_seq].reshape(B, pages_per_seq)
    kp = np.zeros((n_pages, Hkv, P, d), np.uint16)
    vp = np.zeros_like(kp)
    cp = np.zeros((n_pages, Hkv, P, d // 4), np.uint8)
    for b in range(B):
        for i in range(pages_per_seq):
            kp[perm[b, i]] = kc[b][:, i * P:(i + 1) * P]
            vp[perm[b, i]] = vc[b][:, i * P:(i + 1) * P]
            cp[perm[b, i]] = cc[b][:, i * P:(i + 1) * P]
    lens = np.array([2047, 1500], np.int32)       # the first appends at a page boundary
    out, out64, idx, kp2, vp2, cp2 = ora.decode_paged_step(q, kp, vp, cp, perm.astype(np.int32),
                                                           lens, 3 * P, 96, kn, vn)
    o_ref, o64_ref, idx_ref, k2, v2, c2 = ora.decode_append_step(q, kc, vc, cc, lens, 3 * P, 96,
                                                                 kn, vn)
    assert np.array_equal(idx, idx_ref) and np.array_equal(out64, o64_ref)
    for b in range(B):
        L = int(lens[b])
        pg, off = perm[b, L // P], L % P
        assert np.array_equal(kp2[pg][:, off], kn[b]) and np.array_equal(vp2[pg][:, off], vn[b])
        assert np.array_equal(cp2[pg][:, off], c2[b][:, L])
    changed = [(p, h, j) for p, h, j in zip(*np.nonzero((kp2 != kp).any(-1)))]
    assert sorted(changed) == sorted((perm[b, int(lens[b]) // P], h, int(lens[b]) % P)
                                     for b in range(B) for h in range(Hkv))


# --------------------------------------------------------------------------
# §2.2 grouped quantization: one absmax per 128 rotated dimensions
def test_encode_groups_of_128_hand_worked(ora):
    # Choose the rotated vector y directly and encode x = H y / 256 (exact:
    # H H = 256 I and every intermediate is a small multiple of 1/256).
    # y = [100, 1 x 127 | 2, -2, 2, -2, ...]: group 0 has absmax 100, so its
    # 1s (0 <= 1 < 50) code to 2 and the 100 to 3; group 1 has absmax 2, so
    # 2 >= 1 codes to 3 and -2 < -1 to 0.  Packed MSB-first: 3,2,2,2 -> 0xEA,
    # then 0xAA x 31, then 3,0,3,0 -> 0xCC x 32.  One absmax over the whole
    # vector would code group 1 as 2, 1 (0xA6...) instead.
    d = 256
    y = np.array([100] + [1] * 127 + [2, -2] * 64, np.int64)
    x = (sylvester(d) @ y).astype(np.float64) / d
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    p, yr, c = ora.encode_vec(x.astype(np.float32))
    assert np.array_equal(yr, y.astype(np.float32))
    assert bytes(p) == bytes([0xEA] + [0xAA] * 31 + [0xCC] * 32)


def test_encode_groups_are_independent(ora):
    # each 128-dim group of a 256-dim code depends only on its own rotated
    # values: scaling one group's rotated values leaves every code unchanged
    rng = np.random.default_rng(5)
    H = sylvester(256)
    for _ in range(50):
        y = rng.integers(-40, 41, 256)
        x1 = (H @ y).astype(np.float32) / 256
        y2 = y.copy()
        y2[128:] *= 3
        x2 = (H @ y2).astype(np.float32) / 256
        p1, _, c1 = ora.encode_vec(x1)
        p2, _, c2 = ora.encode_vec(x2)
        assert np.array_equal(c1, c2) and bytes(p1) == bytes(p2)


# --------------------------------------------------------------------------
# binary16 rotation variant (the article advises computing the rotation in FP16, §6)
def test_f64_to_f16_matches_numpy(ora):
    # numpy's double -> half conversion is an independent correctly rounded
    # implementation: ties, subnormals, the overflow edge, signs
    rng = np.random.default_rng(2)
    vals = [0.0, -0.0, 1.0, 2049.0, 2051.0, 4097.0, 65504.0, 65519.99, 65520.0, 1e6,
            2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -14 - 2.0 ** -26, 1.0 / 3]
    vals += list(rng.standard_normal(3000) * np.exp(rng.uniform(-18, 12, 3000)))
    for x in vals + [-v for v in vals]:
        got = ora.f64_to_f16_value(x)
        want = float(np.float16(x))
        assert got == want or (np.isinf(got) and np.isinf(want) and np.sign(got) == np.sign(want)), x


def test_fwht_f16_exact_on_small_integers(ora):
    # integers with |H x| <= 2048 stay exact in binary16: the binary16 rotation
    # gives the integer transform itself, and the codes of the fp32 rotation
    rng = np.random.default_rng(4)
    for d in (16, 64, 128):
        H = sylvester(d)
        for _ in range(20):
            x = rng.integers(-2048 // d, 2048 // d + 1, d).astype(np.float32)
            p16, y16, c16 = ora.encode_vec(x, rotate=2)
            p32, _, _ = ora.encode_vec(x)
            assert np.array_equal(y16, (H @ x.astype(np.int64)).astype(np.float32))
            assert bytes(p16) == bytes(p32)


def test_fwht_f16_rounding_hand_worked(ora):
    # d = 2, x = (3072, 1025), both exact binary16: the sum 4097 rounds to
    # 4096 (spacing 4 above 4096), the difference 2047 is exact.  x = (1025,
    # 0.5): the sum 1025.5 is a tie between 1025 and 1026 (spacing 1) and goes
    # to the even 1026; the difference 1024.5 ties to 1024.  x = (3072.625,
    # 1024.375) is first rounded to (3072, 1024) (spacings 2 and 1), so the
    # rotated pair is (4096, 2048) and both code to 3 (2048 >= 4096 / 2),
    # where the binary32 rotation gives (4097, 2048.25): codes 3 and 2.
    _, y, _ = ora.encode_vec(np.array([3072, 1025], np.float32), rotate=2)
    assert y.tolist() == [4096.0, 2047.0]
    _, y, _ = ora.encode_vec(np.array([1025, 0.5], np.float32), rotate=2)
    assert y.tolist() == [1026.0, 1024.0]
    x = np.array([3072.625, 1024.375, 0, 0], np.float32)
    _, y16, c16 = ora.encode_vec(x, rotate=2)
    _, y32, c32 = ora.encode_vec(x)
    assert y16.tolist() == [4096.0, 2048.0, 4096.0, 2048.0]
    assert c16.tolist() == [3, 3, 3, 3] and c32.tolist() == [3, 2, 3, 2]
