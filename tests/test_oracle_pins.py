"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked values,
brute force over all 16 levels, closed forms, invariants, and an independently written
pure-Python loop version on tiny inputs.
"""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import awq_oracle as O
from oracle import naive as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_hand_groups():
    rows = []
    with open(os.path.join(GOLDEN, "hand_groups.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split(";")]
            rows.append(dict(id=parts[0], group=[float(v) for v in parts[1].split()],
                             scale=float(parts[2]), zero=float(parts[3]),
                             codes=[int(v) for v in parts[4].split()],
                             deq=[float(v) for v in parts[5].split()]))
    return rows


def _read_e1():
    kv = {}
    with open(os.path.join(GOLDEN, "e1_search.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = [p.strip() for p in line.split("=", 1)]
            kv[k] = v
    return kv


# ------------------------------------------------------------------ hand-worked values

@pytest.mark.parametrize("case", _read_hand_groups(), ids=lambda c: c["id"])
def test_hand_groups(case):
    y = np.array([case["group"]])
    qr = O.group_quantize(y, 4)
    assert qr.scale[0, 0] == case["scale"]
    assert qr.zero[0, 0] == case["zero"]
    assert qr.q[0].tolist() == case["codes"]
    deq = O.group_dequantize(qr.q, qr.scale, qr.zero, 4)
    assert deq[0].tolist() == case["deq"]
    # the loop version agrees
    codes, scale, zero = N.quantize_group(case["group"])
    assert (codes, scale, zero) == (case["codes"], case["scale"], case["zero"])


def test_e1_end_to_end():
    e = _read_e1()
    g, n = int(e["group_size"]), int(e["n_grid"])
    X = np.array([[float(v) for v in r.split()] for r in e["X"].split(";")])
    W = np.array([[float(v) for v in e["W"].split()]])
    res = O.search_scales(X, W, g, n)
    assert res.act_mean.tolist() == [float(v) for v in e["act_mean"].split()]
    assert res.scales[0].tolist() == [1.0] * 4
    assert res.scales[1].tolist() == [float(v) for v in e["scales_k1"].split()]
    np.testing.assert_allclose(res.losses, [float(v) for v in e["losses"].split()], rtol=1e-12)
    assert res.best_k == int(e["best_k"])
    pk = O.quantize_pack(W, res.best_scales, g)
    assert pk.q[0].tolist() == [int(v) for v in e["codes"].split()]
    assert [f"{b:02x}" for b in pk.codes[0]] == e["packed_hex"].split()
    assert pk.zeros[0, 0] == int(e["zero"]) and pk.qscales[0, 0] == float(e["scale"])
    a, losses, k = N.search(X.tolist(), W.tolist(), g, n)
    assert k == res.best_k
    np.testing.assert_allclose(losses, res.losses, rtol=1e-12)


# ------------------------------------------------------------------ candidate scales

def test_ratio_zero_gives_unit_scales():
    rng = np.random.default_rng(1)
    a = np.abs(rng.standard_normal(300)) * 5
    a[7] = 0.0
    a[11] = 1e-9
    s = O.candidate_scales(a, 0.0)
    assert np.all(s == 1.0)
    assert O.grid_ratios(20)[0] == 0.0


def test_scale_normalisation_and_ratio_law():
    """max(s)*min(s) == 1, s > 0, and s_c / s_c' == (a_c / a_c')^r wherever the 1e-4
    floor is inactive: this fixes both the exponent and the grid r = k / n_grid."""
    rng = np.random.default_rng(2)
    a = np.abs(rng.standard_normal(512)) + 0.05
    a[:5] *= 120.0
    X = rng.standard_normal((64, 512)) * a[None, :]
    W = rng.standard_normal((8, 512)) * 0.02
    res = O.search_scales(X, W, 128, 7)
    for k in range(7):
        s = res.scales[k]
        assert np.all(s > 0)
        assert abs(s.max() * s.min() - 1.0) < 1e-14
        r = k / 7
        i, j = int(np.argmax(res.act_mean)), int(np.argmin(res.act_mean))
        if k == 0:
            assert s[i] == s[j] == 1.0
        else:
            assert math.isclose(math.log(s[i] / s[j]), r * math.log(res.act_mean[i] / res.act_mean[j]),
                                rel_tol=1e-12)


def test_scale_floor_applies_before_normalisation():
    a = np.array([0.0, 1.0, 4.0, 10000.0])
    s = O.candidate_scales(a, 0.5)
    # a^0.5 = [0, 1, 2, 100] -> floor -> [1e-4, 1, 2, 100]; normaliser sqrt(100 * 1e-4) = 0.1
    np.testing.assert_allclose(s, [1e-3, 10.0, 20.0, 1000.0], rtol=1e-14)


# ------------------------------------------------------------------ quantizer: brute force and bounds

@pytest.mark.parametrize("g", [4, 8])
def test_codes_are_nearest_levels_bruteforce(g):
    """Each code is the nearest of the 16 levels (q - zero) * scale to y (ties excluded)."""
    rng = np.random.default_rng(3 + g)
    Y = rng.standard_normal((400, g)) * rng.uniform(0.01, 10, size=(400, 1)) + rng.uniform(-3, 3, (400, 1))
    qr = O.group_quantize(Y, g)
    levels = np.arange(16)
    for r in range(Y.shape[0]):
        sc, z = qr.scale[r, 0], qr.zero[r, 0]
        for c in range(g):
            d = np.abs((levels - z) * sc - Y[r, c])
            best = np.argsort(d)
            if d[best[1]] - d[best[0]] < 1e-9 * sc:
                continue
            assert qr.q[r, c] == best[0]


def test_codes_minimise_group_sse_exhaustive():
    """Over all 16^4 code vectors of a group, the element-wise codes minimise the squared
    reconstruction error for the group's (scale, zero)."""
    rng = np.random.default_rng(5)
    allq = np.array(list(itertools.product(range(16), repeat=4)), dtype=np.float64)
    for _ in range(6):
        y = rng.standard_normal(4) * rng.uniform(0.1, 4)
        qr = O.group_quantize(y[None, :], 4)
        sc, z = qr.scale[0, 0], qr.zero[0, 0]
        sse = (((allq - z) * sc - y[None, :]) ** 2).sum(axis=1)
        assert np.array_equal(allq[np.argmin(sse)].astype(np.int64), qr.q[0])


def test_quantizer_bounds_and_extremes():
    """Every dequantized value is within half a step of the input; the group minimum maps
    to code 0 and the maximum to 15 unless -min/scale is an exact tie."""
    rng = np.random.default_rng(6)
    Y = rng.standard_normal((2000, 128)) * rng.uniform(1e-3, 50, size=(2000, 1))
    qr = O.group_quantize(Y, 128)
    deq = O.group_dequantize(qr.q, qr.scale, qr.zero, 128)
    step = np.repeat(qr.scale, 128, axis=1)
    assert np.all(np.abs(deq - Y) <= 0.5 * step * (1 + 1e-12))
    assert qr.q.min() >= 0 and qr.q.max() <= 15
    tie = np.abs(qr.zt - np.floor(qr.zt) - 0.5) < 1e-9
    amin, amax = np.argmin(Y, axis=1), np.argmax(Y, axis=1)
    rows = np.arange(Y.shape[0])
    assert np.all(qr.q[rows, amin][~tie[:, 0]] == 0)
    assert np.all(qr.q[rows, amax][~tie[:, 0]] == 15)


def test_groups_are_row_local():
    """Groups are runs of consecutive input channels inside one row: permuting rows
    permutes the result, and each group sees only its own values."""
    rng = np.random.default_rng(7)
    Y = rng.standard_normal((6, 256))
    qr = O.group_quantize(Y, 128)
    perm = rng.permutation(6)
    qp = O.group_quantize(Y[perm], 128)
    assert np.array_equal(qp.q, qr.q[perm])
    Y2 = Y.copy()
    Y2[:, 128:] *= 1000.0
    q2 = O.group_quantize(Y2, 128)
    assert np.array_equal(q2.q[:, :128], qr.q[:, :128])


# ------------------------------------------------------------------ scaling direction and loss

def test_on_grid_weights_are_restored_exactly():
    """If W * s already lies on a 16-level grid, quantize-and-restore returns W. With
    power-of-two scales every product is exact, so this fixes the direction (multiply
    before quantizing, divide after)."""
    rng = np.random.default_rng(8)
    d_out, d_in, g = 5, 256, 128
    q = rng.integers(0, 16, size=(d_out, d_in))
    q[:, ::g] = 0
    q[:, 1::g] = 15
    step = 2.0 ** rng.integers(-8, -2, size=(d_out, d_in // g))
    zero = rng.integers(0, 16, size=(d_out, d_in // g)).astype(float)
    Y = O.group_dequantize(q, step, zero, g)
    s = 2.0 ** rng.integers(-3, 4, size=d_in)
    W = Y / s[None, :]
    assert np.array_equal(O.quantize_restore(W, s, g), W)
    assert not np.array_equal(O.quantize_restore(W, 1.0 / s, g), W)


def test_planted_optimum_is_selected():
    """Weights planted on the quantization grid of candidate k (up to rounding) have a
    near-zero loss at k, and the search picks k."""
    rng = np.random.default_rng(9)
    n_tok, d_in, d_out, g, n = 48, 256, 6, 128, 10
    X = rng.standard_normal((n_tok, d_in))
    X[:, [3, 150]] *= 40.0
    a = O.act_mean(X)
    k_plant = 6
    s = O.candidate_scales(a, k_plant / n)
    q = rng.integers(0, 16, size=(d_out, d_in))
    q[:, ::g] = 0
    q[:, 1::g] = 15
    Y = O.group_dequantize(q, np.full((d_out, d_in // g), 0.01), np.full((d_out, d_in // g), 8.0), g)
    W = Y / s[None, :]
    res = O.search_scales(X, W, g, n)
    assert res.best_k == k_plant
    assert res.losses[k_plant] < 1e-20 * res.losses.max()


def test_loss_equals_gram_form():
    """L_k = sum_o d_o (X^T X) d_o^T / (N d_out) with d = What - W: an independent route to
    the same number (fixes the normalisation and which operand is transposed)."""
    rng = np.random.default_rng(10)
    X = rng.standard_normal((40, 256))
    X[:, 9] *= 60.0
    W = rng.standard_normal((24, 256)) * 0.02
    res = O.search_scales(X, W, 128, 5)
    G = X.T @ X
    for k in range(5):
        d = O.quantize_restore(W, res.scales[k], 128) - W
        gram = float(np.einsum("oc,cd,od->", d, G, d)) / (X.shape[0] * W.shape[0])
        assert math.isclose(res.losses[k], gram, rel_tol=1e-10)


def test_equivalent_scaling_identity():
    """X W^T == (X diag(s)^-1)(W diag(s))^T (gsyq section 一), the identity the search relies on."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((16, 64))
    W = rng.standard_normal((8, 64))
    s = np.exp(rng.uniform(-3, 3, 64))
    np.testing.assert_allclose((X / s) @ (W * s).T, X @ W.T, rtol=1e-12, atol=1e-12)


def test_numpy_oracle_matches_loop_oracle():
    rng = np.random.default_rng(12)
    X = rng.standard_normal((20, 16))
    X[:, 5] *= 30.0
    W = rng.standard_normal((5, 16)) * 0.3
    res = O.search_scales(X, W, 8, 6)
    a, losses, k = N.search(X.tolist(), W.tolist(), 8, 6)
    np.testing.assert_allclose(a, res.act_mean, rtol=1e-14)
    np.testing.assert_allclose(losses, res.losses, rtol=1e-10)
    assert k == res.best_k


def test_act_mean_bruteforce():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((33, 12))
    got = O.act_mean(X)
    for c in range(12):
        assert math.isclose(got[c], sum(abs(X[i, c]) for i in range(33)) / 33, rel_tol=1e-14)
    with pytest.raises(ValueError):
        O.act_mean(np.zeros((0, 12)))


# ------------------------------------------------------------------ selection and packing

def test_select_best_rules():
    assert O.select_best([3.0, 1.0, 1.0, 2.0]) == 1
    assert O.select_best([float("nan"), 2.0, float("nan"), 1.5]) == 3
    assert O.select_best([float("nan")] * 4) == 0
    assert O.select_best([float("inf"), float("inf")]) == 0
    assert O.select_best([float("inf"), 5.0]) == 1
    assert O.select_best([2.0]) == 0


def test_pack_roundtrip_and_order():
    rng = np.random.default_rng(14)
    q = rng.integers(0, 16, size=(7, 256))
    p = O.pack_int4(q)
    assert p.shape == (7, 128) and p.dtype == np.uint8
    assert np.array_equal(O.unpack_int4(p), q)
    assert O.pack_int4(np.array([[1, 2]]))[0, 0] == 0x21
    with pytest.raises(ValueError):
        O.pack_int4(np.array([[16, 0]]))


def test_nonfinite_inputs_fall_back_to_unit_scales():
    """NaN in X: every candidate with r > 0 has NaN scales, r = 0 still has unit scales,
    every loss is NaN (the NaN activation reaches every output), so the search returns k = 0."""
    rng = np.random.default_rng(15)
    X = rng.standard_normal((16, 128))
    X[3, 7] = np.nan
    W = rng.standard_normal((4, 128))
    with np.errstate(invalid="ignore"):
        res = O.search_scales(X, W, 128, 4)
    assert np.all(res.scales[0] == 1.0)
    assert np.all(np.isnan(res.scales[1:]))
    assert np.all(np.isnan(res.losses))
    assert res.best_k == 0 and np.all(res.best_scales == 1.0)


def test_blocked_search_matches_gram_form_and_whole_search():
    """The token-blocked search (used for the full-size layers' stored results) against the
    Gram form and the whole search, with a ragged last block and float32 storage of X."""
    rng = np.random.default_rng(13)
    X = rng.standard_normal((300, 256)).astype(np.float32)
    X[:, 9] *= 60.0
    W = rng.standard_normal((40, 256)) * 0.02
    res = O.search_scales_blocked(X, W, 128, 7, block=64)
    whole = O.search_scales(X.astype(np.float64), W, 128, 7)
    np.testing.assert_allclose(res.act_mean, whole.act_mean, rtol=1e-14)
    np.testing.assert_array_equal(res.scales, whole.scales)
    np.testing.assert_allclose(res.losses, whole.losses, rtol=1e-12)
    assert res.best_k == whole.best_k
    X64 = X.astype(np.float64)
    G = X64.T @ X64
    for k in range(7):
        d = O.quantize_restore(W, res.scales[k], 128) - W
        gram = float(np.einsum("oc,cd,od->", d, G, d)) / (X.shape[0] * W.shape[0])
        assert math.isclose(res.losses[k], gram, rel_tol=1e-10)


def test_nonfinite_weight_groups():
    """A NaN weight makes its group's step NaN (max and min propagate NaN) and every restored value
    of the group NaN; an infinity makes the step infinite and the restored values NaN (0 * inf);
    stored codes and zero points of such groups are 0; other groups are untouched."""
    rng = np.random.default_rng(16)
    W = rng.standard_normal((3, 8)) * 0.1
    W[0, 1] = np.nan          # row 0, group 0
    W[1, 6] = np.inf          # row 1, group 1
    W[2, 2] = -np.inf         # row 2, group 0
    W[2, 3] = np.inf
    with np.errstate(invalid="ignore"):
        pq = O.quantize_pack(W, np.ones(8), 4)
        wh = O.quantize_restore(W, np.ones(8), 4)
    assert np.isnan(pq.qscales[0, 0]) and pq.qscales[1, 1] == np.inf and pq.qscales[2, 0] == np.inf
    for r, gi in ((0, 0), (1, 1), (2, 0)):
        assert np.all(pq.q[r, 4 * gi:4 * gi + 4] == 0) and pq.zeros[r, gi] == 0
        assert np.all(np.isnan(wh[r, 4 * gi:4 * gi + 4]))
    # the finite groups are quantized as usual
    for r, gi in ((0, 1), (1, 0), (2, 1)):
        ref = O.quantize_pack(W[r:r + 1, 4 * gi:4 * gi + 4], np.ones(4), 4)
        assert np.array_equal(pq.q[r, 4 * gi:4 * gi + 4], ref.q[0]) and pq.zeros[r, gi] == ref.zeros[0, 0]
        assert np.all(np.isfinite(wh[r, 4 * gi:4 * gi + 4]))
    # the search's losses are then NaN for every ratio, so the ones fallback is chosen
    X = rng.standard_normal((6, 8))
    with np.errstate(invalid="ignore"):
        res = O.search_scales(X, W, 4, 3)
    assert np.all(np.isnan(res.losses)) and res.best_k == 0 and np.all(res.best_scales == 1.0)


def test_zero_point_saturates_to_int32():
    # a constant one-signed group: step floor 1e-8, zero point -min/step = -5e8 fits; -50 gives -5e9
    W = np.array([[5.0, 5.0, 5.0, 5.0], [-50.0, -50.0, -50.0, -50.0]])
    pq = O.quantize_pack(W, np.ones(4), 4)
    assert pq.qscales[0, 0] == 1e-8 and pq.zeros[0, 0] == -500000000
    assert pq.zeros[1, 0] == 2 ** 31 - 1
