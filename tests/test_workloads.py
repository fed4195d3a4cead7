"""The seeded input generator: determinism, shapes, bf16 rounding, outlier structure, and
closed-form expectations of the activation statistic on the generated bulk channels."""
import hashlib
import math

import numpy as np
import pytest

from oracle import awq_oracle as O
from workloads import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_w, make_x,
                       outlier_channels, to_f32, workload)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20],
                    dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7], dtype=np.float32)
    np.testing.assert_array_equal(got, want)
    # idempotent on bf16 values
    b = f32_to_bf16_bits(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(b)), b)


def test_shapes_and_counts():
    expect = {1: 2, 2: 41, 3: 55, 4: 82, 5: 86}
    for cid, wl in WORKLOADS.items():
        idx, mult = outlier_channels(wl)
        assert len(idx) == expect[cid]
        assert np.all(np.diff(idx) > 0) and idx.max() < wl.d_in
        assert np.all((mult >= wl.outlier_lo) & (mult <= wl.outlier_hi))
        assert wl.d_in % wl.group_size == 0
    assert workload(3).d_in // 128 == 86


def test_deterministic_and_row_ranges():
    wl = workload(2)
    a = make_x(wl, row_range=(0, 700), threads=1)
    b = make_x(wl, row_range=(0, 700), threads=4)
    assert np.array_equal(a, b)
    c = make_x(wl, row_range=(300, 650))
    assert np.array_equal(c, a[300:650])
    w1 = make_w(wl, row_range=(100, 130))
    w2 = make_w(wl, row_range=(90, 140))
    assert np.array_equal(w1, w2[10:40])
    x1 = make_x(workload(1))
    assert x1.dtype == np.float32 and x1.shape == (512, 256)
    assert hashlib.sha256(x1.tobytes()).hexdigest() == hashlib.sha256(make_x(workload(1)).tobytes()).hexdigest()


def test_config5_weight_boost():
    wl = workload(5)
    w = to_f32(make_w(wl, row_range=(0, 64)))
    big = np.abs(w) > 6 * wl.w_std * 8 * 0.5
    # ~0.1% of entries carry the x8 boost
    frac = (np.abs(w) > 5.5 * wl.w_std).mean()
    assert 0.0002 < frac < 0.003
    assert big.any()


@pytest.mark.parametrize("cid,bulk", [
    (2, math.sqrt(2 / math.pi)),          # E|N(0,1)|
    (3, 1 / math.pi),                     # E|SiLU(a) b| = (E|a| / 2) E|b|, by sigma(a) + sigma(-a) = 1
    (4, math.sqrt(2 / math.pi)),
    (5, 0.2 * math.sqrt(3) / math.pi),    # 0.1 E|t_3| = 0.1 * 2 sqrt(3) / pi
])
def test_act_mean_closed_forms(cid, bulk):
    """The oracle's statistic on generated rows matches the closed-form expectation of the
    bulk channels, and outlier channels are their multiplier times the bulk value."""
    wl = workload(cid)
    rows = 2048 if wl.d_in <= 8192 else 512
    X = to_f32(make_x(wl, row_range=(0, rows)))
    a = O.act_mean(X)
    idx, mult = outlier_channels(wl)
    mask = np.ones(wl.d_in, bool)
    mask[idx] = False
    sd = {2: 0.603, 3: 0.45, 4: 0.603, 5: 0.134}[cid]  # std of |x| for one bulk element (rough)
    se = sd / math.sqrt(rows * mask.sum())
    assert abs(a[mask].mean() - bulk) < 6 * se + 2e-3 * bulk
    rel = a[idx] / (mult * bulk)
    assert np.all(np.abs(rel - 1) < 0.25)
