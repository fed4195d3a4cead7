"""Pins for the oracle of the grid and quantizer variants: hand-worked values, closed forms and
special cases that reduce to the main definitions (CPU only)."""
import math

import numpy as np
import pytest

from oracle import awq_oracle as O
from oracle import awq_variants as V


def test_grids():
    assert V.grid_ms(4) == [0.0, 0.25, 0.5, 0.75]
    assert V.grid_linspace(5) == [0.0, 0.25, 0.5, 0.75, 1.0]
    assert V.grid_linspace(1) == [0.0]
    assert V.grid_tenths()[0] == 0.0 and V.grid_tenths()[-1] == 1.0 and len(V.grid_tenths()) == 11


def test_msmodelslim_formula_is_the_main_one():
    a = np.array([0.5, 2.0, 7.0, 0.0])
    for r in (0.0, 0.3, 0.95):
        assert np.array_equal(V.candidate_scales(V.FORMULA_MSMODELSLIM, a, r), O.candidate_scales(a, r))


def test_rms_formula_hand_values():
    # a = [1, 4], r = 1/2: s = [1, 2] / sqrt((1 + 4) / 2)
    got = V.candidate_scales(V.FORMULA_RMS, np.array([1.0, 4.0]), 0.5)
    assert np.allclose(got, [1 / math.sqrt(2.5), 2 / math.sqrt(2.5)], rtol=1e-15)
    # r = 0 gives ones; the 1e-5 floor on the statistic, then the 1e-4 floor after normalising
    assert np.array_equal(V.candidate_scales(V.FORMULA_RMS, np.array([0.0, 3.0]), 0.0), [1.0, 1.0])
    got = V.candidate_scales(V.FORMULA_RMS, np.array([1e-12, 1.0]), 1.0)
    rms = math.sqrt((1e-10 + 1.0) / 2)
    assert got[0] == 1e-4 and math.isclose(got[1], 1.0 / rms, rel_tol=1e-15)


def test_duo_formula_closed_forms():
    a = np.array([0.5, 2.0, 8.0])
    wm = np.array([0.01, 0.02, 0.04])
    # r = 1: a / (1 + 1e-6), and the constant cancels in the normalisation
    got = V.candidate_scales(V.FORMULA_DUO, a, 1.0, wm)
    assert np.allclose(got, a / math.sqrt(a.max() * a.min()), rtol=1e-14)
    # r = 0: 1 / (wm + 1e-6), normalised
    t = 1.0 / (wm + 1e-6)
    assert np.allclose(V.candidate_scales(V.FORMULA_DUO, a, 0.0, wm), t / math.sqrt(t.max() * t.min()), rtol=1e-14)
    # the 1e-4 floor applies before normalising: a = [0, 1], r = 1
    got = V.candidate_scales(V.FORMULA_DUO, np.array([0.0, 1.0]), 1.0, np.array([1.0, 1.0]))
    f = 1.0 / (1 + 1e-6)
    assert np.allclose(got, np.array([1e-4, f]) / math.sqrt(1e-4 * f), rtol=1e-14)


def test_weight_mean():
    assert np.array_equal(V.weight_mean([[1.0, -2.0], [-3.0, 6.0]]), [2.0, 4.0])


def test_int4_row_quantizer_hand_values():
    # step = 7.5 / 15 = 0.5; y / 0.500001 rounds to [-3, 1, 2, 12]
    y = np.array([[-1.5, 0.3, 1.0, 6.0]])
    assert np.array_equal(V.quantize_restore_row(y, V.QUANT_INT4_ROW), [[-1.5, 0.5, 1.0, 6.0]])
    # the + 1e-6 in the divisor moves an exact half: 0.75 / 0.500001 < 1.5 -> 1 (not 2)
    y = np.array([[-1.5, 0.75, 6.0]])
    assert np.array_equal(V.quantize_restore_row(y, V.QUANT_INT4_ROW), [[-1.5, 0.5, 6.0]])


def test_int8_symmetric_quantizer_hand_values():
    # max |y| = 31.75 -> step 0.25; 1.125 / 0.25 = 4.5 -> 4 (half to even), 0.375 -> 1.5 -> 2
    y = np.array([[-31.75, 1.125, 0.375]])
    assert np.array_equal(V.quantize_restore_row(y, V.QUANT_INT8_ROW_SYM), [[-31.75, 1.0, 0.5]])
    # all-zero row: the 1e-8 floor, zeros restored
    assert np.array_equal(V.quantize_restore_row(np.zeros((1, 4)), V.QUANT_INT8_ROW_SYM), np.zeros((1, 4)))
    # brute force: each code is the nearest level in [-127, 127]
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 50))
    q = V.quantize_restore_row(y, V.QUANT_INT8_ROW_SYM)
    step = np.abs(y).max(axis=1, keepdims=True) / 127
    levels = np.arange(-127, 128)[None, None, :] * step[:, :, None]   # [3, 1, 255]
    idx = np.abs(levels - y[:, :, None]).argmin(-1)                     # [3, 50]
    nearest = np.take_along_axis(levels[:, 0, :], idx, axis=1)
    assert np.allclose(q, nearest, rtol=0, atol=1e-15)


def test_restore_dispatch_and_scaling_direction():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((4, 256)) * 0.02
    s = 2.0 ** rng.integers(-3, 4, 256)
    assert np.array_equal(V.restore(W, s, V.QUANT_INT4_GROUP), O.quantize_restore(W, s, 128))
    # on-grid rows restore exactly: with power-of-two scales (W * s) / s is exact
    grid = np.round(rng.standard_normal((2, 256)) * 20) * 0.25
    grid[:, 0] = 127 * 0.25  # max |y| = 31.75 -> step 0.25 exactly
    Wg = grid / s
    assert np.array_equal(V.restore(Wg, s, V.QUANT_INT8_ROW_SYM), Wg)


def test_search_variants_run_and_fall_back_to_ones():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((64, 256))
    X[:, 7] *= 40
    W = rng.standard_normal((32, 256)) * 0.02
    for formula, grid in ((V.FORMULA_RMS, V.grid_tenths()), (V.FORMULA_DUO, V.grid_linspace(6))):
        for quant in (V.QUANT_INT4_GROUP, V.QUANT_INT4_ROW, V.QUANT_INT8_ROW_SYM):
            scales, losses, k, best = V.search(X, W, grid, formula, quant)
            assert np.all(np.isfinite(losses)) and losses[k] == losses.min()
            assert np.array_equal(best, scales[k])
    Xn = X.copy()
    Xn[0, 3] = np.nan
    scales, losses, k, best = V.search(Xn, W, V.grid_linspace(3), V.FORMULA_DUO, V.QUANT_INT4_ROW)
    assert k == 0 and np.all(np.isnan(losses)) and np.array_equal(best, np.ones(256))


def test_int4_row_codes_are_nearest_multiples_brute_force():
    # q = round(y / (step + 1e-6)) is the integer j nearest to y / (step + 1e-6): brute force over j
    rng = np.random.default_rng(6)
    y = rng.standard_normal((4, 64)) * np.array([[0.1], [1.0], [3.0], [0.01]])
    step = (y.max(axis=1, keepdims=True) - y.min(axis=1, keepdims=True)) / 15.0
    d = step + 1e-6
    js = np.arange(-40, 41)[None, None, :]
    best_j = np.take_along_axis(np.broadcast_to(js, y.shape + (81,)),
                                np.abs(js * d[:, :, None] - y[:, :, None]).argmin(-1)[..., None], -1)[..., 0]
    assert np.array_equal(V.quantize_restore_row(y, V.QUANT_INT4_ROW), best_j * step)
    # every row spans 16 consecutive integers at most (max - min = 15 steps)
    q = best_j
    assert np.all(q.max(axis=1) - q.min(axis=1) <= 15)


def test_rms_formula_unit_mean_square_and_ratio_law():
    rng = np.random.default_rng(8)
    a = np.exp(rng.normal(0, 1, 300))
    for r in (0.2, 0.5, 0.9):
        s = V.candidate_scales(V.FORMULA_RMS, a, r)
        assert s.min() > 1e-4  # no floor active on these values
        assert math.isclose(float(np.mean(s ** 2)), 1.0, rel_tol=1e-13)
        assert np.allclose(s[1:] / s[0], (a[1:] / a[0]) ** r, rtol=1e-12)


def test_weight_mean_brute_force_over_stacked_rows():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((7, 5))
    want = [sum(abs(W[o, c]) for o in range(7)) / 7 for c in range(5)]
    assert np.allclose(V.weight_mean(W), want, rtol=1e-15)
