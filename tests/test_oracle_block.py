"""Pins for the block-level (MLP) objective oracle (oracle/awq_block.py): activation values, the
block by brute-force loops, the linearity the GPU path relies on, a lossless case and the ones
fallback (CPU only)."""
import math

import numpy as np

from oracle import awq_block as K
from oracle import awq_oracle as O


def test_activations():
    v = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = K.act(v, K.ACT_SILU)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)   # 0.7310585786...
    assert math.isclose(s[2], -1.0 / (1.0 + math.e), rel_tol=1e-15)
    assert math.isclose(s[3], 40.0, rel_tol=1e-15) and abs(s[4]) < 1e-15
    assert s[5] == 800.0 and s[6] == 0.0                                      # no overflow warning
    assert list(K.act(v, K.ACT_RELU)) == [0.0, 1.0, 0.0, 40.0, 0.0, 800.0, 0.0]


def test_mlp_by_brute_force():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 5))
    Wg, Wu, Wd = rng.standard_normal((4, 5)), rng.standard_normal((4, 5)), rng.standard_normal((2, 4))
    y = K.mlp(X, Wg, Wu, Wd, K.ACT_SILU)
    for i in range(3):
        for o in range(2):
            acc = 0.0
            for f in range(4):
                g = sum(X[i, c] * Wg[f, c] for c in range(5))
                u = sum(X[i, c] * Wu[f, c] for c in range(5))
                acc += (g / (1 + math.exp(-g))) * u * Wd[o, f]
            assert math.isclose(y[i, o], acc, rel_tol=1e-12, abs_tol=1e-12)


def test_output_difference_is_hidden_difference_times_down():
    # y_ref - y_k = (h_ref - h_k) Wd^T: the GPU scores the hidden difference with the error GEMM
    rng = np.random.default_rng(2)
    X = rng.standard_normal((16, 256))
    Wg, Wu = rng.standard_normal((64, 256)) * 0.05, rng.standard_normal((64, 256)) * 0.05
    Wd = rng.standard_normal((32, 64)) * 0.05
    s = O.candidate_scales(O.act_mean(X), 0.5)
    Wgh, Wuh = O.quantize_restore(Wg, s, 128), O.quantize_restore(Wu, s, 128)
    dy = K.mlp(X, Wg, Wu, Wd) - K.mlp(X, Wgh, Wuh, Wd)
    dh = K.mlp_hidden(X, Wg, Wu) - K.mlp_hidden(X, Wgh, Wuh)
    np.testing.assert_allclose(dy, dh @ Wd.T, rtol=1e-10, atol=1e-14)


def test_lossless_weights_choose_ratio_zero():
    # gate and up on the INT4 grid with power-of-two steps (every group spans the 16 levels): at
    # r = 0 (s = 1) quantization is exact, the block loss is 0, and the first minimum is k = 0
    rng = np.random.default_rng(3)
    X = rng.standard_normal((24, 256))
    X[:, 3] *= 30.0
    def on_grid(rows):
        q = rng.integers(0, 16, (rows, 256))
        q[:, 0::128], q[:, 1::128] = 0, 15
        z = rng.integers(0, 16, (rows, 2))
        return (q - np.repeat(z, 128, 1)) * 2.0 ** -6
    Wg, Wu = on_grid(8), on_grid(8)
    Wd = rng.standard_normal((4, 8))
    scales, losses, k, best = K.block_search(X, Wg, Wu, Wd, n_grid=4)
    assert losses[0] == 0.0 and k == 0 and np.all(best == 1.0)
    assert np.all(losses[1:] > 0)


def test_nonfinite_falls_back_to_ones():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((8, 128))
    X[2, 5] = np.nan
    W = rng.standard_normal((4, 128)) * 0.05
    with np.errstate(invalid="ignore"):
        _, losses, k, best = K.block_search(X, W, W, rng.standard_normal((3, 4)), n_grid=3)
    assert np.all(np.isnan(losses)) and k == 0 and np.all(best == 1.0)


def test_bf16_operand_losses_reduce_to_the_block_losses():
    """Without the operand roundings the difference form equals the block search's losses (the
    linearity of down_proj); with them, bfloat16 operands that are already exact change nothing."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((24, 128))
    X[:, 5] *= 30
    Wg, Wu = rng.standard_normal((64, 128)) * 0.05, rng.standard_normal((64, 128)) * 0.05
    Wd = rng.standard_normal((16, 64)) * 0.05
    for kind in (K.ACT_SILU, K.ACT_RELU):
        scales, losses, _, _ = K.block_search(X, Wg, Wu, Wd, 4, kind)
        diff = K.block_losses_bf16_operands(X, Wg, Wu, Wd, scales, kind, round_operands=False)
        np.testing.assert_allclose(diff, losses, rtol=1e-9)
        rounded = K.block_losses_bf16_operands(X, Wg, Wu, Wd, scales, kind)
        assert np.all(np.abs(rounded - losses) <= 5e-3 * losses)  # two roundings of 2^-9 each
    # round to nearest even at the bfloat16 precision: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    assert K._bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -9)])).tolist() == \
        [1.0, 1.0 + 2.0 ** -6, -1.0]
