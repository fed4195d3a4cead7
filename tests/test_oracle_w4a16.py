"""Pins for the W4A16 consumer oracle (oracle/awq_w4a16.py): hand-worked dequantization, the
round trip from the search's own quantizer through the deployment form, rounding to the 16-bit
operand, and the product by brute force (CPU only)."""
import numpy as np

from oracle import awq_export as XP
from oracle import awq_oracle as O
from oracle import awq_w4a16 as Q


def _deploy(codes_q, steps, zeros):
    """Hand-built deployment form from unpacked codes [rows, d_in], float16 steps and int zeros."""
    rows, d_in = codes_q.shape
    codes = (codes_q[:, 0::2] | (codes_q[:, 1::2] << 4)).astype(np.uint8)
    sb = np.asarray(steps, np.float16).view(np.uint16)
    g = d_in // 128
    zp = np.zeros((rows, (g + 1) // 2), np.uint8)
    zp |= zeros[:, 0::2].astype(np.uint8)
    if g > 1:
        zp[:, : g // 2] |= zeros[:, 1::2].astype(np.uint8) << 4
    return codes, sb, zp


def test_hand_dequantization_and_nibble_order():
    q = np.zeros((1, 256), np.int64)
    q[0, :4] = [3, 12, 0, 15]          # byte 0 = 0xC3, byte 1 = 0xF0
    q[0, 128:130] = [9, 1]
    codes, sb, zp = _deploy(q, np.array([[0.5, 0.25]]), np.array([[8, 1]]))
    assert codes[0, 0] == 0xC3 and codes[0, 1] == 0xF0 and zp[0, 0] == 0x18
    w = Q.dequant_deploy(codes, sb, zp, 256, "bf16")
    assert list(w[0, :4]) == [-2.5, 2.0, -4.0, 3.5]          # (q - 8) * 0.5
    assert list(w[0, 128:130]) == [2.0, 0.0]                  # (q - 1) * 0.25
    assert w[0, 5] == -4.0 and w[0, 200] == -0.25             # code 0 elsewhere


def test_rounding_to_the_operand_type():
    # (15 - 0) * step with step = 1 + 2^-10 (a float16 value): 15 + 15 * 2^-10 = 15.0146484375
    # needs 14 significant bits: bfloat16 keeps 8 (-> 15.0), float16 keeps 11 (-> 15.015625)
    q = np.zeros((1, 128), np.int64)
    q[0, 0] = 15
    codes, sb, zp = _deploy(q, np.array([[1 + 2 ** -10]]), np.array([[0]]))
    assert Q.dequant_deploy(codes, sb, zp, 128, "bf16")[0, 0] == 15.0
    assert Q.dequant_deploy(codes, sb, zp, 128, "f16")[0, 0] == 15.015625
    # a tie in bfloat16: 3 * (1 + 2^-8) = 3 + 3 * 2^-8 = 0b11.00000011 -> 9 significant bits,
    # halfway between 3.0078125 and 3.015625; nearest even keeps 3.015625
    q[0, 0] = 3
    codes, sb, zp = _deploy(q, np.array([[1 + 2 ** -8]]), np.array([[0]]))
    assert Q.dequant_deploy(codes, sb, zp, 128, "bf16")[0, 0] == 3.015625


def test_round_trip_from_the_search_quantizer():
    # power-of-two steps are exact in float16 and the dequantized values exact in bfloat16, so the
    # deployment chain reproduces (q - zero) * step of the main quantizer exactly
    rng = np.random.default_rng(3)
    rows, d_in = 6, 512
    step = 2.0 ** rng.integers(-8, -3, (rows, d_in // 128))
    zero = rng.integers(0, 16, (rows, d_in // 128))
    q = rng.integers(0, 16, (rows, d_in))
    q[:, 0::128], q[:, 1::128] = 0, 15  # every group spans the 16 levels: the quantizer finds step again
    W = (q - np.repeat(zero, 128, 1)) * np.repeat(step, 128, 1)
    pk = O.quantize_pack(W, np.ones(d_in), 128)
    hb, zu4, bad_z, bad_s = XP.export_fp16(pk.qscales.astype(np.float32), pk.zeros)
    assert bad_z == 0 and bad_s == 0
    w_hat = Q.dequant_deploy(pk.codes, hb, zu4, d_in, "bf16")
    assert np.array_equal(w_hat, O.group_dequantize(O.unpack_int4(pk.codes), pk.qscales, pk.zeros, 128))
    assert np.array_equal(w_hat, W)


def test_product_by_brute_force_and_the_scaling_identity():
    rng = np.random.default_rng(4)
    n, rows, d_in = 3, 4, 256
    q = rng.integers(0, 16, (rows, d_in))
    z = rng.integers(0, 16, (rows, 2))
    st = np.float16(2.0 ** -5) * (1 + rng.integers(0, 1024, (rows, 2)) / 1024.0).astype(np.float16)
    codes, sb, zp = _deploy(q, st, z)
    X = rng.standard_normal((n, d_in)).astype(np.float32).astype(np.float64)
    Y = Q.w4a16_matmul(X, codes, sb, zp, "f16")
    w = Q.dequant_deploy(codes, sb, zp, d_in, "f16")
    for i in range(n):
        for o in range(rows):
            assert abs(Y[i, o] - sum(X[i, c] * w[o, c] for c in range(d_in))) < 1e-12
    # the consumer of an export of W * s fed X / s approximates X W^T within the quantization error
    Wt = rng.standard_normal((rows, d_in)) * 0.02
    s = np.exp(rng.normal(0, 0.5, d_in))
    pk = O.quantize_pack(Wt, s, 128)
    hb, zu4, _, _ = XP.export_fp16(pk.qscales.astype(np.float32), pk.zeros)
    Xs = X / s[None, :]
    Y = Q.w4a16_matmul(Xs, pk.codes, hb, zu4, "f16")
    bound = np.abs(Xs) @ np.repeat(pk.qscales, 128, 1).T  # one step per input, generous
    assert np.all(np.abs(Y - X @ Wt.T) <= bound)


def test_abs_product_sums():
    q = np.full((2, 128), 3, np.int64)
    codes, sb, zp = _deploy(q, np.array([[0.5], [1.0]]), np.array([[1], [5]]))
    X = np.array([[1.0] * 128, [-2.0] * 128])
    np.testing.assert_array_equal(Q.abs_product_sums(X, codes, sb, zp), [[128.0, 256.0], [256.0, 512.0]])
