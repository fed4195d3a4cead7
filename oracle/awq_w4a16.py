"""CPU oracle for the inference consumer of the export: the W4A16 product Y = X * W_hat^T, where
W_hat is dequantized on the fly from the deployment form (4-bit codes two per byte, float16
per-group steps, 4-bit zero points two per byte).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the CPU baseline leg
of the benchmark may import or run this module. The GPU library never calls it and shares no code
with it.

Pages cited below, by title and section:

* bjdmk.com.cn AWQ article, section "GPU 硬件级反量化算子内联融合": the packed 4-bit weights are
  brought in with wide loads, split into their low and high 4 bits, converted to floating point,
  scaled by the per-group FP16 scale with its offset, and fed to the matrix units together with the
  16-bit activations; the weights are never written out in 16-bit form.
* qqiyuan.cn, "基于awq 4-bit量化技术的大模型推理优化实战": ``dequantize`` is ``(q - zero) * scale``.
* gsyq.cn, "AWQ 离群激活平滑实操", section 一: ``X W^T = (X diag(s)^-1)(W diag(s))^T`` — the codes
  hold W * s, so the consumer is fed the activations already divided by s.

Readings taken where the pages are silent:

* The dequantized weight is ``(q - zero) * step`` with the float16 step, computed exactly (a 4-bit
  integer times an 11-bit mantissa is exact in float32 and float64) and rounded once, to nearest
  even, to the type of the activations (bfloat16 or float16): the matrix units take both operands
  in one 16-bit type. The page's scale-and-offset form ``q * scale - zero * scale`` is the same
  value before that rounding.
* Codes are those of the export: element 2j of a row in the low 4 bits of byte j; zero points of
  groups 2i and 2i+1 in the low and high 4 bits of byte i of the row's zero bytes.
* The product is accumulated exactly here (float64 over exactly representable products); the GPU
  accumulates in float32, so parity allows the float32 accumulation error (the tests derive the
  bound), except on inputs whose sums are exact in float32, which must match bit for bit.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def unpack_nibbles(packed, n: int) -> np.ndarray:
    """[rows, ceil(n/2)] uint8 -> [rows, n] int64: element 2j from the low 4 bits of byte j."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out[..., :n]


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to_operand(v, operand: str) -> np.ndarray:
    """float64 values (exact in float32) -> the value after rounding to bfloat16 or float16,
    nearest even, returned as float64."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), np.asarray(v, dtype=np.float64)):
        raise ValueError("the dequantized value must be exact in float32 before rounding")
    if operand == "f16":
        with np.errstate(over="ignore"):
            return v32.astype(np.float16).astype(np.float64)
    if operand == "bf16":
        u = v32.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(operand)


def dequant_deploy(codes, steps_f16, zeros_u4, d_in: int, operand: str = "bf16") -> np.ndarray:
    """W_hat [rows, d_in] (float64 holding the 16-bit operand values) from the deployment form:
    (q - zero) * step per group of 128 consecutive inputs, rounded to the operand type."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    if d_in % GROUP or codes.shape[1] * 2 != d_in:
        raise ValueError("codes must be [rows, d_in / 2] with d_in a multiple of 128")
    g = d_in // GROUP
    q = unpack_nibbles(codes, d_in)                               # [rows, d_in]
    z = unpack_nibbles(zeros_u4, g)                               # [rows, g]
    step = f16_bits_to_f64(steps_f16).reshape(rows, g)            # [rows, g]
    exact = (q - np.repeat(z, GROUP, axis=1)) * np.repeat(step, GROUP, axis=1)
    return round_to_operand(exact, operand)


def w4a16_matmul(X, codes, steps_f16, zeros_u4, operand: str = "bf16") -> np.ndarray:
    """Y = X * W_hat^T in float64, X [n_tokens, d_in] holding 16-bit values."""
    X = np.asarray(X, dtype=np.float64)
    W_hat = dequant_deploy(codes, steps_f16, zeros_u4, X.shape[1], operand)
    return X @ W_hat.T


def abs_product_sums(X, codes, steps_f16, zeros_u4, operand: str = "bf16") -> np.ndarray:
    """sum_c |X[n, c]| |W_hat[o, c]| per output: the scale of the float32 accumulation error."""
    X = np.asarray(X, dtype=np.float64)
    W_hat = dequant_deploy(codes, steps_f16, zeros_u4, X.shape[1], operand)
    return np.abs(X) @ np.abs(W_hat).T
