"""Comparison rules between the GPU results and the CPU oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (tests, smoke check and benchmark only).

Rules (floating point deciding an integer is compared where the decision is unique):
* act_mean within 1e-5 relative; per-ratio losses within 1e-3 relative.
* k*: equal to the oracle's, unless the oracle's own losses at the two indices differ by
  less than 1e-6 relative (then either is a correct minimum).
* INT4 codes and zero points bit-exact, except an element whose oracle pre-rounding value
  t = y/step lies within 1e-5 of a half-integer, and every element and the zero point of a
  group whose -min/step lies within 1e-5 of a half-integer (all of its codes shift with it).
* Per-group steps within 1e-6 relative of the oracle's float64 step (they are exported as
  float32).
* delta = What - W (an intermediate) element-wise within delta_tolerance below.
"""
from __future__ import annotations

import numpy as np

TIE_BAND = 1e-5
LOSS_RTOL = 1e-3
ACT_RTOL = 1e-5
KSTAR_RTOL = 1e-6
STEP_RTOL = 1e-6


def delta_tolerance(d_or, W, qscales, s, group_size: int = 128) -> np.ndarray:
    """Allowed |delta_gpu - delta_oracle| per element, where delta = What - W is an intermediate
    of the search (it feeds the error GEMM) and is stored in the input dtype:
    * 2^-8 |delta| for the bfloat16 rounding of the stored value;
    * 2^-16 step / s for evaluating t = y / step in float32: when every decision agrees with
      the float64 definition, |t32 - t| < 1.3e-5, so the restored value -(t - round t) step / s
      is that close in units of step / s;
    * 2^-40 |w| for forming delta as -(t - round t) step / s rather than What - W, which leaves a
      residue of order 1e-16 |w| where the oracle's difference is exactly zero (weights already
      on the quantization grid).
    Elements whose oracle decision sits within TIE_BAND of a rounding tie are exempt as usual."""
    step = np.repeat(np.asarray(qscales, np.float64), group_size, axis=1)
    return (2.0 ** -8 * np.abs(d_or) + 2.0 ** -16 * step / np.asarray(s, np.float64)[None, :]
            + 2.0 ** -40 * np.abs(W))


def near_half(v: np.ndarray, band: float = TIE_BAND) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return np.abs(v - np.floor(v) - 0.5) < band


def exempt_masks(t: np.ndarray, zt: np.ndarray, group_size: int = 128):
    """(element mask [rows, d_in], group mask [rows, groups]) of tie-exempt positions."""
    gm = near_half(zt)
    em = near_half(t) | np.repeat(gm, group_size, axis=1)
    return em, gm


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def max_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), 1e-300)
    return float(np.max(np.abs(a - b) / den)) if a.size else 0.0


def compare_codes(gpu_codes, gpu_qscales, gpu_zeros, oracle_pack, group_size: int = 128) -> dict:
    """Bit-exact comparison with tie exemptions. Returns counts; 'mismatch' must be 0."""
    q_gpu = unpack_codes(gpu_codes)
    em, gm = exempt_masks(oracle_pack.t, oracle_pack.zt, group_size)
    bad_codes = (q_gpu != oracle_pack.q) & ~em
    bad_zeros = (np.asarray(gpu_zeros, np.int64) != oracle_pack.zeros) & ~gm
    step_rel = np.abs(np.asarray(gpu_qscales, np.float64) - oracle_pack.qscales) / np.abs(oracle_pack.qscales)
    return {
        "elements": int(q_gpu.size),
        "exempt_elements": int(em.sum()),
        "exempt_groups": int(gm.sum()),
        "mismatch": int(bad_codes.sum()),
        "zero_mismatch": int(bad_zeros.sum()),
        "step_max_rel": float(step_rel.max()) if step_rel.size else 0.0,
        "raw_code_diff": int((q_gpu != oracle_pack.q).sum()),
    }


def kstar_ok(k_gpu: int, k_oracle: int, oracle_losses) -> bool:
    if k_gpu == k_oracle:
        return True
    lo = np.asarray(oracle_losses, np.float64)
    return bool(lo[k_gpu] <= lo[k_oracle] * (1 + KSTAR_RTOL))
