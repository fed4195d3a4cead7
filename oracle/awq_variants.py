"""CPU oracle for the grid and quantizer variants the pages describe beside the main search:
the candidate-scale formulas of the three pages, arbitrary ratio grids, and two quantizers other
than the asymmetric INT4 group quantizer. The loss (output MSE) and the selection (first strict
minimum) are those of ``awq_oracle``.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the CPU baseline leg
of the benchmark may import or run this module. The GPU library never calls it and shares no code
with it.

Pages cited below, by title and section:

* msModelSlim docs, "AWQ：激活感知权重量化算法说明": 原理 / 算法公式 (``act_mean.pow(ratio)``
  floored at 1e-4, divided by ``sqrt(max * min)``; ratio over [0, 1) in steps of 1/n_grid), YAML
  配置示例 (``weight_qconfig``: per-channel, int8, symmetric, minmax).
* gsyq.cn, "AWQ 离群激活平滑实操：逐通道等价缩放与 4-bit 精度无损转换", section 二
  (``search_smooth_scaling_factors``: the statistic floored at 1e-5, ``alpha = 0, 0.1, ..., 1.0``,
  ``s = stat ** alpha``, divided by ``sqrt(mean(s ** 2))``, then floored at 1e-4).
* bjdmk.com.cn AWQ article, section "数学等价变换与通道自适应缩放" (``AWQChannelScaler``:
  ``weight_mean = mean |W|`` over the output rows, ``p`` over ``linspace(0, 1, steps)``,
  ``act_mean ** p / (weight_mean ** (1 - p) + 1e-6)`` floored at 1e-4, divided by
  ``sqrt(max * min)``; the quantizer takes each row's max and min, ``step = (max - min) / 15``, and
  rounds ``y / (step + 1e-6)`` to a multiple of ``step``, with no zero point and no clamp).

Readings taken where the pages are silent or garbled:

* Grids are given as explicit ratio lists: [0, 1) with step 1/n (msModelSlim), ``linspace(0, 1,
  n)`` = k / (n - 1) (bjdmk), and 0.1 steps over [0, 1] (gsyq).
* The per-channel symmetric int8 quantizer (msModelSlim's YAML names it without defining it):
  per output row ``step = max |y| / 127`` floored at 1e-8 (the floor of the INT4 quantizer),
  ``q = clip(round(y / step), -127, 127)``, dequantized ``q * step``.
* Rounding is to nearest even throughout; every quotient is an IEEE float64 division.
"""
from __future__ import annotations

import numpy as np

FORMULA_MSMODELSLIM = 0  # max(a^r, 1e-4) / sqrt(max * min)
FORMULA_RMS = 1          # max(max(a, 1e-5)^r / sqrt(mean(s^2)), 1e-4)  (gsyq)
FORMULA_DUO = 2          # max(a^r / (wm^(1-r) + 1e-6), 1e-4) / sqrt(max * min)  (bjdmk)

QUANT_INT4_GROUP = 0     # awq_oracle.group_quantize (gsyq pseudo_quantize_int4)
QUANT_INT4_ROW = 1       # bjdmk: per row, round(y / (step + 1e-6)) * step, no zero point
QUANT_INT8_ROW_SYM = 2   # msModelSlim weight_qconfig: per row, symmetric int8 min-max


def grid_ms(n: int) -> list[float]:
    """[0, 1) with step 1/n (msModelSlim)."""
    return [k / n for k in range(n)]


def grid_linspace(n: int) -> list[float]:
    """linspace(0, 1, n): k / (n - 1) (bjdmk); one point (0) when n == 1."""
    return [0.0] if n == 1 else [k / (n - 1) for k in range(n)]


def grid_tenths() -> list[float]:
    """0, 0.1, ..., 1.0 (gsyq)."""
    return [k / 10 for k in range(11)]


def weight_mean(W) -> np.ndarray:
    """Per-input-channel mean of |W| over the output rows (bjdmk ``weight.abs().mean(dim=0)``)."""
    W = np.asarray(W, dtype=np.float64)
    return np.abs(W).mean(axis=0)


def candidate_scales(formula: int, act_mean, ratio: float, w_mean=None) -> np.ndarray:
    a = np.asarray(act_mean, dtype=np.float64)
    r = float(ratio)
    if formula == FORMULA_MSMODELSLIM:
        s = np.maximum(a ** r, 1e-4)
        return s / np.sqrt(s.max() * s.min())
    if formula == FORMULA_RMS:
        s = np.maximum(a, 1e-5) ** r
        s = s / np.sqrt(np.mean(s ** 2))
        return np.maximum(s, 1e-4)
    if formula == FORMULA_DUO:
        wm = np.asarray(w_mean, dtype=np.float64)
        s = np.maximum(a ** r / (wm ** (1.0 - r) + 1e-6), 1e-4)
        return s / np.sqrt(s.max() * s.min())
    raise ValueError(formula)


def quantize_restore_row(Y, quantizer: int) -> np.ndarray:
    """Dequantized values of Y = W * s under one of the per-row quantizers (rows of Y)."""
    Y = np.asarray(Y, dtype=np.float64)
    if quantizer == QUANT_INT4_ROW:
        step = (Y.max(axis=1, keepdims=True) - Y.min(axis=1, keepdims=True)) / 15.0
        return np.rint(Y / (step + 1e-6)) * step
    if quantizer == QUANT_INT8_ROW_SYM:
        step = np.maximum(np.abs(Y).max(axis=1, keepdims=True) / 127.0, 1e-8)
        return np.clip(np.rint(Y / step), -127, 127) * step
    raise ValueError(quantizer)


def restore(W, s, quantizer: int, group_size: int = 128) -> np.ndarray:
    """What = dequant(quant(W * s)) / s for any quantizer."""
    from oracle import awq_oracle as O
    W = np.asarray(W, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if quantizer == QUANT_INT4_GROUP:
        return O.quantize_restore(W, s, group_size)
    return quantize_restore_row(W * s[None, :], quantizer) / s[None, :]


def search(X, W, ratios, formula: int = FORMULA_MSMODELSLIM, quantizer: int = QUANT_INT4_GROUP,
           group_size: int = 128):
    """The grid search over explicit ratios with a scale formula and a quantizer; loss and
    selection as the main oracle (output MSE, first strict minimum)."""
    from oracle import awq_oracle as O
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    a = O.act_mean(X)
    wm = weight_mean(W) if formula == FORMULA_DUO else None
    scales = np.stack([candidate_scales(formula, a, r, wm) for r in ratios])
    losses = [O.output_mse(X, W, restore(W, s, quantizer, group_size)) for s in scales]
    k = O.select_best(losses)
    # the pages start from best_scale = ones and keep it when no loss is below +inf
    best = scales[k] if any(np.isfinite(losses)) else np.ones(W.shape[1])
    return scales, np.array(losses), k, best
