"""CPU oracle for the AWQ activation-aware scale search and INT4 group quantization.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import or run this module. The GPU library never
calls it and shares no code with it.

Everything is computed in float64 with numpy, step by step as the pages define it.

Pages cited below, by title and section:

* gsyq.cn, "AWQ 离群激活平滑实操：逐通道等价缩放与 4-bit 精度无损转换":
  section 一 (the equivalent-scaling identity), section 二 (``pseudo_quantize_int4``
  and ``search_smooth_scaling_factors``).
* bjdmk.com.cn AWQ article (weight-only W4A16): section "显著权重的识别" (the activation
  statistic S_X), section "数学等价变换与通道自适应缩放" (the loss L(s) and the grid
  search), section "GPU 硬件级反量化算子内联融合" (two 4-bit values per uint8 byte).
* qqiyuan.cn, "基于awq 4-bit量化技术的大模型推理优化实战": ``group_quantize`` /
  ``dequantize`` (uint8 codes, per-group scale and zero point returned).
* msModelSlim docs, "AWQ：激活感知权重量化算法说明": 原理 → 算法公式 (the candidate
  scale formula and the ratio grid), 缩放因子搜索流程 (the order of the search steps),
  YAML 配置字段详解 (``n_grid``, a positive integer, default 20).

Readings taken where the pages are silent, garbled or disagree:

* The statistic is the mean of |X| over all tokens, with no floor (msModelSlim 算法公式;
  bjdmk S_X). gsyq's extra ``clamp(min=1e-5)`` is not applied.
* Candidate scales: ``s = max(act_mean ** r, 1e-4)``, then ``s / sqrt(max(s) * min(s))``
  (msModelSlim 算法公式), for ``r = k / n_grid``, ``k = 0 .. n_grid - 1`` (the grid is [0, 1)).
* Quantizer: gsyq's asymmetric INT4 group quantizer, groups of ``group_size``
  consecutive input channels of one row: ``scale = max((max - min) / 15, 1e-8)``,
  ``zero = round(-min / scale)``, ``q = clip(round(y / scale) + zero, 0, 15)``;
  dequantized value ``(q - zero) * scale``. The extraction lost the ``+`` between
  ``round(w_flat / scale)`` and ``zero_point``; it is restored. ``round`` is
  round-half-to-even. The zero point is not clamped.
* Loss: the mean over all outputs of ``(X W^T - X What^T)^2`` with
  ``What = dequant(quant(W * s)) / s`` (gsyq section 二; bjdmk L(s)). For a fused set of
  linears sharing an input, ``W`` is the row-stack of their weights.
* Selection: scan the grid in order with a strict ``<`` from +inf; start from the
  all-ones scale (gsyq section 二; bjdmk ``if error < best_error``). So the lowest index
  among equal minima wins, NaN is never chosen, and if no loss is below +inf the result
  is ``k = 0``, whose scale is exactly all ones.
* Packing: along ``d_in``, element ``2j`` in the low nibble and ``2j+1`` in the high
  nibble of byte ``j`` (bjdmk names the low and high 4 bits, not their order).
* Non-finite weights: the group's max and min propagate NaN (as torch's and numpy's do), so
  a group holding a NaN has a NaN step and every restored value in it is NaN; an infinity
  gives an infinite step and NaN restored values (0 times infinity). A NaN code or zero point
  has no 4-bit value: the stored form writes it as 0. Zero points are stored as int32 and
  saturate to its range.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SCALE_FLOOR = 1e-4     # msModelSlim 算法公式: clamp(min=1e-4) on the candidate scales
QSCALE_FLOOR = 1e-8    # gsyq section 二: clamp(scale, min=1e-8) on the quantization step
QMAX = 15              # gsyq section 二: 4 bits, 16 levels, step (max - min) / 15


def act_mean(X) -> np.ndarray:
    """Per-input-channel mean of |X| over all tokens (bjdmk S_X; msModelSlim 算法公式)."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("X must be [tokens, d_in]")
    if X.shape[0] == 0:
        raise ValueError("no activation mean: zero calibration tokens")
    return np.abs(X).mean(axis=0)


def grid_ratios(n_grid: int) -> list[float]:
    """Ratios k / n_grid for k = 0 .. n_grid-1: the grid over [0, 1) (msModelSlim 算法公式)."""
    if int(n_grid) != n_grid or n_grid < 1:
        raise ValueError("n_grid must be a positive integer")
    return [k / n_grid for k in range(int(n_grid))]


def candidate_scales(act_mean_vec, ratio: float) -> np.ndarray:
    """One candidate: ``s = max(a ** r, 1e-4)``; ``s / sqrt(max(s) * min(s))``
    (msModelSlim 算法公式, both lines). NaN in ``a`` propagates to every channel when r > 0."""
    a = np.asarray(act_mean_vec, dtype=np.float64)
    s = np.maximum(np.power(a, ratio), SCALE_FLOOR)
    return s / math.sqrt(s.max() * s.min())


@dataclass
class GroupQuant:
    q: np.ndarray      # int64 codes [rows, d_in], in [0, 15]
    scale: np.ndarray  # float64 [rows, d_in / group]
    zero: np.ndarray   # float64, integer valued [rows, d_in / group]
    t: np.ndarray      # float64 pre-rounding y / scale [rows, d_in]
    zt: np.ndarray     # float64 pre-rounding -min / scale [rows, d_in / group]


def group_quantize(Y, group_size: int = 128) -> GroupQuant:
    """Asymmetric INT4 quantization of each run of ``group_size`` consecutive input
    channels of a row (gsyq section 二 ``pseudo_quantize_int4``; qqiyuan ``group_quantize``
    returns the uint8 codes with their scale and zero point)."""
    Y = np.asarray(Y, dtype=np.float64)
    rows, d = Y.shape
    if group_size < 1 or d % group_size:
        raise ValueError("d_in must be a multiple of group_size")
    g = Y.reshape(rows, d // group_size, group_size)
    mx = g.max(axis=-1, keepdims=True)
    mn = g.min(axis=-1, keepdims=True)
    scale = np.maximum((mx - mn) / QMAX, QSCALE_FLOOR)
    zt = -mn / scale
    zero = np.rint(zt)
    t = g / scale
    q = np.clip(np.rint(t) + zero, 0, QMAX)
    q = np.where(np.isnan(q), 0.0, q)  # no 4-bit value for a NaN code (non-finite group)
    return GroupQuant(q=q.reshape(rows, d).astype(np.int64), scale=scale[..., 0],
                      zero=zero[..., 0], t=t.reshape(rows, d), zt=zt[..., 0])


def group_dequantize(q, scale, zero, group_size: int = 128) -> np.ndarray:
    """``(q - zero) * scale`` per group (gsyq section 二; qqiyuan ``dequantize``)."""
    q = np.asarray(q, dtype=np.float64)
    rows, d = q.shape
    g = q.reshape(rows, d // group_size, group_size)
    out = (g - np.asarray(zero, np.float64)[..., None]) * np.asarray(scale, np.float64)[..., None]
    return out.reshape(rows, d)


def quantize_restore(W, s, group_size: int = 128) -> np.ndarray:
    """Scale W per input channel, quantize, dequantize, divide the scale back out:
    ``What = dequant(quant(W * s)) / s`` (gsyq section 二 ``restored_w``; msModelSlim
    缩放因子搜索流程, the apply / quantize / inverse-scale steps)."""
    W = np.asarray(W, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    qr = group_quantize(W * s[None, :], group_size)
    return group_dequantize(qr.q, qr.scale, qr.zero, group_size) / s[None, :]


def output_mse(X, W, W_hat) -> float:
    """Mean squared difference of the float and quantized layer outputs,
    ``mean((X W^T - X What^T)^2)`` (gsyq section 二; bjdmk L(s))."""
    X = np.asarray(X, dtype=np.float64)
    target = X @ np.asarray(W, dtype=np.float64).T
    actual = X @ np.asarray(W_hat, dtype=np.float64).T
    return float(np.mean((target - actual) ** 2))


def select_best(losses) -> int:
    """Strict-``<`` scan from +inf, keeping the first minimum; 0 if nothing is below +inf
    (gsyq section 二 ``best_loss = inf``, ``best_scale = ones``; bjdmk ``if error < best_error``)."""
    best_loss, best_k = math.inf, 0
    for k, loss in enumerate(losses):
        if loss < best_loss:
            best_loss, best_k = loss, k
    return best_k


def pack_int4(q) -> np.ndarray:
    """Two codes per byte along d_in: element 2j low nibble, 2j+1 high nibble
    (bjdmk "GPU 硬件级反量化算子内联融合")."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("d_in must be even to pack two codes per byte")
    if q.size and (q.min() < 0 or q.max() > QMAX):
        raise ValueError("codes must lie in [0, 15]")
    lo = q[..., 0::2].astype(np.uint8)
    hi = q[..., 1::2].astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


@dataclass
class SearchResult:
    act_mean: np.ndarray      # [d_in]
    ratios: list              # [n_grid]
    scales: np.ndarray        # [n_grid, d_in] candidate scales
    losses: np.ndarray        # [n_grid]
    best_k: int
    best_scales: np.ndarray   # [d_in]


def search_scales(X, W, group_size: int = 128, n_grid: int = 20) -> SearchResult:
    """The grid search in msModelSlim's order (缩放因子搜索流程): the activation mean,
    the float reference output, then for every ratio the candidate scales, their
    normalisation, scaling, quantization, inverse scaling and the output MSE; finally
    the ratio with the smallest MSE. Inputs are not modified (the restore step)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if X.shape[1] != W.shape[1]:
        raise ValueError("X and W disagree on d_in")
    a = act_mean(X)
    ratios = grid_ratios(n_grid)
    target = X @ W.T
    scales = np.empty((len(ratios), W.shape[1]))
    losses = np.empty(len(ratios))
    for k, r in enumerate(ratios):
        s = candidate_scales(a, r)
        W_hat = quantize_restore(W, s, group_size)
        actual = X @ W_hat.T
        scales[k] = s
        losses[k] = float(np.mean((target - actual) ** 2))
    k_best = select_best(losses)
    return SearchResult(a, ratios, scales, losses, k_best, scales[k_best].copy())


def search_scales_blocked(X, W, group_size: int = 128, n_grid: int = 20,
                          block: int = 4096) -> SearchResult:
    """``search_scales`` with the calibration tokens taken ``block`` rows at a time, for layers
    whose full output matrices do not fit in host memory at once. Same steps in the same
    order (msModelSlim 缩放因子搜索流程): the statistic (a sum of |X| over the blocks, divided
    once by the token count), the float reference ``X_b W^T`` of every block computed once and
    kept across the ratios, then per ratio the candidate scales, ``What``, and the output
    squared error summed block by block and divided by the number of outputs. Only the order
    of float64 additions differs from ``search_scales``. ``X`` is any array whose row slices
    convert to float64 (float32 holds bf16 values exactly)."""
    W = np.asarray(W, dtype=np.float64)
    n_tok, d_in = X.shape
    if d_in != W.shape[1]:
        raise ValueError("X and W disagree on d_in")
    if n_tok == 0:
        raise ValueError("no activation mean: zero calibration tokens")
    bounds = [(r0, min(n_tok, r0 + block)) for r0 in range(0, n_tok, block)]
    abs_sum = np.zeros(d_in)
    targets = []
    for r0, r1 in bounds:
        xb = np.asarray(X[r0:r1], dtype=np.float64)
        abs_sum += np.abs(xb).sum(axis=0)
        targets.append(xb @ W.T)
    a = abs_sum / n_tok
    ratios = grid_ratios(n_grid)
    scales = np.empty((len(ratios), d_in))
    losses = np.empty(len(ratios))
    n_out = n_tok * W.shape[0]
    for k, r in enumerate(ratios):
        s = candidate_scales(a, r)
        W_hat_t = quantize_restore(W, s, group_size).T
        sse = 0.0
        for (r0, r1), target in zip(bounds, targets):
            diff = target - np.asarray(X[r0:r1], dtype=np.float64) @ W_hat_t
            sse += float(np.einsum("ij,ij->", diff, diff))
        scales[k] = s
        losses[k] = sse / n_out
    k_best = select_best(losses)
    return SearchResult(a, ratios, scales, losses, k_best, scales[k_best].copy())


@dataclass
class PackedQuant:
    codes: np.ndarray    # uint8 [d_out, d_in / 2]
    qscales: np.ndarray  # float64 [d_out, d_in / group]
    zeros: np.ndarray    # int64 [d_out, d_in / group]
    q: np.ndarray        # int64 unpacked codes [d_out, d_in]
    t: np.ndarray        # pre-rounding y / scale, for tie bookkeeping
    zt: np.ndarray       # pre-rounding -min / scale


def quantize_pack(W, s, group_size: int = 128) -> PackedQuant:
    """Final export: codes of ``W * s`` packed two per byte, with per-group scale and zero
    (gsyq section 二 quantizer; qqiyuan ``group_quantize`` outputs; bjdmk packing)."""
    W = np.asarray(W, dtype=np.float64)
    qr = group_quantize(W * np.asarray(s, np.float64)[None, :], group_size)
    z = np.clip(np.where(np.isnan(qr.zero), 0.0, qr.zero), -2.0 ** 31, 2.0 ** 31 - 1)
    return PackedQuant(codes=pack_int4(qr.q), qscales=qr.scale, zeros=z.astype(np.int64),
                       q=qr.q, t=qr.t, zt=qr.zt)
