"""CPU oracle for the block-level objective of the search: the error is measured at the output of
the lowest common ancestor of the searched linears instead of at the linears' own outputs. For the
gate/up pair of a gated MLP (one fused set sharing the post-norm input) that ancestor is the MLP
block itself: y = down(act(x gate^T) * (x up^T)).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the CPU baseline leg
of the benchmark may import or run this module. The GPU library never calls it and shares no code
with it.

Pages cited below, by title and section:

* msModelSlim docs, "AWQ：激活感知权重量化算法说明": 原理 / 关键特性 (block-level error: the lowest
  common ancestor of the target modules is found, its inputs cached, and the quantization error is
  measured on its output rather than on a single linear), 缩放因子搜索流程 (float reference of the
  ancestor with the original weights; per ratio: scales, normalise, scale the target linears,
  quantize, inverse-scale, run the ancestor, mean squared error, restore; choose the minimum),
  支持的子图类型 (NormLinearSubgraph: all target linears share the search; UpDownSubgraph's example
  block y = down_proj(act(gate_proj(x)) * up_proj(x))).
* gsyq.cn, "AWQ 离群激活平滑实操", section 四: the SwiGLU gate and up projections must share one s.

Readings taken where the pages are silent:

* The block is the gated MLP with activation SiLU(v) = v / (1 + e^-v) (LLaMA's) or ReLU (the page's
  UpDown example); down_proj keeps its original weights while gate/up are searched.
* The loss is the mean over tokens and output features of the squared difference of the block's
  outputs, in float64; the selection is the main search's (first strict minimum, ones otherwise).
"""
from __future__ import annotations

import numpy as np

ACT_SILU = 0
ACT_RELU = 1


def act(v, kind: int) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    if kind == ACT_SILU:
        with np.errstate(over="ignore"):
            return v / (1.0 + np.exp(-v))
    if kind == ACT_RELU:
        return np.maximum(v, 0.0)
    raise ValueError(kind)


def mlp_hidden(X, Wg, Wu, kind: int = ACT_SILU) -> np.ndarray:
    """h = act(X Wg^T) * (X Wu^T), [n_tokens, d_ff]."""
    X = np.asarray(X, dtype=np.float64)
    return act(X @ np.asarray(Wg, np.float64).T, kind) * (X @ np.asarray(Wu, np.float64).T)


def mlp(X, Wg, Wu, Wd, kind: int = ACT_SILU) -> np.ndarray:
    """y = h Wd^T, [n_tokens, d_model]."""
    return mlp_hidden(X, Wg, Wu, kind) @ np.asarray(Wd, np.float64).T


def block_search(X, Wg, Wu, Wd, n_grid: int = 20, kind: int = ACT_SILU, group_size: int = 128):
    """The grid search with the MLP block as the scored module: per ratio, gate and up are scaled by
    the same s, quantized, inverse-scaled; the loss is mean((mlp_ref - mlp_k)^2)."""
    from oracle import awq_oracle as O
    X = np.asarray(X, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    Wu = np.asarray(Wu, dtype=np.float64)
    a = O.act_mean(X)
    y_ref = mlp(X, Wg, Wu, Wd, kind)
    scales, losses = [], []
    for r in O.grid_ratios(n_grid):
        s = O.candidate_scales(a, r)
        y = mlp(X, O.quantize_restore(Wg, s, group_size), O.quantize_restore(Wu, s, group_size), Wd, kind)
        scales.append(s)
        losses.append(float(np.mean((y_ref - y) ** 2)))
    k = O.select_best(losses)
    best = scales[k] if any(np.isfinite(losses)) else np.ones(X.shape[1])
    return np.stack(scales), np.array(losses), k, best


def _bf16(v) -> np.ndarray:
    """float64 -> float32 -> bfloat16 values, each rounding to nearest even (the sequence of a float32
    value stored as a bfloat16 operand)."""
    from oracle.awq_export import f32_to_bf16_rne
    bits = f32_to_bf16_rne(np.asarray(v, dtype=np.float64).astype(np.float32))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def block_losses_bf16_operands(X, Wg, Wu, Wd, scales, kind: int = ACT_SILU, group_size: int = 128,
                               round_operands: bool = True) -> np.ndarray:
    """The block losses of ``block_search`` computed through the difference form a bfloat16 matrix-core
    path takes: y_ref - y_k = dh_k Wd^T with dh_k = act(G) U - act(G + E_g)(U + E_u), G = X Wg^T,
    E_g = X dWg^T (likewise up), where the two GEMM operands that the path holds in bfloat16, the
    weight differences dW = What - W and the hidden difference dh, are rounded to bfloat16; everything
    else is float64. With ``round_operands=False`` it is the float64 difference form of the same
    losses. A diagnostic for how far those two specified roundings alone move the losses."""
    from oracle import awq_oracle as O
    X = np.asarray(X, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    Wu = np.asarray(Wu, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    rnd = _bf16 if round_operands else (lambda v: np.asarray(v, dtype=np.float64))
    G, U = X @ Wg.T, X @ Wu.T
    h_ref = act(G, kind) * U
    out = []
    for s in np.asarray(scales, dtype=np.float64):
        dWg = rnd(O.quantize_restore(Wg, s, group_size) - Wg)
        dWu = rnd(O.quantize_restore(Wu, s, group_size) - Wu)
        Eg, Eu = X @ dWg.T, X @ dWu.T
        dh = rnd(h_ref - act(G + Eg, kind) * (U + Eu))
        out.append(float(np.mean((dh @ Wd.T) ** 2)))
    return np.array(out)
