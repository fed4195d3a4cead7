"""CPU oracle for the steps either side of the AWQ search: the activation statistic gathered over
several calibration batches, folding the inverse scales into the source operator, and the compact
deployment form of the per-group quantization parameters.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the CPU baseline leg
of the benchmark may import or run this module. The GPU library never calls it and shares no code
with it.

Pages cited below, by title and section:

* msModelSlim docs, "AWQ：激活感知权重量化算法说明": 预处理阶段 (forward hooks collect the
  per-channel mean of |activation| while calibration batches run), 支持的子图类型 (after the
  search the norm gets the inverse scaling and the linears the forward scaling — norm-linear;
  linear1 inverse / linear2 forward — linear-linear; v_proj inverse / o_proj forward — ov;
  up_proj inverse / down_proj forward — up-down).
* gsyq.cn, "AWQ 离群激活平滑实操：逐通道等价缩放与 4-bit 精度无损转换", section 四 (fold
  diag(s)^-1 into the preceding normalisation so that the equivalence X W^T =
  (X diag(s)^-1)(W diag(s))^T holds without an extra operator).
* bjdmk.com.cn AWQ article, section "GPU 硬件级反量化算子内联融合" (deployment: packed 4-bit
  weights with FP16 per-group scales and offsets, unpacked from the low and high 4 bits).

Readings taken where the pages are silent:

* Statistic over batches: the mean over the concatenation of all batches, i.e. per-channel sums
  of |X| accumulated batch by batch and divided by the total token count once.
* Fold: row c of the source operator (the norm weight, or row c of the source linear's weight and
  its bias) is divided by s[c]. The quotient is formed in float64, rounded to float32 and then to
  the storage dtype (round to nearest even at each step), as a float32 computation stored in the
  model's dtype would round it.
* Output-value subgraph with grouped KV heads (MQA, GQA; MHA is the case of one query head per KV
  head): o_proj input channel (h, d) (query head h, head dimension d, channel h * head_dim + d) is
  the attention output of head h, a mix of the value rows of KV head h // g with
  g = n_heads / n_kv_heads (consecutive query heads share a KV head). Dividing v_proj output row
  (kv, d) by t scales every channel (h, d) with h // g = kv by 1 / t, so the forward scales of
  o_proj must be tied across the g query heads of a group: s[(h, d)] = t[(h // g, d)]. The search
  then runs on a tied statistic: channel (h, d) takes the mean, over the g query heads of its group
  in head order, of the per-channel means of |X| (the mean of |X| over all the entries one v_proj
  scale reaches); the candidate formula applied to it gives tied scales, and v_proj row (kv, d) is
  folded with the scale of channel (kv * g, d).
* Deployment form: each float32 step rounded to float16 (nearest even); zero points packed two per
  byte along the groups of a row, even group in the low nibble, clipped to [0, 15] (a zero point
  outside that range — only one-signed groups have one — is counted, since the packed form cannot
  hold it; the int32 zero points stay exact). Steps whose float16 value is not a normal number
  (below 2^-14 or overflowing) are counted too.
"""
from __future__ import annotations

import numpy as np


def act_sums(X) -> np.ndarray:
    """Per-channel sum of |X| over the tokens of one batch, in float64 (msModelSlim 预处理阶段)."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("X must be [tokens, d_in]")
    return np.abs(X).sum(axis=0)


def act_mean_batches(batches) -> np.ndarray:
    """Mean of |X| over all tokens of all batches: the batch sums added, then divided once."""
    total = None
    n = 0
    for X in batches:
        s = act_sums(X)
        total = s if total is None else total + s
        n += np.asarray(X).shape[0]
    if total is None or n == 0:
        raise ValueError("no tokens")
    return total / n


def f32_to_bf16_rne(v) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest even; NaN stays a quiet NaN."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def fold_scales(src, s, dtype: str):
    """Source-side inverse scaling: row c of ``src`` ([rows, cols]) divided by s[c].

    Returns the stored values: float32 for ``dtype == "f32"``, bfloat16 bits (uint16) for
    ``dtype == "bf16"``; the quotient is float64, rounded to float32, then to the dtype."""
    src = np.asarray(src, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if src.ndim == 1:
        src = src[:, None]
    if src.shape[0] != s.shape[0]:
        raise ValueError("one scale per source row")
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q32 = (src / s[:, None]).astype(np.float32)
    if dtype == "f32":
        return q32
    if dtype == "bf16":
        return f32_to_bf16_rne(q32)
    raise ValueError(dtype)


def export_fp16(qscales_f32, zeros):
    """Deployment form of the per-group parameters of a [rows, groups] export.

    Returns (steps as float16 bits [rows, groups] uint16, zero points packed two per byte
    [rows, ceil(groups / 2)] uint8, count of zero points outside [0, 15], count of steps whose
    float16 value is not a normal number)."""
    qs = np.asarray(qscales_f32, dtype=np.float32)
    z = np.asarray(zeros, dtype=np.int64)
    if qs.shape != z.shape or qs.ndim != 2:
        raise ValueError("qscales and zeros must both be [rows, groups]")
    with np.errstate(over="ignore", invalid="ignore"):
        h = qs.astype(np.float16)
    hb = h.view(np.uint16)
    with np.errstate(invalid="ignore"):
        bad_step = ~(np.isfinite(h) & (np.abs(h.astype(np.float32)) >= np.float32(2.0 ** -14)))
    zc = np.clip(z, 0, 15)
    bad_zero = z != zc
    rows, g = z.shape
    gp = (g + 1) // 2
    packed = np.zeros((rows, gp), dtype=np.uint8)
    packed |= zc[:, 0::2].astype(np.uint8)
    if g > 1:
        packed[:, : g // 2] |= (zc[:, 1::2].astype(np.uint8) << 4)
    return hb, packed, int(bad_zero.sum()), int(bad_step.sum())


def _head_groups(n_heads: int, n_kv_heads: int, head_dim: int) -> int:
    if n_heads < 1 or n_kv_heads < 1 or head_dim < 1 or n_heads % n_kv_heads:
        raise ValueError("n_heads must be a positive multiple of n_kv_heads")
    return n_heads // n_kv_heads


def tie_heads(act_mean, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Statistic of the o_proj input channels with each channel (h, d) replaced by the mean over
    the query heads sharing its KV head (msModelSlim 支持的子图类型, OVSubgraph: MHA, MQA, GQA;
    o_proj forward scaling, v_proj inverse). Sum in head order, divided once by the group size."""
    g = _head_groups(n_heads, n_kv_heads, head_dim)
    a = np.asarray(act_mean, dtype=np.float64)
    if a.shape != (n_heads * head_dim,):
        raise ValueError("act_mean must have n_heads * head_dim channels")
    a = a.reshape(n_kv_heads, g, head_dim)
    tot = a[:, 0, :].copy()
    for j in range(1, g):
        tot = tot + a[:, j, :]
    mean = tot / g
    return np.repeat(mean[:, None, :], g, axis=1).reshape(-1)


def head_group_scales(s, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Scales of the v_proj output rows: row (kv, d) takes o_proj channel (kv * g, d), the first
    query head of its group (all heads of a group carry the same tied scale)."""
    g = _head_groups(n_heads, n_kv_heads, head_dim)
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (n_heads * head_dim,):
        raise ValueError("s must have n_heads * head_dim channels")
    return s.reshape(n_kv_heads, g, head_dim)[:, 0, :].reshape(-1).copy()


def search_scales_tied(X, W, n_heads: int, n_kv_heads: int, head_dim: int, group_size: int = 128,
                       n_grid: int = 20):
    """The main search (msModelSlim 缩放因子搜索流程) on o_proj with the tied statistic: the
    candidate scales come from ``tie_heads(act_mean(X))``; quantizer, loss and choice unchanged."""
    from oracle import awq_oracle as O
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    a = tie_heads(O.act_mean(X), n_heads, n_kv_heads, head_dim)
    scales = np.stack([O.candidate_scales(a, r) for r in O.grid_ratios(n_grid)])
    losses = np.array([O.output_mse(X, W, O.quantize_restore(W, sk, group_size)) for sk in scales])
    k = O.select_best(losses)
    return O.SearchResult(a, O.grid_ratios(n_grid), scales, losses, k, scales[k].copy())
