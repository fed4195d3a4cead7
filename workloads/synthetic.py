"""Seeded synthetic layer inputs for the AWQ scale search.

Each workload is a calibration-activation matrix ``X [n_tokens, d_in]`` and a weight
matrix ``W [d_out, d_in]`` (the stacked rows of every linear that shares the input).
The activations follow the outlier structure the pages describe: a bulk of values of
magnitude about one, plus at most 1% "salient" input channels at fixed indices whose
magnitudes are tens to a couple of hundred times larger
(bjdmk.com.cn AWQ article, section "显著权重的识别：激活幅值的决定性地位";
gsyq.cn "AWQ 离群激活平滑实操", opening outlier diagram;
hncyxsy.com outlier essay, section 1.1 "把每一层激活…").

This module draws random numbers and rounds them to the storage dtype. It computes no
step of the method: both the CPU oracle and the GPU path receive the arrays it returns.

Generation is deterministic: numpy ``PCG64`` streams seeded by
``SeedSequence([seed, config_id, tensor_id, chunk])``, one stream per block of rows, so
any row range can be regenerated alone and blocks can be drawn in parallel threads.
Values are drawn in float32 and rounded once to bfloat16 (round to nearest even) for
the bf16 workloads; bf16 tensors are returned as their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

# tensor ids inside a config's seed sequence
_T_X, _T_X2, _T_OUTLIER, _T_W, _T_WBOOST = 0, 1, 2, 3, 4

_CHUNK_ELEMS = 1 << 21  # elements per seeded row block (rounded to whole rows)


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic layer."""

    config_id: int
    name: str
    n_tokens: int
    d_in: int
    d_out: int
    dtype: str  # "f32" or "bf16": storage dtype of X and W
    group_size: int
    n_grid: int
    x_kind: str  # "normal", "silu_gate", "student_t3"
    x_scale: float  # multiplier applied to the base distribution of X
    outlier_channels: int  # number of salient input channels
    outlier_lo: float  # per-channel multiplier drawn from U[lo, hi] (lo == hi: fixed)
    outlier_hi: float
    fixed_outlier_idx: tuple = ()  # explicit channel indices (overrides the random draw)
    w_std: float = 0.02
    w_boost_frac: float = 0.0  # fraction of W entries multiplied by w_boost
    w_boost: float = 1.0
    parts: tuple = ()  # row counts of the fused linears stacked in W (informational)

    @property
    def flops_per_candidate(self) -> int:
        return 2 * self.n_tokens * self.d_in * self.d_out


def _outlier_count(frac: float, d_in: int) -> int:
    return int(round(frac * d_in))


WORKLOADS: dict[int, Workload] = {
    1: Workload(1, "tiny-fp32", 512, 256, 256, "f32", 128, 20, "normal", 1.0,
                2, 50.0, 50.0, fixed_outlier_idx=(17, 200), w_std=0.02),
    2: Workload(2, "7b-qkv-fused", 4096, 4096, 12288, "bf16", 128, 20, "normal", 1.0,
                _outlier_count(0.01, 4096), 20.0, 150.0, w_std=0.02, parts=(4096, 4096, 4096)),
    3: Workload(3, "7b-down-proj", 16384, 11008, 4096, "bf16", 128, 20, "silu_gate", 1.0,
                _outlier_count(0.005, 11008), 10.0, 60.0, w_std=0.015),
    4: Workload(4, "70b-gate-up-fused", 8192, 8192, 57344, "bf16", 128, 20, "normal", 1.0,
                _outlier_count(0.01, 8192), 20.0, 180.0, w_std=0.01, parts=(28672, 28672)),
    5: Workload(5, "70b-down-proj-stress", 65536, 28672, 8192, "bf16", 128, 40, "student_t3", 0.1,
                _outlier_count(0.003, 28672), 50.0, 180.0, w_std=0.008,
                w_boost_frac=0.001, w_boost=8.0),
}


def workload(config_id: int) -> Workload:
    return WORKLOADS[config_id]


def custom_workload(n_tokens: int, d_in: int, d_out: int, dtype: str = "bf16", *,
                    group_size: int = 128, n_grid: int = 20, x_kind: str = "normal",
                    outlier_channels: int = 2, outlier_lo: float = 20.0,
                    outlier_hi: float = 150.0, w_std: float = 0.02,
                    config_id: int = 100, name: str = "custom") -> Workload:
    """A workload of arbitrary shape with the same value recipe (for ragged parity cases)."""
    return Workload(config_id, name, n_tokens, d_in, d_out, dtype, group_size, n_grid,
                    x_kind, 1.0, outlier_channels, outlier_lo, outlier_hi, w_std=w_std)


# ---------------------------------------------------------------- bf16 storage helpers

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(arr: np.ndarray) -> np.ndarray:
    """float32 view of a generated tensor (bf16 bit patterns are widened exactly)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)


def to_torch(arr: np.ndarray, device="cpu"):
    """torch tensor with the generated bytes (uint16 bit patterns become torch.bfloat16)."""
    import torch

    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


# ---------------------------------------------------------------- generation

def _rng(wl: Workload, seed: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.config_id, tensor_id, chunk])))


def _rows_per_chunk(d: int) -> int:
    return max(1, _CHUNK_ELEMS // d)


def outlier_channels(wl: Workload, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Sorted salient-channel indices and their per-channel multipliers."""
    if wl.fixed_outlier_idx:
        idx = np.array(sorted(wl.fixed_outlier_idx), dtype=np.int64)
        return idx, np.full(idx.shape, wl.outlier_lo, dtype=np.float32)
    g = _rng(wl, seed, _T_OUTLIER, 0)
    idx = np.sort(g.choice(wl.d_in, size=wl.outlier_channels, replace=False)).astype(np.int64)
    mult = g.uniform(wl.outlier_lo, wl.outlier_hi, size=idx.shape).astype(np.float32)
    return idx, mult


def _w_boost_entries(wl: Workload, seed: int) -> np.ndarray:
    n = int(round(wl.w_boost_frac * wl.d_out * wl.d_in))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    g = _rng(wl, seed, _T_WBOOST, 0)
    return np.sort(g.choice(wl.d_out * wl.d_in, size=n, replace=False)).astype(np.int64)


def _x_chunk(wl: Workload, seed: int, chunk: int, r0: int, r1: int, idx, mult) -> np.ndarray:
    g = _rng(wl, seed, _T_X, chunk)
    shape = (r1 - r0, wl.d_in)
    if wl.x_kind == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
    elif wl.x_kind == "silu_gate":
        a = g.standard_normal(shape, dtype=np.float32)
        b = _rng(wl, seed, _T_X2, chunk).standard_normal(shape, dtype=np.float32)
        x = (a / (np.float32(1.0) + np.exp(-a))) * b  # SiLU(a) * b, the gated-MLP activation
    elif wl.x_kind == "student_t3":
        x = g.standard_t(3.0, size=shape).astype(np.float32)
    else:
        raise ValueError(wl.x_kind)
    if wl.x_scale != 1.0:
        x *= np.float32(wl.x_scale)
    x[:, idx] *= mult[None, :]
    return x


def _w_chunk(wl: Workload, seed: int, chunk: int, r0: int, r1: int, boost) -> np.ndarray:
    g = _rng(wl, seed, _T_W, chunk)
    w = g.standard_normal((r1 - r0, wl.d_in), dtype=np.float32)
    w *= np.float32(wl.w_std)
    if boost.size:
        lo, hi = np.searchsorted(boost, [r0 * wl.d_in, r1 * wl.d_in])
        flat = boost[lo:hi] - r0 * wl.d_in
        w.reshape(-1)[flat] *= np.float32(wl.w_boost)
    return w


def _generate(wl: Workload, rows: int, d: int, row_range, make_chunk, threads) -> np.ndarray:
    r_lo, r_hi = (0, rows) if row_range is None else row_range
    if not (0 <= r_lo <= r_hi <= rows):
        raise ValueError(f"row range {row_range} outside [0, {rows}]")
    per = _rows_per_chunk(d)
    out = np.empty((r_hi - r_lo, d), dtype=np.uint16 if wl.dtype == "bf16" else np.float32)
    chunks = range(r_lo // per, (r_hi + per - 1) // per) if r_hi > r_lo else range(0)

    def one(c):
        c0, c1 = c * per, min(rows, (c + 1) * per)
        vals = make_chunk(c, c0, c1)
        a0, a1 = max(c0, r_lo), min(c1, r_hi)
        sl = vals[a0 - c0:a1 - c0]
        out[a0 - r_lo:a1 - r_lo] = f32_to_bf16_bits(sl) if wl.dtype == "bf16" else sl

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or len(chunks) <= 1:
        for c in chunks:
            one(c)
    else:
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, chunks))
    return out


def make_x(wl: Workload, seed: int = 0, row_range=None, threads: int | None = None) -> np.ndarray:
    """Calibration activations ``X [n_tokens, d_in]`` (uint16 bf16 bits, or float32)."""
    idx, mult = outlier_channels(wl, seed)
    return _generate(wl, wl.n_tokens, wl.d_in, row_range,
                     lambda c, r0, r1: _x_chunk(wl, seed, c, r0, r1, idx, mult), threads)


def make_w(wl: Workload, seed: int = 0, row_range=None, threads: int | None = None) -> np.ndarray:
    """Stacked weights ``W [d_out, d_in]`` (uint16 bf16 bits, or float32)."""
    boost = _w_boost_entries(wl, seed)
    return _generate(wl, wl.d_out, wl.d_in, row_range,
                     lambda c, r0, r1: _w_chunk(wl, seed, c, r0, r1, boost), threads)
