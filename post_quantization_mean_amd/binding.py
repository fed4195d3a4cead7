"""Thin Python binding of libawq_mi355x.so (include/awq.h).

Every function has the name of the C entry point it calls and only marshals arguments:
torch supplies device memory (tensors, workspaces) and the stream; every step of the
computation runs in the library's HIP kernels. If the library is missing the functions
raise instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libawq_mi355x.so")

AWQ_OK = 0
AWQ_DTYPE_F32 = 0
AWQ_DTYPE_BF16 = 1
AWQ_DTYPE_F16 = 2
AWQ_INFO_ALL_NONFINITE = 1
AWQ_MAX_PARTS = 8
AWQ_MAX_RATIOS = 64
GROUP_SIZE = 128
AWQ_FORMULA_MSMODELSLIM = 0
AWQ_FORMULA_RMS = 1
AWQ_FORMULA_DUO = 2
AWQ_QUANT_INT4_GROUP = 0
AWQ_QUANT_INT4_ROW = 1
AWQ_QUANT_INT8_ROW_SYM = 2
AWQ_ACT_SILU = 0
AWQ_ACT_RELU = 1

_c_int, _c_i64, _c_size, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGNATURES = {
    "awq_abi_version": (_c_int, []),
    "awq_status_string": (ctypes.c_char_p, [_c_int]),
    "awq_last_error": (ctypes.c_char_p, []),
    "awq_act_stats_workspace_bytes": (_c_size, [_c_int, _c_i64, _c_i64]),
    "awq_act_stats": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_size, _vp]),
    "awq_candidate_scales": (_c_int, [_vp, _c_i64, _c_int, _vp, _vp]),
    "awq_quant_delta": (_c_int, [_vp, _vp, _c_int, _c_int, _c_i64, _c_int, _vp, _c_int, _vp, _vp]),
    "awq_error_tiles": (_c_i64, [_c_i64, _c_i64]),
    "awq_error_sse": (_c_int, [_vp, _c_i64, _vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp]),
    "awq_loss_argmin": (_c_int, [_vp, _c_i64, _c_int, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp, _vp, _vp]),
    "awq_search_workspace_bytes": (_c_size, [_c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int]),
    "awq_search_scales": (_c_int, [_vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_i64, _c_i64, _vp, _c_int,
                                   _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "awq_search_scales_noalloc": (_c_int, [_vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_i64, _c_i64, _vp, _c_int,
                                           _c_int, _vp, _vp, _vp, _vp, _vp]),
    "awq_quantize_pack": (_c_int, [_vp, _vp, _c_int, _c_int, _c_i64, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "awq_act_stats_accumulate": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_size, _vp]),
    "awq_act_stats_finalize": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp]),
    "awq_fold_scales": (_c_int, [_vp, _c_i64, _c_int, _c_i64, _c_i64, _vp, _vp, _c_i64, _vp]),
    "awq_export_fp16": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "awq_tie_heads": (_c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "awq_head_group_scales": (_c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "awq_weight_mean": (_c_int, [_vp, _vp, _c_int, _c_int, _c_i64, _vp, _vp, _c_size, _vp]),
    "awq_candidate_scales_ex": (_c_int, [_vp, _vp, _c_i64, _vp, _c_int, _c_int, _vp, _vp]),
    "awq_quant_delta_ex": (_c_int, [_vp, _vp, _c_int, _c_int, _c_i64, _c_int, _vp, _c_int, _vp, _vp]),
    "awq_search_scales_ex": (_c_int, [_vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_i64, _c_i64, _vp, _vp, _vp,
                                      _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "awq_w4a16_gemm": (_c_int, [_vp, _c_i64, _c_int, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i64, _c_int,
                                _vp]),
    "awq_mlp_hidden_ref": (_c_int, [_vp, _c_i64, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp]),
    "awq_mlp_hidden_delta": (_c_int, [_vp, _c_i64, _vp, _vp, _vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "awq_search_loss_form": (_c_int, [_c_int, _c_i64, _c_i64, _c_i64, _c_int]),
    "awq_gram_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "awq_gram": (_c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _c_size, _vp]),
    "awq_quant_delta_f16": (_c_int, [_vp, _vp, _c_int, _c_i64, _c_int, _vp, _c_int, _vp, _vp, _vp]),
    "awq_gram_error_sse": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "awq_search_workspace_bytes_mlp": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int]),
    "awq_search_scales_mlp": (_c_int, [_vp, _c_i64, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _c_int,
                                       _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
}

_lib = None


class AwqError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m post_quantization_mean_amd.build` "
                           "(or __graft_entry__.build()); there is no other implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> list[str]:
    return list(_SIGNATURES)


def _check(status: int) -> None:
    if status != AWQ_OK:
        lib = load_library()
        raise AwqError(status, lib.awq_status_string(status).decode(), lib.awq_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return AWQ_DTYPE_BF16
    if t.dtype == torch.float32:
        return AWQ_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _buf(t: torch.Tensor, name: str, dtype, numel: int, device=None) -> int:
    """Pointer of a caller-supplied tensor that the library reads or writes as `numel` contiguous
    elements of `dtype` (`dtype` may be a tuple of accepted dtypes). The C entry points see only a
    pointer, so a wrong dtype, a strided view or a short buffer is refused here."""
    p = _dev(t, name)
    ok = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in ok:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in ok)}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    return p


def _parts(w_parts, dtype=None):
    """Device pointers and row counts of the weight parts (one dtype, one d_in, one device; with
    `dtype`, the activations' dtype, which the library assumes for both operands)."""
    if isinstance(w_parts, torch.Tensor):
        w_parts = [w_parts]
    w_parts = list(w_parts)
    if not w_parts:
        raise ValueError("no weight parts")
    w0 = w_parts[0]
    for i, w in enumerate(w_parts):
        if not isinstance(w, torch.Tensor) or w.dim() != 2 or not w.is_contiguous():
            raise ValueError(f"weight part {i} must be a contiguous [rows, d_in] matrix")
        if w.dtype != w0.dtype or w.shape[1] != w0.shape[1] or w.device != w0.device:
            raise ValueError(f"weight part {i} differs from part 0 in dtype, d_in or device")
    if dtype is not None and w0.dtype != dtype:
        raise TypeError(f"the weights are {w0.dtype} and the activations {dtype}: they must agree")
    ptrs = (ctypes.c_void_p * len(w_parts))(*[_dev(w, "weight part") for w in w_parts])
    rows = (ctypes.c_int64 * len(w_parts))(*[w.shape[0] for w in w_parts])
    return w_parts, ptrs, rows, sum(w.shape[0] for w in w_parts)


def _x_args(x: torch.Tensor):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a [n_tokens, d_in] matrix with unit stride along d_in")
    return _dev(x, "x"), x.shape[0], x.shape[1], x.stride(0)


def _vec(t: torch.Tensor, name: str) -> int:
    """Length of a 1-D tensor argument."""
    if not isinstance(t, torch.Tensor) or t.dim() != 1:
        raise ValueError(f"{name} must be a 1-D tensor")
    return t.shape[0]


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, {nbytes} needed")
    return workspace


# ------------------------------------------------------------------ entry points

def awq_abi_version() -> int:
    return load_library().awq_abi_version()


def awq_act_stats_workspace_bytes(dtype: int, n_tokens: int, d_in: int) -> int:
    return load_library().awq_act_stats_workspace_bytes(dtype, n_tokens, d_in)


def awq_act_stats(x: torch.Tensor, act_mean: torch.Tensor | None = None, workspace=None, stream=None):
    """a1: float64 [d_in] mean of |x| over tokens."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    dt = _dtype_code(x)
    if act_mean is None:
        act_mean = torch.empty(d, dtype=torch.float64, device=x.device)
    pa = _buf(act_mean, "act_mean", torch.float64, d, x.device)
    ws = _workspace(lib.awq_act_stats_workspace_bytes(dt, n, d), x.device, workspace)
    _check(lib.awq_act_stats(px, dt, n, d, ld, pa, ws.data_ptr(),
                             ws.numel() * ws.element_size(), _stream(stream)))
    return act_mean


def awq_candidate_scales(act_mean: torch.Tensor, n_grid: int, cand_scales=None, stream=None):
    """a2: float64 [n_grid, d_in] candidate scales."""
    lib = load_library()
    d = _vec(act_mean, "act_mean")
    pa = _buf(act_mean, "act_mean", torch.float64, d)
    if cand_scales is None:
        cand_scales = torch.empty((n_grid, d), dtype=torch.float64, device=act_mean.device)
    pc = _buf(cand_scales, "cand_scales", torch.float64, max(n_grid, 0) * d, act_mean.device)
    _check(lib.awq_candidate_scales(pa, d, n_grid, pc, _stream(stream)))
    return cand_scales


def awq_quant_delta(w_parts, cand_scales: torch.Tensor, group_size: int = GROUP_SIZE, delta=None, stream=None):
    """a3: [n_cand, d_out, d_in] delta = What - W in the weights' dtype."""
    lib = load_library()
    parts, ptrs, rows, d_out = _parts(w_parts)
    d_in = parts[0].shape[1]
    n_cand, pc = _cand_arg(cand_scales, d_in)
    if delta is None:
        delta = torch.empty((n_cand, d_out, d_in), dtype=parts[0].dtype, device=parts[0].device)
    pd = _buf(delta, "delta", parts[0].dtype, n_cand * d_out * d_in, parts[0].device)
    _check(lib.awq_quant_delta(ptrs, rows, len(parts), _dtype_code(parts[0]), d_in, group_size, pc, n_cand, pd,
                               _stream(stream)))
    return delta


def _cand_arg(cand_scales: torch.Tensor, d_in: int):
    """(n_cand, pointer) of a float64 [n_cand, d_in] candidate-scale matrix."""
    if not isinstance(cand_scales, torch.Tensor) or cand_scales.dim() != 2 or cand_scales.shape[1] != d_in:
        raise ValueError(f"cand_scales must be a [n_cand, {d_in}] matrix")
    return cand_scales.shape[0], _buf(cand_scales, "cand_scales", torch.float64, cand_scales.numel())


def awq_error_tiles(n_tokens: int, d_out: int) -> int:
    return load_library().awq_error_tiles(n_tokens, d_out)


def awq_error_sse(x: torch.Tensor, delta: torch.Tensor, tile_sse=None, stream=None):
    """a4: float64 [n_cand, tiles] per-tile sums of squares of x @ delta_j^T."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    if not isinstance(delta, torch.Tensor) or delta.dim() != 3:
        raise ValueError("delta must be a [n_cand, d_out, d_in] tensor")
    n_cand, d_out, d_in = delta.shape
    if d_in != d:
        raise ValueError("x and delta disagree on d_in")
    pd = _buf(delta, "delta", x.dtype, delta.numel(), x.device)
    tiles = lib.awq_error_tiles(n, d_out)
    if tile_sse is None:
        tile_sse = torch.empty((n_cand, tiles), dtype=torch.float64, device=x.device)
    pt = _buf(tile_sse, "tile_sse", torch.float64, n_cand * tiles, x.device)
    _check(lib.awq_error_sse(px, ld, pd, _dtype_code(x), n, d, d_out, n_cand, pt, _stream(stream)))
    return tile_sse


AWQ_LOSS_DIRECT, AWQ_LOSS_GRAM = 0, 1


def awq_search_loss_form(dtype: int, n_tokens: int, d_in: int, d_out: int, n_grid: int) -> int:
    """AWQ_LOSS_GRAM when awq_search_scales computes the losses through G = X^T X for these sizes."""
    return load_library().awq_search_loss_form(dtype, n_tokens, d_in, d_out, n_grid)


def awq_gram_workspace_bytes(n_tokens: int, d_in: int) -> int:
    return load_library().awq_gram_workspace_bytes(n_tokens, d_in)


def awq_gram(x: torch.Tensor, gram=None, gram_exp=None, workspace=None, stream=None):
    """G = X^T X of bfloat16 activations as (float16 [d_in, d_in] holding G * 2^e, int32 [1] = e)."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("awq_gram takes bfloat16 activations")
    gram = torch.empty((d, d), dtype=torch.float16, device=x.device) if gram is None else gram
    gram_exp = torch.empty(1, dtype=torch.int32, device=x.device) if gram_exp is None else gram_exp
    nb = lib.awq_gram_workspace_bytes(n, d)
    ws = _workspace(nb, x.device, workspace)
    _check(lib.awq_gram(px, ld, n, d, _buf(gram, "gram", torch.float16, d * d, x.device),
                        _buf(gram_exp, "gram_exp", torch.int32, 1, x.device), _dev(ws, "workspace"), nb,
                        _stream(stream)))
    return gram, gram_exp


def awq_quant_delta_f16(w_parts, cand_scales: torch.Tensor, group_size: int = GROUP_SIZE, delta=None,
                        delta_exp=None, stream=None):
    """a3 for the Gram form: (float16 [n_cand, d_out, d_in] holding delta * 2^e_k, int32 [n_cand + 1]
    with e_k first)."""
    lib = load_library()
    parts, ptrs, rows, d_out = _parts(w_parts, torch.bfloat16)
    d_in = parts[0].shape[1]
    n_cand, pc = _cand_arg(cand_scales, d_in)
    dev = parts[0].device
    delta = torch.empty((n_cand, d_out, d_in), dtype=torch.float16, device=dev) if delta is None else delta
    delta_exp = torch.empty(n_cand + 1, dtype=torch.int32, device=dev) if delta_exp is None else delta_exp
    _check(lib.awq_quant_delta_f16(ptrs, rows, len(parts), d_in, group_size, pc, n_cand,
                                   _buf(delta, "delta", torch.float16, n_cand * d_out * d_in, dev),
                                   _buf(delta_exp, "delta_exp", torch.int32, n_cand + 1, dev), _stream(stream)))
    return delta, delta_exp


def awq_gram_error_sse(gram: torch.Tensor, gram_exp: torch.Tensor, delta: torch.Tensor, delta_exp: torch.Tensor,
                       n_tokens: int, tile_sse=None, stream=None):
    """a4 in the Gram form: float64 [n_cand, awq_error_tiles(n_tokens, d_out)] tile shares of each
    candidate's sum_o delta[o] G delta[o]^T (zeros past its own tiles), for awq_loss_argmin."""
    lib = load_library()
    if not isinstance(delta, torch.Tensor) or delta.dim() != 3:
        raise ValueError("delta must be a [n_cand, d_out, d_in] tensor")
    n_cand, d_out, d_in = delta.shape
    dev = delta.device
    if not isinstance(gram, torch.Tensor) or tuple(gram.shape) != (d_in, d_in):
        raise ValueError(f"gram must be a [{d_in}, {d_in}] matrix")
    tiles = lib.awq_error_tiles(n_tokens, d_out)
    tile_sse = torch.empty((n_cand, tiles), dtype=torch.float64, device=dev) if tile_sse is None else tile_sse
    _check(lib.awq_gram_error_sse(_buf(gram, "gram", torch.float16, d_in * d_in, dev),
                                  _buf(gram_exp, "gram_exp", torch.int32, 1, dev),
                                  _buf(delta, "delta", torch.float16, delta.numel(), dev),
                                  _buf(delta_exp, "delta_exp", torch.int32, n_cand + 1, dev), n_cand, n_tokens, d_in,
                                  d_out, _buf(tile_sse, "tile_sse", torch.float64, n_cand * tiles, dev),
                                  _stream(stream)))
    return tile_sse


def awq_loss_argmin(tile_sse: torch.Tensor, n_tokens: int, d_out: int, cand_scales: torch.Tensor,
                    losses=None, best_scales=None, best_info=None, stream=None):
    """a5: (losses [n_grid] f64, best_scales [d_in] f64, best_info [2] i32 = {k*, flags})."""
    lib = load_library()
    if not isinstance(tile_sse, torch.Tensor) or tile_sse.dim() != 2:
        raise ValueError("tile_sse must be a [n_grid, tiles] matrix")
    n_grid, tiles = tile_sse.shape
    dev = tile_sse.device
    pt = _buf(tile_sse, "tile_sse", torch.float64, n_grid * tiles)
    if not isinstance(cand_scales, torch.Tensor) or cand_scales.dim() != 2 or cand_scales.shape[0] < n_grid:
        raise ValueError(f"cand_scales must be a [n_grid >= {n_grid}, d_in] matrix")
    d_in = cand_scales.shape[1]
    pc = _buf(cand_scales, "cand_scales", torch.float64, n_grid * d_in, dev)
    losses = torch.empty(n_grid, dtype=torch.float64, device=dev) if losses is None else losses
    best_scales = torch.empty(d_in, dtype=torch.float64, device=dev) if best_scales is None else best_scales
    best_info = torch.empty(2, dtype=torch.int32, device=dev) if best_info is None else best_info
    _check(lib.awq_loss_argmin(pt, tiles, n_grid, n_tokens, d_out, pc, d_in,
                               _buf(losses, "losses", torch.float64, n_grid, dev),
                               _buf(best_scales, "best_scales", torch.float64, d_in, dev),
                               _buf(best_info, "best_info", torch.int32, 2, dev), _stream(stream)))
    return losses, best_scales, best_info


def _search_outputs(out, n_grid: int, d_in: int, dev):
    """The four outputs of a search (caller-supplied in `out`, else allocated) and their pointers."""
    out = out or {}
    spec = {"cand_scales": ((max(n_grid, 1), d_in), torch.float64), "losses": ((max(n_grid, 1),), torch.float64),
            "best_scales": ((d_in,), torch.float64), "best_info": ((2,), torch.int32)}
    res, ptrs = {}, []
    for name, (shape, dtype) in spec.items():
        t = out.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
        numel = 1
        for v in shape:
            numel *= v
        ptrs.append(_buf(t, name, dtype, numel, dev))
        res[name] = t
    return res, ptrs


def awq_search_workspace_bytes(dtype: int, n_tokens: int, d_in: int, d_out: int, group_size: int,
                               n_grid: int, cand_per_pass: int) -> int:
    return load_library().awq_search_workspace_bytes(dtype, n_tokens, d_in, d_out, group_size, n_grid,
                                                     cand_per_pass)


def awq_search_scales(x: torch.Tensor, w_parts, act_mean: torch.Tensor, n_grid: int = 20,
                      group_size: int = GROUP_SIZE, cand_per_pass: int | None = None, workspace=None,
                      out=None, stream=None) -> dict:
    """a2..a5 in one call. Returns device tensors: cand_scales, losses, best_scales, best_info."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    dt = _dtype_code(x)
    parts, ptrs, rows, d_out = _parts(w_parts, x.dtype)
    if parts[0].shape[1] != d:
        raise ValueError("x and the weights disagree on d_in")
    if cand_per_pass is None:
        cand_per_pass = n_grid
    dev = x.device
    pa = _buf(act_mean, "act_mean", torch.float64, d, dev)
    res, (pc, pl, pb, pi) = _search_outputs(out, n_grid, d, dev)
    need = lib.awq_search_workspace_bytes(dt, n, d, d_out, group_size, n_grid, cand_per_pass)
    ws = _workspace(need, dev, workspace)
    _check(lib.awq_search_scales(px, ld, ptrs, rows, len(parts), dt, n, d, pa, group_size, n_grid, cand_per_pass,
                                 pc, pl, pb, pi, ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))
    return res


def awq_search_scales_noalloc(x: torch.Tensor, w_parts, act_mean: torch.Tensor, n_grid: int = 20,
                              group_size: int = GROUP_SIZE, out=None, stream=None) -> dict:
    """awq_search_scales with the library's fixed device scratch instead of a workspace: the C call
    allocates nothing (pass `out` to allocate nothing here either). Overlapping calls on one GPU race."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    dt = _dtype_code(x)
    parts, ptrs, rows, d_out = _parts(w_parts, x.dtype)
    if parts[0].shape[1] != d:
        raise ValueError("x and the weights disagree on d_in")
    dev = x.device
    pa = _buf(act_mean, "act_mean", torch.float64, d, dev)
    res, (pc, pl, pb, pi) = _search_outputs(out, n_grid, d, dev)
    _check(lib.awq_search_scales_noalloc(px, ld, ptrs, rows, len(parts), dt, n, d, pa, group_size, n_grid, pc, pl,
                                         pb, pi, _stream(stream)))
    return res


def awq_quantize_pack(w_parts, s: torch.Tensor, group_size: int = GROUP_SIZE, out=None, stream=None) -> dict:
    """a6: codes [d_out, d_in/2] u8, qscales [d_out, d_in/128] f32, zeros [d_out, d_in/128] i32."""
    lib = load_library()
    parts, ptrs, rows, d_out = _parts(w_parts)
    d_in = parts[0].shape[1]
    dev = parts[0].device
    out = out or {}
    g = d_in // group_size
    codes = out.get("codes")
    if codes is None:
        codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    qs = out.get("qscales")
    if qs is None:
        qs = torch.empty((d_out, g), dtype=torch.float32, device=dev)
    zs = out.get("zeros")
    if zs is None:
        zs = torch.empty((d_out, g), dtype=torch.int32, device=dev)
    _check(lib.awq_quantize_pack(ptrs, rows, len(parts), _dtype_code(parts[0]), d_in, group_size,
                                 _buf(s, "s", torch.float64, d_in, dev),
                                 _buf(codes, "codes", torch.uint8, d_out * (d_in // 2), dev),
                                 _buf(qs, "qscales", torch.float32, d_out * g, dev),
                                 _buf(zs, "zeros", torch.int32, d_out * g, dev), _stream(stream)))
    return {"codes": codes, "qscales": qs, "zeros": zs}


def awq_act_stats_accumulate(x: torch.Tensor, sums: torch.Tensor, workspace=None, stream=None):
    """sums (float64 [d_in], device) += per-channel sum of |x| over this batch's tokens."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    dt = _dtype_code(x)
    ps = _buf(sums, "sums", torch.float64, d, x.device)
    ws = _workspace(lib.awq_act_stats_workspace_bytes(dt, n, d), x.device, workspace)
    _check(lib.awq_act_stats_accumulate(px, dt, n, d, ld, ps, ws.data_ptr(),
                                        ws.numel() * ws.element_size(), _stream(stream)))
    return sums


def awq_act_stats_finalize(sums: torch.Tensor, total_tokens: int, act_mean=None, stream=None):
    """act_mean = sums / total_tokens (float64 [d_in])."""
    lib = load_library()
    d = _vec(sums, "sums")
    ps = _buf(sums, "sums", torch.float64, d)
    if act_mean is None:
        act_mean = torch.empty_like(sums)
    _check(lib.awq_act_stats_finalize(ps, d, total_tokens, _buf(act_mean, "act_mean", torch.float64, d, sums.device),
                                      _stream(stream)))
    return act_mean


def awq_fold_scales(src: torch.Tensor, s: torch.Tensor, dst=None, stream=None):
    """Row r of src ([rows] or [rows, cols], bf16 or f32) divided by s[r] (float64 [rows])."""
    lib = load_library()
    src2 = src.unsqueeze(1) if src.dim() == 1 else src
    if src2.dim() != 2 or src2.stride(1) != 1:
        raise ValueError("src must be [rows] or a [rows, cols] matrix with unit stride along cols")
    if dst is None:
        dst = torch.empty_like(src)
    dst2 = dst.unsqueeze(1) if dst.dim() == 1 else dst
    if dst2.shape != src2.shape or dst2.stride(1) != 1 or dst2.dtype != src2.dtype:
        raise ValueError("dst must match src")
    rows, cols = src2.shape
    _check(lib.awq_fold_scales(_dev(src2, "src"), src2.stride(0) if rows > 1 else cols, _dtype_code(src2), rows,
                               cols, _buf(s, "s", torch.float64, rows, src.device), _dev(dst2, "dst"),
                               dst2.stride(0) if rows > 1 else cols, _stream(stream)))
    return dst


def awq_tie_heads(act_mean: torch.Tensor, n_heads: int, n_kv_heads: int, head_dim: int, out=None, stream=None):
    """Statistic of the o_proj input channels tied across the query heads that share a KV head
    (float64 [n_heads * head_dim]); `out` may be act_mean."""
    lib = load_library()
    n = n_heads * head_dim
    a = _buf(act_mean, "act_mean", torch.float64, n)
    if out is None:
        out = torch.empty(n, dtype=torch.float64, device=act_mean.device)
    _check(lib.awq_tie_heads(a, n_heads, n_kv_heads, head_dim, _buf(out, "out", torch.float64, n, act_mean.device),
                             _stream(stream)))
    return out


def awq_head_group_scales(s: torch.Tensor, n_heads: int, n_kv_heads: int, head_dim: int, out=None, stream=None):
    """The v_proj row scales (float64 [n_kv_heads * head_dim]) of tied o_proj scales s."""
    lib = load_library()
    p = _buf(s, "s", torch.float64, n_heads * head_dim)
    if out is None:
        out = torch.empty(n_kv_heads * head_dim, dtype=torch.float64, device=s.device)
    _check(lib.awq_head_group_scales(p, n_heads, n_kv_heads, head_dim,
                                     _buf(out, "out", torch.float64, n_kv_heads * head_dim, s.device),
                                     _stream(stream)))
    return out


def awq_export_fp16(qscales: torch.Tensor, zeros: torch.Tensor, out=None, stream=None) -> dict:
    """Float16 steps (uint16 bits) and zero points packed two per byte, with the two counts."""
    lib = load_library()
    if not isinstance(qscales, torch.Tensor) or qscales.dim() != 2:
        raise ValueError("qscales must be a [rows, groups] matrix")
    rows, g = qscales.shape
    dev = qscales.device
    pq = _buf(qscales, "qscales", torch.float32, rows * g)
    pz = _buf(zeros, "zeros", torch.int32, rows * g, dev)
    out = out or {}
    steps = out.get("steps_f16")
    if steps is None:
        steps = torch.empty((rows, g), dtype=torch.int16, device=qscales.device)
    zu4 = out.get("zeros_u4")
    if zu4 is None:
        zu4 = torch.empty((rows, (g + 1) // 2), dtype=torch.uint8, device=qscales.device)
    counts = out.get("counts")
    if counts is None:
        counts = torch.zeros(2, dtype=torch.int32, device=qscales.device)
    _check(lib.awq_export_fp16(pq, pz, rows, g, _buf(steps, "steps_f16", _HALF_BITS, rows * g, dev),
                               _buf(zu4, "zeros_u4", torch.uint8, rows * ((g + 1) // 2), dev),
                               _buf(counts, "counts", torch.int32, 2, dev), _stream(stream)))
    return {"steps_f16": steps, "zeros_u4": zu4, "counts": counts}


def _ratios(ratios):
    r = [float(v) for v in ratios]
    return (ctypes.c_double * max(len(r), 1))(*r), len(r)


_HALF_BITS = (torch.int16, torch.uint16, torch.float16)  # 16-bit containers of float16 bits


def awq_weight_mean(w_parts, w_mean=None, workspace=None, stream=None):
    """float64 [d_in] mean of |W| over the stacked output rows of the parts."""
    lib = load_library()
    parts, ptrs, rows, d_out = _parts(w_parts)
    d_in = parts[0].shape[1]
    dt = _dtype_code(parts[0])
    dev = parts[0].device
    if w_mean is None:
        w_mean = torch.empty(d_in, dtype=torch.float64, device=dev)
    pw = _buf(w_mean, "w_mean", torch.float64, d_in, dev)
    need = max(lib.awq_act_stats_workspace_bytes(dt, r, d_in) for r in rows)
    ws = _workspace(need, dev, workspace)
    _check(lib.awq_weight_mean(ptrs, rows, len(parts), dt, d_in, pw, ws.data_ptr(),
                               ws.numel() * ws.element_size(), _stream(stream)))
    return w_mean


def awq_candidate_scales_ex(act_mean: torch.Tensor, ratios, formula: int = AWQ_FORMULA_MSMODELSLIM,
                            w_mean=None, cand_scales=None, stream=None):
    """float64 [len(ratios), d_in] candidate scales of a formula over an explicit ratio list."""
    lib = load_library()
    d = _vec(act_mean, "act_mean")
    dev = act_mean.device
    pa = _buf(act_mean, "act_mean", torch.float64, d)
    pw = 0 if w_mean is None else _buf(w_mean, "w_mean", torch.float64, d, dev)
    rv, n = _ratios(ratios)
    if cand_scales is None:
        cand_scales = torch.empty((max(n, 1), d), dtype=torch.float64, device=dev)
    pc = _buf(cand_scales, "cand_scales", torch.float64, n * d, dev)
    _check(lib.awq_candidate_scales_ex(pa, pw, d, rv, n, formula, pc, _stream(stream)))
    return cand_scales


def awq_quant_delta_ex(w_parts, cand_scales: torch.Tensor, quantizer: int = AWQ_QUANT_INT4_GROUP, delta=None,
                       stream=None):
    """[n_cand, d_out, d_in] delta = What - W under the chosen quantizer, in the weights' dtype."""
    lib = load_library()
    parts, ptrs, rows, d_out = _parts(w_parts)
    d_in = parts[0].shape[1]
    n_cand, pc = _cand_arg(cand_scales, d_in)
    if delta is None:
        delta = torch.empty((n_cand, d_out, d_in), dtype=parts[0].dtype, device=parts[0].device)
    pd = _buf(delta, "delta", parts[0].dtype, n_cand * d_out * d_in, parts[0].device)
    _check(lib.awq_quant_delta_ex(ptrs, rows, len(parts), _dtype_code(parts[0]), d_in, quantizer, pc, n_cand, pd,
                                  _stream(stream)))
    return delta


def awq_search_scales_ex(x: torch.Tensor, w_parts, act_mean: torch.Tensor, ratios,
                         formula: int = AWQ_FORMULA_MSMODELSLIM, quantizer: int = AWQ_QUANT_INT4_GROUP,
                         w_mean=None, cand_per_pass: int | None = None, workspace=None, out=None,
                         stream=None) -> dict:
    """The search over an explicit ratio list with a scale formula and a quantizer."""
    lib = load_library()
    px, n, d, ld = _x_args(x)
    dt = _dtype_code(x)
    parts, ptrs, rows, d_out = _parts(w_parts, x.dtype)
    if parts[0].shape[1] != d:
        raise ValueError("x and the weights disagree on d_in")
    rv, n_r = _ratios(ratios)
    if cand_per_pass is None:
        cand_per_pass = n_r
    dev = x.device
    pa = _buf(act_mean, "act_mean", torch.float64, d, dev)
    pw = 0 if w_mean is None else _buf(w_mean, "w_mean", torch.float64, d, dev)
    res, (pc, pl, pb, pi) = _search_outputs(out, n_r, d, dev)
    need = lib.awq_search_workspace_bytes(dt, n, d, d_out, GROUP_SIZE, n_r, cand_per_pass)
    ws = _workspace(need, dev, workspace)
    _check(lib.awq_search_scales_ex(px, ld, ptrs, rows, len(parts), dt, n, d, pa, pw, rv, n_r, formula, quantizer,
                                    cand_per_pass, pc, pl, pb, pi, ws.data_ptr(), ws.numel() * ws.element_size(),
                                    _stream(stream)))
    return res


def awq_w4a16_gemm(x: torch.Tensor, codes: torch.Tensor, steps_f16: torch.Tensor, zeros_u4: torch.Tensor,
                   out_dtype=torch.float32, y=None, stream=None):
    """Y [n_tokens, d_out] = x @ W_hat^T, W_hat dequantized on the fly from the deployment form
    (codes [d_out, d_in/2] u8, float16 steps as int16/uint16 bits [d_out, d_in/128], zero points
    packed two per byte [d_out, ceil(d_in/256)]). x is bfloat16 or float16; Y float32 or x's dtype."""
    lib = load_library()
    if x.dtype == torch.bfloat16:
        xd = AWQ_DTYPE_BF16
    elif x.dtype == torch.float16:
        xd = AWQ_DTYPE_F16
    else:
        raise TypeError("x must be torch.bfloat16 or torch.float16")
    px, n, d_in, ld = _x_args(x)
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2 or codes.shape[1] * 2 != d_in:
        raise ValueError(f"codes must be a [d_out, {d_in // 2}] matrix")
    d_out = codes.shape[0]
    g = d_in // GROUP_SIZE
    if out_dtype == torch.float32:
        yd = AWQ_DTYPE_F32
    elif out_dtype == x.dtype:
        yd = xd
    else:
        raise TypeError("out_dtype must be torch.float32 or x's dtype")
    if y is None:
        y = torch.empty((n, d_out), dtype=out_dtype, device=x.device)
    if y.dim() != 2 or tuple(y.shape) != (n, d_out) or y.stride(1) != 1 or y.dtype != out_dtype:
        raise ValueError("y must be a [n_tokens, d_out] matrix of out_dtype with unit stride along d_out")
    dev = x.device
    _check(lib.awq_w4a16_gemm(px, ld, xd, _buf(codes, "codes", torch.uint8, d_out * (d_in // 2), dev),
                              _buf(steps_f16, "steps_f16", _HALF_BITS, d_out * g, dev),
                              _buf(zeros_u4, "zeros_u4", torch.uint8, d_out * ((g + 1) // 2), dev), n, d_in, d_out,
                              _dev(y, "y"), y.stride(0), yd, _stream(stream)))
    return y


def _bf16_matrix(t: torch.Tensor, name: str, shape, device) -> int:
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a {list(shape)} matrix")
    return _buf(t, name, torch.bfloat16, t.numel(), device)


def _x_bf16(x: torch.Tensor):
    """x arguments of the block-level entry points, which take bfloat16 activations."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16:
        raise TypeError("x must be torch.bfloat16")
    return _x_args(x)


def awq_mlp_hidden_ref(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, g_ref=None, u_ref=None,
                       stream=None):
    """(g_ref, u_ref) = (x @ w_gate^T, x @ w_up^T) in float32, [n_tokens, d_ff] each."""
    lib = load_library()
    px, n, d_in, ld = _x_bf16(x)
    if not isinstance(w_gate, torch.Tensor) or w_gate.dim() != 2:
        raise ValueError("w_gate must be a [d_ff, d_in] matrix")
    d_ff = w_gate.shape[0]
    dev = x.device
    g_ref = torch.empty((n, d_ff), dtype=torch.float32, device=dev) if g_ref is None else g_ref
    u_ref = torch.empty((n, d_ff), dtype=torch.float32, device=dev) if u_ref is None else u_ref
    _check(lib.awq_mlp_hidden_ref(px, ld, _bf16_matrix(w_gate, "w_gate", (d_ff, d_in), dev),
                                  _bf16_matrix(w_up, "w_up", (d_ff, d_in), dev), n, d_in, d_ff,
                                  _buf(g_ref, "g_ref", torch.float32, n * d_ff, dev),
                                  _buf(u_ref, "u_ref", torch.float32, n * d_ff, dev), _stream(stream)))
    return g_ref, u_ref


def awq_mlp_hidden_delta(x: torch.Tensor, dw_gate: torch.Tensor, dw_up: torch.Tensor, g_ref: torch.Tensor,
                         u_ref: torch.Tensor, act: int = AWQ_ACT_SILU, dh=None, stream=None):
    """dh = act(g) u - act(g + x dw_gate^T)(u + x dw_up^T), bfloat16 [n_tokens, d_ff]."""
    lib = load_library()
    px, n, d_in, ld = _x_bf16(x)
    if not isinstance(dw_gate, torch.Tensor) or dw_gate.dim() != 2:
        raise ValueError("dw_gate must be a [d_ff, d_in] matrix")
    d_ff = dw_gate.shape[0]
    dev = x.device
    dh = torch.empty((n, d_ff), dtype=torch.bfloat16, device=dev) if dh is None else dh
    _check(lib.awq_mlp_hidden_delta(px, ld, _bf16_matrix(dw_gate, "dw_gate", (d_ff, d_in), dev),
                                    _bf16_matrix(dw_up, "dw_up", (d_ff, d_in), dev),
                                    _buf(g_ref, "g_ref", torch.float32, n * d_ff, dev),
                                    _buf(u_ref, "u_ref", torch.float32, n * d_ff, dev), act, n, d_in, d_ff,
                                    _buf(dh, "dh", torch.bfloat16, n * d_ff, dev), _stream(stream)))
    return dh


def awq_search_workspace_bytes_mlp(n_tokens: int, d_in: int, d_ff: int, d_model: int, n_grid: int,
                                   cand_per_pass: int) -> int:
    return load_library().awq_search_workspace_bytes_mlp(n_tokens, d_in, d_ff, d_model, n_grid, cand_per_pass)


def awq_search_scales_mlp(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                          act_mean: torch.Tensor, act: int = AWQ_ACT_SILU, n_grid: int = 20,
                          cand_per_pass: int | None = None, workspace=None, out=None, stream=None) -> dict:
    """The gate/up search scored at the gated MLP block's output. Device tensors: cand_scales, losses,
    best_scales, best_info."""
    lib = load_library()
    px, n, d_in, ld = _x_bf16(x)
    if not isinstance(w_gate, torch.Tensor) or w_gate.dim() != 2 or not isinstance(w_down, torch.Tensor) \
            or w_down.dim() != 2:
        raise ValueError("w_gate and w_down must be matrices")
    d_ff, d_model = w_gate.shape[0], w_down.shape[0]
    cand_per_pass = cand_per_pass or n_grid
    dev = x.device
    pg = _bf16_matrix(w_gate, "w_gate", (d_ff, d_in), dev)
    pu = _bf16_matrix(w_up, "w_up", (d_ff, d_in), dev)
    pdn = _bf16_matrix(w_down, "w_down", (d_model, d_ff), dev)
    pa = _buf(act_mean, "act_mean", torch.float64, d_in, dev)
    res, (pc, pl, pb, pi) = _search_outputs(out, n_grid, d_in, dev)
    ws = _workspace(lib.awq_search_workspace_bytes_mlp(n, d_in, d_ff, d_model, n_grid, cand_per_pass), dev,
                    workspace)
    _check(lib.awq_search_scales_mlp(px, ld, pg, pu, pdn, n, d_in, d_ff, d_model, pa, act, n_grid, cand_per_pass,
                                     pc, pl, pb, pi, ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return res


def awq_layer(x: torch.Tensor, w_parts, n_grid: int = 20, group_size: int = GROUP_SIZE,
              cand_per_pass: int | None = None, stream=None) -> dict:
    """The whole hot path for one layer: statistic, search, final quantize + pack."""
    act_mean = awq_act_stats(x, stream=stream)
    res = awq_search_scales(x, w_parts, act_mean, n_grid, group_size, cand_per_pass, stream=stream)
    res.update(awq_quantize_pack(w_parts, res["best_scales"], group_size, stream=stream))
    res["act_mean"] = act_mean
    return res
