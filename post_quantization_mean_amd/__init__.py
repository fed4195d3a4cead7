"""MI355X (gfx950) AWQ activation-aware scale search and INT4 group quantization.

The computation lives in the HIP library libawq_mi355x.so behind the C ABI of
include/awq.h; `binding` exposes its entry points to Python with the same names.
"""
from . import binding  # noqa: F401
from .binding import (AwqError, awq_act_stats, awq_candidate_scales, awq_error_sse, awq_error_tiles,
                      awq_layer, awq_loss_argmin, awq_quant_delta, awq_quantize_pack, awq_search_scales,
                      load_library)

__all__ = ["AwqError", "awq_act_stats", "awq_candidate_scales", "awq_error_sse", "awq_error_tiles",
           "awq_layer", "awq_loss_argmin", "awq_quant_delta", "awq_quantize_pack", "awq_search_scales",
           "load_library", "binding"]
