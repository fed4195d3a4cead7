// Interface of the error GEMM (err_gemm.hip): its tile shape and launches. Kept apart from the
// other internal declarations so that the GEMM compiles from err_gemm.hip and this file only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

// ---- a4
constexpr int kTileM = 256;  // tokens per error-GEMM tile
constexpr int kTileN = 256;  // weight rows per error-GEMM tile
hipError_t launch_error_sse(const void* x, int64_t ld_x, const void* delta, int dtype,
                            int64_t n_tokens, int64_t d_in, int64_t d_out, int n_cand,
                            double* tile_sse, hipStream_t stream);
// The Gram form: G = X^T X in float32 from X^T ([d_in, n_pad] bf16, n_pad a multiple of 64, zero
// past the tokens), the 256 x 256 tiles on and above the diagonal stored (row pitch d_in) ...
hipError_t launch_gram_store(const uint16_t* xt, int64_t n_pad, int64_t d_in, float* g, hipStream_t stream);
// ... and per tile a share of sum_o delta_k[o] G delta_k[o]^T from float16 G (scaled by 2^gexp[0])
// and float16 delta_k (scaled by 2^dexp[k]), unscaled exactly, in tile_sse[k * cand_stride + tile].
// Reads only G's 256-blocks on and above the diagonal; the diagonal blocks are stored halved
// (launch_gram) and each tile's sum is doubled.
hipError_t launch_quad_sse(const uint16_t* g16, const int32_t* gexp, const uint16_t* delta16, const int32_t* dexp,
                           int n_cand, int64_t d_in, int64_t d_out, int64_t cand_stride, double* tile_sse,
                           hipStream_t stream);

}  // namespace awq
