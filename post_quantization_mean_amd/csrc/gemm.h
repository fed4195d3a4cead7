// Interface of the error GEMM (err_gemm.hip): its tile shape and launch. Kept apart from the
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

}  // namespace awq
