// Internal declarations of the W4A16 consumer (w4a16.hip), shared with the host-side C ABI. Not
// part of the public interface (include/awq.h is).
#pragma once

#include "internal.h"

namespace awq {

// A single token with d_in <= 32768 uses the one-token kernel (each wave streams whole rows in 1 KiB
// windows); launches with at most this many tokens otherwise use the few-token kernel (weights
// streamed once per 16 tokens); larger ones the many-token kernels (activations staged in LDS per
// block).
constexpr int64_t kW4a16SmallMaxTokens = 32;

bool w4a16_uses_big_kernel(int64_t n_tokens);
// kind 0: bfloat16 activations and operands, 1: float16. y is float32 (y_f32) or the activations' type.
hipError_t launch_w4a16_gemm(const void* x, int64_t ld_x, int kind, const uint8_t* codes, const uint16_t* steps_f16,
                             const uint8_t* zeros_u4, int64_t n_tokens, int64_t d_in, int64_t d_out, void* y,
                             int64_t ld_y, bool y_f32, hipStream_t stream);

}  // namespace awq
