// Internal declarations of the block-level (gated MLP) objective (block_gemm.hip), shared with the
// host-side C ABI. Not part of the public interface (include/awq.h is).
#pragma once

#include "internal.h"
#include "device_common.h"

namespace awq {

constexpr int kModeRef = 0;    // G = X Wg^T, U = X Wu^T (float32)
constexpr int kModeDelta = 1;  // dh = act(G) U - act(G + X dWg^T)(U + X dWu^T) (bfloat16)
constexpr int kActSilu = 0;
constexpr int kActRelu = 1;

// x: bfloat16 [n_tokens, ld_x]; wg / wu: bfloat16 [d_ff, d_in] (weights in kModeRef, their deltas in
// kModeDelta); g_io / u_io: float32 [n_tokens, d_ff], written (kModeRef) or read (kModeDelta); dh:
// bfloat16 [n_tokens, d_ff], written in kModeDelta.
hipError_t launch_mlp_hidden(int mode, int act, const void* x, int64_t ld_x, const void* wg, const void* wu,
                             int64_t n_tokens, int64_t d_in, int64_t d_ff, float* g_io, float* u_io, void* dh,
                             hipStream_t stream);

}  // namespace awq
