// Internal declarations shared by the host-side C ABI (abi.hip) and the kernel files.
// Not part of the public interface (include/awq.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm.h"

namespace awq {

constexpr int kMaxParts = 8;
constexpr int kGroup = 128;  // channels per quantization group (one row, consecutive)

// A fused set of weight matrices whose rows are stacked: part p covers stacked rows
// [row_begin[p], row_begin[p+1]) and points at a contiguous [rows, d_in] matrix.
struct WParts {
  const void* ptr[kMaxParts];
  int64_t row_begin[kMaxParts + 1];
  int n;
};

// ---- a1: activation statistic
struct ActStatsPlan {
  int lanes_per_row;   // lanes that cover one row slice (16 or 32)
  int64_t col_blocks;  // blocks along d_in
  int64_t row_chunks;  // blocks along n_tokens (partial sums kept per chunk)
  int64_t rows_per_chunk;
};
ActStatsPlan act_stats_plan(int dtype, int64_t n_tokens, int64_t d_in);
// accumulate: act_mean[c] += sum_i |x[i,c]| instead of act_mean[c] = mean_i |x[i,c]|
hipError_t launch_act_stats(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                            double* act_mean, double* partial, const ActStatsPlan& plan,
                            hipStream_t stream, bool accumulate = false);
hipError_t launch_act_mean_from_sums(const double* sums, int64_t d_in, int64_t total_tokens, double* act_mean,
                                     hipStream_t stream);

// ---- a2 / a5
hipError_t launch_candidate_scales(const double* act_mean, int64_t d_in, int n_grid,
                                   double* cand_scales, hipStream_t stream);
hipError_t launch_loss_argmin(const double* tile_sse, int64_t tiles_per_cand, int n_grid,
                              int64_t n_tokens, int64_t d_out, const double* cand_scales,
                              int64_t d_in, double* losses, double* best_scales,
                              int32_t* best_info, hipStream_t stream);

// ---- a3 / a6
hipError_t launch_quant_delta(const WParts& w, int dtype, int64_t d_in, const double* cand_scales,
                              int n_cand, void* delta, hipStream_t stream);
hipError_t launch_quantize_pack(const WParts& w, int dtype, int64_t d_in, const double* s,
                                uint8_t* codes, float* qscales, int32_t* zeros,
                                hipStream_t stream);
// the same delta in float16, scaled by 2^dexp[k] (bfloat16 weights)
hipError_t launch_quant_delta_f16(const WParts& w, int64_t d_in, const double* cand_scales, int n_cand,
                                  uint16_t* delta, const int32_t* dexp, hipStream_t stream);

// ---- the Gram form of the loss (gram.hip)
int64_t gram_n_pad(int64_t n_tokens);  // tokens of X^T's rows: a multiple of 64
// X^T into xt ([d_in, gram_n_pad]), G = X^T X into g32 ([d_in, d_in] float32), its scale exponent
// into gexp[0] and float16(G * 2^gexp) into g16, the 256 x 256 blocks on the diagonal times 1/2 (a
// float16 product), the operand launch_quad_sse takes
hipError_t launch_gram(const void* x, int64_t ld_x, int64_t n_tokens, int64_t d_in, uint16_t* xt, float* g32,
                       uint16_t* g16, int32_t* gexp, hipStream_t stream);
// dexp[k] for k < n_cand: the scale exponent of ratio k's delta, from the bound
// (1.5 max|W| max(s_k) + b) / min(s_k) + max|W| (b: 1e-8 for the INT4 quantizers, 1.27e-6 for the
// symmetric INT8 one); dexp[n_cand]: max |W| (scratch)
hipError_t launch_delta_exp(const WParts& w, int64_t d_in, const double* cand_scales, int n_cand, double b,
                            int32_t* dexp, hipStream_t stream);
hipError_t launch_fill_f64(double* p, int64_t n, double v, hipStream_t stream);

// ---- around the search: source fold and deployment form
hipError_t launch_fold_scales(const void* src, int64_t ld_src, int dtype, int64_t rows, int64_t cols,
                              const double* s, void* dst, int64_t ld_dst, bool vec, hipStream_t stream);
hipError_t launch_tie_heads(const double* act_mean, int64_t n_heads, int64_t n_kv, int64_t head_dim, double* tied,
                            hipStream_t stream);
hipError_t launch_head_group_scales(const double* s, int64_t n_heads, int64_t n_kv, int64_t head_dim, double* s_kv,
                                    hipStream_t stream);
hipError_t launch_export_fp16(const float* qscales, const int32_t* zeros, int64_t rows, int64_t n_groups,
                              uint16_t* steps_f16, uint8_t* zeros_u4, int32_t* counts, hipStream_t stream);

}  // namespace awq
