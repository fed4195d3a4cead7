// Internal declarations of the grid and quantizer variants (variants.hip), shared with the
// host-side C ABI. Not part of the public interface (include/awq.h is).
#pragma once

#include "internal.h"

namespace awq {

// ---- variants of a2 and a3 (scale formulas over explicit ratio lists, per-row quantizers)
constexpr int kMaxRatios = 64;
struct RatioList {
  double r[kMaxRatios];
};
constexpr int kFormulaMs = 0;    // max(a^r, 1e-4) / sqrt(max * min)
constexpr int kFormulaRms = 1;   // max(max(a, 1e-5)^r / sqrt(mean(.^2)), 1e-4)
constexpr int kFormulaDuo = 2;   // max(a^r / (wm^(1-r) + 1e-6), 1e-4) / sqrt(max * min)
constexpr int kQuantInt4Group = 0;
constexpr int kQuantInt4Row = 1;
constexpr int kQuantInt8RowSym = 2;
hipError_t launch_candidate_scales_ex(const double* act_mean, const double* w_mean, int64_t d_in,
                                      const RatioList& ratios, int n_ratios, int formula, double* cand_scales,
                                      hipStream_t stream);
hipError_t launch_quant_delta_row(const WParts& w, int dtype, int64_t d_in, int quantizer, const double* cand_scales,
                                  int n_cand, void* delta, hipStream_t stream);
// the per-row quantizers for the Gram form: bfloat16 weights, delta as float16 of delta * 2^dexp[k]
hipError_t launch_quant_delta_row_f16(const WParts& w, int64_t d_in, int quantizer, const double* cand_scales,
                                      int n_cand, uint16_t* delta, const int32_t* dexp, hipStream_t stream);
hipError_t launch_fill(double* p, int64_t n, double v, hipStream_t stream);

}  // namespace awq
