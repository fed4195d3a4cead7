// Variants of the candidate-scale step (a2) and of the quantizer inside the quantize -> delta
// step (a3) that the pages describe beside the main search. The loss (error GEMM) and the
// choice are unchanged.
//
// Scale formulas, for a ratio r taken from an explicit list:
//   msModelSlim "AWQ：激活感知权重量化算法说明", 原理 / 算法公式:
//       s = max(a^r, 1e-4);  s /= sqrt(max(s) * min(s))
//   gsyq.cn "AWQ 离群激活平滑实操", section 二 (search_smooth_scaling_factors):
//       s = max(a, 1e-5)^r;  s /= sqrt(mean(s^2));  s = max(s, 1e-4)
//   bjdmk.com.cn AWQ article, section "数学等价变换与通道自适应缩放" (AWQChannelScaler):
//       s = max(a^r / (wm^(1-r) + 1e-6), 1e-4);  s /= sqrt(max(s) * min(s)),  wm = mean_o |W[o, c]|
//
// Per-row quantizers of y = W * s (one step per output row):
//   bjdmk, same section: step = (max(y) - min(y)) / 15; restored = round(y / (step + 1e-6)) * step
//       (no zero point, no clamp);
//   msModelSlim YAML 配置示例 (weight_qconfig: per-channel, int8, symmetric, minmax), read as
//       step = max(max|y| / 127, 1e-8); restored = clip(round(y / step), -127, 127) * step.
// delta = restored / s - W is written in the weights' dtype. Every operation that decides a
// rounding is the float64 operation of the definition; a quotient y / d is first formed as
// y * (1/d) and replaced by the exact division whenever the product could round differently, and
// restored / s is the correctly rounded quotient, so delta equals the definition's float64 value.
#include <math.h>

#include "internal.h"
#include "variants.h"
#include "device_common.h"

#pragma clang fp contract(off)

namespace awq {
namespace {

constexpr int kScaleThreads = 1024;
constexpr int kThreads = 256;
constexpr int kRowWaves = kThreads / 64;

__device__ __forceinline__ double nan_max(double v, double lo) { return (v != v) ? v : (v < lo ? lo : v); }

__device__ __forceinline__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kScaleThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// One block per ratio. Pass 1 writes the unnormalised values and gathers what the
// normaliser needs; pass 2 divides (and, for the RMS formula, floors).
template <int F>
__global__ __launch_bounds__(kScaleThreads) void candidate_scales_ex_kernel(const double* __restrict__ a,
                                                                       const double* __restrict__ wm,
                                                                       int64_t d_in, RatioList ratios,
                                                                       double* __restrict__ out) {
  const int k = blockIdx.x;
  const double r = ratios.r[k];
  double* row = out + (int64_t)k * d_in;
  double mx = -INFINITY, mn = INFINITY, sq = 0.0;
  int has_nan = 0;
  for (int64_t c = threadIdx.x; c < d_in; c += kScaleThreads) {
    double v;
    if constexpr (F == kFormulaRms) {
      v = pow(nan_max(a[c], 1e-5), r);
      sq += v * v;
    } else if constexpr (F == kFormulaDuo) {
      v = nan_max(pow(a[c], r) / (pow(wm[c], 1.0 - r) + 1e-6), 1e-4);
    } else {
      v = nan_max(pow(a[c], r), 1e-4);
    }
    row[c] = v;
    if (v != v) {
      has_nan = 1;
    } else {
      mx = fmax(mx, v);
      mn = fmin(mn, v);
    }
  }
  __shared__ double red[kScaleThreads];
  __shared__ int nan_flag;
  if (threadIdx.x == 0) nan_flag = 0;
  __syncthreads();
  if (has_nan) nan_flag = 1;
  double norm;
  if constexpr (F == kFormulaRms) {
    norm = sqrt(block_sum(sq, red) / (double)d_in);  // NaN sums stay NaN
  } else {
    __shared__ double smn[kScaleThreads];
    red[threadIdx.x] = mx;
    smn[threadIdx.x] = mn;
    __syncthreads();
    for (int s = kScaleThreads / 2; s > 0; s >>= 1) {
      if (threadIdx.x < s) {
        red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + s]);
        smn[threadIdx.x] = fmin(smn[threadIdx.x], smn[threadIdx.x + s]);
      }
      __syncthreads();
    }
    norm = nan_flag ? (double)NAN : sqrt(red[0] * smn[0]);
  }
  for (int64_t c = threadIdx.x; c < d_in; c += kScaleThreads) {
    const double v = row[c] / norm;
    row[c] = (F == kFormulaRms) ? nan_max(v, 1e-4) : v;
  }
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmin(v, __shfl_xor(v, m, 64));
  return v;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, double (&w)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = (double)bf16_to_f32(v[j] & 0xFFFFu);
      w[2 * j + 1] = (double)bf16_to_f32(v[j] >> 16);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
}

__device__ __forceinline__ void load8s(const double* p, double (&s)[8]) {
  typedef double f64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f64x2 v = reinterpret_cast<const f64x2*>(p)[j];
    s[2 * j] = v.x;
    s[2 * j + 1] = v.y;
  }
}

template <typename T>
__device__ __forceinline__ const T* part_row(const WParts& w, int o, int64_t d_in) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < w.n && o >= (int)w.row_begin[i]) p = i;
  return static_cast<const T*>(w.ptr[p]) + (int64_t)(o - (int)w.row_begin[p]) * d_in;
}

// round(y / d) with d > 0: the product with the reciprocal decides unless it lies within
// 2^-30 of a rounding boundary (its error is below 2^-32 while |y/d| < 2^20); otherwise the
// exact quotient decides.
__device__ __forceinline__ double round_quotient(double y, double d, double rd) {
  const double t = y * rd;
  const double q = rint(t);
  if (fabs(t) < 0x1p20 && fabs(t - q) < 0.5 - 0x1p-30) return q;
  return rint(y / d);
}

// (q step) / s with the correctly rounded reciprocal rs = 1/s: the product, its exact residual, and one
// fused correction give the correctly rounded quotient (Markstein's theorem on division by
// multiplication; the values here are far from under- and overflow).
__device__ __forceinline__ double div_by(double a, double s, double rs) {
  const double q = a * rs;
  const double r = fma(-q, s, a);
  return fma(r, rs, q);
}

// Each wave owns kRowsPerWave output rows and runs through every candidate for them, so the rows'
// weights come from HBM once and from the caches after that. Per candidate a first pass over each row
// finds its extremes; the second goes through the row in 512-channel slices (lane l: channels 8l ..
// 8l+7 of the slice), forms each channel's reciprocal scale once for the wave's rows, and writes the
// rows' deltas: in the weights' type, or with F16 (bfloat16 weights, the Gram form of the loss) as
// float16 of delta * 2^dexp[k].
constexpr int kRowsPerWave = 4;

// v * sc (sc a power of two: exact) as float16, round to nearest even, one v_cvt_pk_f16_f32 per pair
__device__ __forceinline__ void store8_f16(uint16_t* p, const float (&v)[8], float sc) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f2 pair = {v[2 * j] * sc, v[2 * j + 1] * sc};
    h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, h2));
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(h[0], h[1], h[2], h[3]);
}

template <typename T, int Q, bool F16 = false>
__global__ __launch_bounds__(kThreads) void quant_delta_row_kernel(WParts w, int64_t d_in, int d_out,
                                                                  const double* __restrict__ cand, int n_cand,
                                                                  T* __restrict__ delta,
                                                                  const int32_t* __restrict__ dexp = nullptr) {
  constexpr int R = kRowsPerWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int o0 = (blockIdx.x * kRowWaves + wave) * R;
  if (o0 >= d_out) return;
  const T* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = part_row<T>(w, min(o0 + r, d_out - 1), d_in);
  for (int k = 0; k < n_cand; ++k) {
    const double* s = cand + (int64_t)k * d_in;
    const float sc = F16 ? ldexpf(1.f, dexp[k]) : 1.f;
    double mx[R], mn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      mx[r] = -INFINITY;
      mn[r] = INFINITY;
    }
    for (int64_t c = lane * 8; c < d_in; c += 512) {
      double sv[8];
      load8s(s + c, sv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double wv[8];
        load8(wr[r] + c, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double y = wv[j] * sv[j];
          if constexpr (Q == kQuantInt8RowSym) {
            mx[r] = fmax(mx[r], fabs(y));
          } else {
            mx[r] = fmax(mx[r], y);
            mn[r] = fmin(mn[r], y);
          }
        }
      }
    }
    double step[R], div[R], rdiv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double hi = wave_max(mx[r]);
      if constexpr (Q == kQuantInt8RowSym) {
        step[r] = hi / 127.0;
        step[r] = step[r] < 1e-8 ? 1e-8 : step[r];
        div[r] = step[r];
      } else {
        step[r] = (hi - wave_min(mn[r])) / 15.0;
        div[r] = step[r] + 1e-6;
      }
      rdiv[r] = 1.0 / div[r];
    }
    for (int64_t c = lane * 8; c < d_in; c += 512) {
      double sv[8], rs[8];
      load8s(s + c, sv);
#pragma unroll
      for (int j = 0; j < 8; ++j) rs[j] = 1.0 / sv[j];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (o0 + r >= d_out) break;  // wave-uniform
        double wv[8];
        load8(wr[r] + c, wv);
        float out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double y = wv[j] * sv[j];
          double q = round_quotient(y, div[r], rdiv[r]);
          if constexpr (Q == kQuantInt8RowSym) q = q < -127.0 ? -127.0 : (q > 127.0 ? 127.0 : q);
          out[j] = (float)(div_by(q * step[r], sv[j], rs[j]) - wv[j]);
        }
        if constexpr (F16)
          store8_f16(delta + ((int64_t)k * d_out + o0 + r) * d_in + c, out, sc);
        else
          store8(delta + ((int64_t)k * d_out + o0 + r) * d_in + c, out);
      }
    }
  }
}

__global__ void fill_kernel(double* p, int64_t n, double v) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_candidate_scales_ex(const double* act_mean, const double* w_mean, int64_t d_in,
                                      const RatioList& ratios, int n_ratios, int formula, double* cand_scales,
                                      hipStream_t st) {
  if (formula == kFormulaRms)
    hipLaunchKernelGGL(candidate_scales_ex_kernel<kFormulaRms>, dim3(n_ratios), dim3(kScaleThreads), 0, st,
                       act_mean, w_mean, d_in, ratios, cand_scales);
  else if (formula == kFormulaDuo)
    hipLaunchKernelGGL(candidate_scales_ex_kernel<kFormulaDuo>, dim3(n_ratios), dim3(kScaleThreads), 0, st,
                       act_mean, w_mean, d_in, ratios, cand_scales);
  else
    hipLaunchKernelGGL(candidate_scales_ex_kernel<kFormulaMs>, dim3(n_ratios), dim3(kScaleThreads), 0, st,
                       act_mean, w_mean, d_in, ratios, cand_scales);
  return hipGetLastError();
}

hipError_t launch_quant_delta_row(const WParts& w, int dtype, int64_t d_in, int quantizer, const double* cand_scales,
                                  int n_cand, void* delta, hipStream_t st) {
  const int d_out = (int)w.row_begin[w.n];
  const dim3 grid((unsigned)((d_out + kRowWaves * kRowsPerWave - 1) / (kRowWaves * kRowsPerWave)));
  if (dtype == 1) {
    if (quantizer == kQuantInt8RowSym)
      hipLaunchKernelGGL((quant_delta_row_kernel<uint16_t, kQuantInt8RowSym>), grid, dim3(kThreads), 0, st, w, d_in,
                         d_out, cand_scales, n_cand, static_cast<uint16_t*>(delta));
    else
      hipLaunchKernelGGL((quant_delta_row_kernel<uint16_t, kQuantInt4Row>), grid, dim3(kThreads), 0, st, w, d_in,
                         d_out, cand_scales, n_cand, static_cast<uint16_t*>(delta));
  } else {
    if (quantizer == kQuantInt8RowSym)
      hipLaunchKernelGGL((quant_delta_row_kernel<float, kQuantInt8RowSym>), grid, dim3(kThreads), 0, st, w, d_in,
                         d_out, cand_scales, n_cand, static_cast<float*>(delta));
    else
      hipLaunchKernelGGL((quant_delta_row_kernel<float, kQuantInt4Row>), grid, dim3(kThreads), 0, st, w, d_in,
                         d_out, cand_scales, n_cand, static_cast<float*>(delta));
  }
  return hipGetLastError();
}

hipError_t launch_quant_delta_row_f16(const WParts& w, int64_t d_in, int quantizer, const double* cand_scales,
                                      int n_cand, uint16_t* delta, const int32_t* dexp, hipStream_t st) {
  const int d_out = (int)w.row_begin[w.n];
  const dim3 grid((unsigned)((d_out + kRowWaves * kRowsPerWave - 1) / (kRowWaves * kRowsPerWave)));
  if (quantizer == kQuantInt8RowSym)
    hipLaunchKernelGGL((quant_delta_row_kernel<uint16_t, kQuantInt8RowSym, true>), grid, dim3(kThreads), 0, st, w,
                       d_in, d_out, cand_scales, n_cand, delta, dexp);
  else
    hipLaunchKernelGGL((quant_delta_row_kernel<uint16_t, kQuantInt4Row, true>), grid, dim3(kThreads), 0, st, w,
                       d_in, d_out, cand_scales, n_cand, delta, dexp);
  return hipGetLastError();
}

hipError_t launch_fill(double* p, int64_t n, double v, hipStream_t st) {
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace awq
