// a2: the candidate scales of every grid ratio, and a5: per-ratio losses and the choice.
//
// a2 follows msModelSlim "AWQ：激活感知权重量化算法说明", 原理 / 算法公式:
//   scales = act_mean.pow(ratio).clamp(min=1e-4);  scales = scales / sqrt(scales.max() * scales.min())
// with ratio = k / n_grid, k = 0 .. n_grid-1 (the grid covers [0, 1) in steps of 1/n_grid).
// a5 follows gsyq.cn "AWQ 离群激活平滑实操", section 二: start from best_loss = +inf with unit
// scales and keep a ratio only when its loss is strictly smaller (unit scales remain when none is).
#include <math.h>

#include "internal.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kScaleThreads = 1024;

// One block per ratio. The clamped powers are written first, then divided by the
// normaliser once the block knows the maximum and minimum. NaN in any channel makes the
// normaliser NaN (the maximum and minimum of a vector holding NaN are NaN).
__global__ __launch_bounds__(kScaleThreads) void candidate_scales_kernel(const double* __restrict__ a,
                                                                    int64_t d_in, int n_grid,
                                                                    double* __restrict__ out) {
  const int k = blockIdx.x;
  const double r = (double)k / (double)n_grid;
  double* row = out + (int64_t)k * d_in;
  double mx = -INFINITY, mn = INFINITY;
  int has_nan = 0;
  for (int64_t c = threadIdx.x; c < d_in; c += kScaleThreads) {
    double v = (k == 0) ? 1.0 : pow(a[c], r);
    if (!(v != v) && v < 1e-4) v = 1e-4;
    row[c] = v;
    if (v != v) {
      has_nan = 1;
    } else {
      mx = fmax(mx, v);
      mn = fmin(mn, v);
    }
  }
  __shared__ double smx[kScaleThreads], smn[kScaleThreads];
  __shared__ int snan[kScaleThreads];
  smx[threadIdx.x] = mx;
  smn[threadIdx.x] = mn;
  snan[threadIdx.x] = has_nan;
  __syncthreads();
  for (int s = kScaleThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      smx[threadIdx.x] = fmax(smx[threadIdx.x], smx[threadIdx.x + s]);
      smn[threadIdx.x] = fmin(smn[threadIdx.x], smn[threadIdx.x + s]);
      snan[threadIdx.x] |= snan[threadIdx.x + s];
    }
    __syncthreads();
  }
  const double norm = snan[0] ? (double)NAN : sqrt(smx[0] * smn[0]);
  for (int64_t c = threadIdx.x; c < d_in; c += kScaleThreads) row[c] = row[c] / norm;
}

// One block per ratio: the fixed-order float64 sum of that ratio's tile sums.
__global__ __launch_bounds__(kThreads) void loss_reduce_kernel(const double* __restrict__ tile_sse,
                                                               int64_t tiles, double denom,
                                                               double* __restrict__ losses) {
  const int k = blockIdx.x;
  const double* t = tile_sse + (int64_t)k * tiles;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < tiles; i += kThreads) s += t[i];
  __shared__ double red[kThreads];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) losses[k] = red[0] / denom;
}

__global__ __launch_bounds__(kThreads) void argmin_kernel(const double* __restrict__ losses,
                                                          int n_grid,
                                                          const double* __restrict__ cand_scales,
                                                          int64_t d_in, double* __restrict__ best,
                                                          int32_t* __restrict__ info) {
  __shared__ int kbest, knone;
  if (threadIdx.x == 0) {
    double best_loss = INFINITY;
    int kb = 0;
    for (int k = 0; k < n_grid; ++k) {
      const double l = losses[k];
      if (l < best_loss) {
        best_loss = l;
        kb = k;
      }
    }
    kbest = kb;
    info[0] = kb;
    knone = (best_loss < INFINITY) ? 0 : 1;
    info[1] = knone;
  }
  __syncthreads();
  // with no loss below +inf the scales stay at their starting value, ones (the k = 0 row of the
  // msModelSlim grid is exactly that; other grids and formulas need not start there)
  const bool none = knone != 0;
  const double* src = cand_scales + (int64_t)kbest * d_in;
  for (int64_t c = threadIdx.x; c < d_in; c += kThreads) best[c] = none ? 1.0 : src[c];
}

}  // namespace

hipError_t launch_candidate_scales(const double* act_mean, int64_t d_in, int n_grid,
                                   double* cand_scales, hipStream_t st) {
  hipLaunchKernelGGL(candidate_scales_kernel, dim3(n_grid), dim3(kScaleThreads), 0, st, act_mean, d_in,
                     n_grid, cand_scales);
  return hipGetLastError();
}

hipError_t launch_loss_argmin(const double* tile_sse, int64_t tiles_per_cand, int n_grid,
                              int64_t n_tokens, int64_t d_out, const double* cand_scales,
                              int64_t d_in, double* losses, double* best_scales,
                              int32_t* best_info, hipStream_t st) {
  const double denom = (double)n_tokens * (double)d_out;
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(n_grid), dim3(kThreads), 0, st, tile_sse,
                     tiles_per_cand, denom, losses);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(kThreads), 0, st, losses, n_grid, cand_scales,
                     d_in, best_scales, best_info);
  return hipGetLastError();
}

}  // namespace awq
