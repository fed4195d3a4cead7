// The steps either side of the search: folding the inverse scales into the source operator, and
// the float16 / packed-zero deployment form of an export.
//
// Fold: after the search the source operator of the searched linears gets the inverse scaling
// (msModelSlim "AWQ：激活感知权重量化算法说明", 支持的子图类型: the norm for norm-linear, linear1,
// v_proj, up_proj) so that X W^T = (X diag(s)^-1)(W diag(s))^T needs no extra operator
// (gsyq.cn "AWQ 离群激活平滑实操", section 四). Row r of the source (the norm weight, or row r of
// the source linear's weight or bias) is divided by s[r]; the quotient is float64, rounded to
// float32 and then to the storage dtype, both to nearest even. The output-value subgraph with
// grouped KV heads (MQA, GQA: msModelSlim 支持的子图类型, OVSubgraph) ties the o_proj scales across
// the query heads that share a KV head (tie_heads_kernel on the statistic) and folds v_proj row
// (kv, d) with the scale of o_proj channel (kv * g, d) (head_group_scales_kernel).
//
// Deployment form: float16 per-group scales and 4-bit values two per byte (bjdmk.com.cn AWQ
// article, section "GPU 硬件级反量化算子内联融合"): steps rounded to float16, zero points clipped
// to [0, 15] and packed with the even group in the low nibble; zero points outside the range and
// steps whose float16 value is not normal are counted.
#include <algorithm>

#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;

// v / s correctly rounded in float64, then rounded to float32. rs is the correctly rounded 1/s (one
// exact division per row), and a row flag `fast` says that s is a positive normal number in
// [2^-500, 2^500]. For a finite non-zero v the product q = v * rs, its exact residual
// r = v - q * s (one fma) and the fused correction q + r * rs give the correctly rounded quotient
// (Markstein's theorem on division by multiplication with a correctly rounded reciprocal; with
// |v| in the float32 range and s in that range nothing under- or overflows). Zeros, infinities and
// NaN (and rows whose s is outside the range) take the exact division, which also keeps the sign
// of a zero.
__device__ __forceinline__ float fold1(float v, double s, double rs, bool fast) {
  const double a = (double)v;
  if (fast && a != 0.0 && __builtin_isfinite(a)) {
    const double q = a * rs;
    const double r = fma(-q, s, a);
    return (float)fma(r, rs, q);
  }
  return (float)(a / s);
}

__device__ __forceinline__ bool fold_fast_row(double s) { return s >= 0x1p-500 && s <= 0x1p500; }

// 8 consecutive elements of one row per thread (16-byte aligned rows, cols % 8 == 0).
template <typename T>
__global__ __launch_bounds__(kThreads) void fold_vec_kernel(const T* __restrict__ src, int64_t ld_src,
                                                            int64_t rows, int64_t cols8,
                                                            const double* __restrict__ s, T* dst,
                                                            int64_t ld_dst) {
  const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (j >= cols8 * 8) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const double sr = s[r];
    const bool fast = fold_fast_row(sr);
    const double rs = 1.0 / sr;
    const T* p = src + r * ld_src + j;
    T* q = dst + r * ld_dst + j;
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = pack_bf16x2(fold1(bf16_to_f32(w[k] & 0xFFFFu), sr, rs, fast),
                           fold1(bf16_to_f32(w[k] >> 16), sr, rs, fast));
      *reinterpret_cast<uint4*>(q) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
      const f32x4 oa = {fold1(a.x, sr, rs, fast), fold1(a.y, sr, rs, fast), fold1(a.z, sr, rs, fast),
                        fold1(a.w, sr, rs, fast)};
      const f32x4 ob = {fold1(b.x, sr, rs, fast), fold1(b.y, sr, rs, fast), fold1(b.z, sr, rs, fast),
                        fold1(b.w, sr, rs, fast)};
      *reinterpret_cast<f32x4*>(q) = oa;
      *reinterpret_cast<f32x4*>(q + 4) = ob;
    }
  }
}

// Any shape: one element per thread.
template <typename T>
__global__ __launch_bounds__(kThreads) void fold_any_kernel(const T* __restrict__ src, int64_t ld_src,
                                                            int64_t rows, int64_t cols,
                                                            const double* __restrict__ s, T* dst,
                                                            int64_t ld_dst) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= cols) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const T v = src[r * ld_src + j];
    const double sr = s[r];
    const bool fast = fold_fast_row(sr);
    const double rs = 1.0 / sr;
    if constexpr (sizeof(T) == 2) {
      dst[r * ld_dst + j] = (uint16_t)(pack_bf16x2(fold1(bf16_to_f32(v), sr, rs, fast), 0.f) & 0xFFFFu);
    } else {
      dst[r * ld_dst + j] = fold1(v, sr, rs, fast);
    }
  }
}

// One thread per pair of groups of a row: two float16 steps and one byte of zero points.
__global__ __launch_bounds__(kThreads) void export_fp16_kernel(const float* __restrict__ qscales,
                                                               const int32_t* __restrict__ zeros,
                                                               int64_t rows, int64_t n_groups,
                                                               uint16_t* __restrict__ steps_f16,
                                                               uint8_t* __restrict__ zeros_u4,
                                                               int32_t* __restrict__ counts) {
  const int64_t gp = (n_groups + 1) / 2;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int bad_zero = 0, bad_step = 0;
  if (i < rows * gp) {
    const int64_t r = i / gp, jp = i % gp;
    uint32_t byte = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t j = 2 * jp + h;
      if (j >= n_groups) break;
      const _Float16 f = (_Float16)qscales[r * n_groups + j];
      const uint16_t fb = __builtin_bit_cast(uint16_t, f);
      steps_f16[r * n_groups + j] = fb;
      const uint32_t ex = (fb >> 10) & 0x1F;  // exponent field: 0 = zero/subnormal, 31 = inf/NaN
      bad_step += (ex == 0 || ex == 31) ? 1 : 0;
      const int32_t z = zeros[r * n_groups + j];
      const int32_t zc = z < 0 ? 0 : (z > 15 ? 15 : z);
      bad_zero += (zc != z) ? 1 : 0;
      byte |= (uint32_t)zc << (4 * h);
    }
    zeros_u4[r * gp + jp] = (uint8_t)byte;
  }
  // one atomic per wave for each count
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    bad_zero += __shfl_xor(bad_zero, m, 64);
    bad_step += __shfl_xor(bad_step, m, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    if (bad_zero) atomicAdd(&counts[0], bad_zero);
    if (bad_step) atomicAdd(&counts[1], bad_step);
  }
}

// Output-value subgraph with grouped KV heads: output channel (kv * g + j, d) of the statistic,
// for every j < g, is the mean over j of the input channels (kv * g + j, d) — summed in head order,
// divided once by g. One thread per (kv, d); it reads and writes only its own g channels, so the
// output may be the input.
__global__ __launch_bounds__(kThreads) void tie_heads_kernel(const double* a, int64_t n_kv, int64_t g,
                                                             int64_t hd, double* out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_kv * hd) return;
  const int64_t kv = i / hd, d = i % hd;
  const double* p = a + kv * g * hd + d;
  double t = p[0];
  for (int64_t j = 1; j < g; ++j) t += p[j * hd];
  t = t / (double)g;
  for (int64_t j = 0; j < g; ++j) out[(kv * g + j) * hd + d] = t;
}

// v_proj row (kv, d) takes the scale of o_proj input channel (kv * g, d).
__global__ __launch_bounds__(kThreads) void head_group_scales_kernel(const double* __restrict__ s, int64_t n_kv,
                                                                     int64_t g, int64_t hd,
                                                                     double* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_kv * hd) return;
  out[i] = s[(i / hd) * g * hd + i % hd];
}

}  // namespace

hipError_t launch_tie_heads(const double* act_mean, int64_t n_heads, int64_t n_kv, int64_t head_dim, double* tied,
                            hipStream_t st) {
  const int64_t n = n_kv * head_dim;
  hipLaunchKernelGGL(tie_heads_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     act_mean, n_kv, n_heads / n_kv, head_dim, tied);
  return hipGetLastError();
}

hipError_t launch_head_group_scales(const double* s, int64_t n_heads, int64_t n_kv, int64_t head_dim, double* s_kv,
                                    hipStream_t st) {
  const int64_t n = n_kv * head_dim;
  hipLaunchKernelGGL(head_group_scales_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, s, n_kv, n_heads / n_kv, head_dim, s_kv);
  return hipGetLastError();
}

hipError_t launch_fold_scales(const void* src, int64_t ld_src, int dtype, int64_t rows, int64_t cols,
                              const double* s, void* dst, int64_t ld_dst, bool vec, hipStream_t st) {
  const unsigned gy = (unsigned)std::min<int64_t>(rows, 65535);
  if (vec) {
    const int64_t cols8 = cols / 8;
    dim3 grid((unsigned)((cols8 + kThreads - 1) / kThreads), gy);
    if (dtype == 1)
      hipLaunchKernelGGL(fold_vec_kernel<uint16_t>, grid, dim3(kThreads), 0, st, static_cast<const uint16_t*>(src),
                         ld_src, rows, cols8, s, static_cast<uint16_t*>(dst), ld_dst);
    else
      hipLaunchKernelGGL(fold_vec_kernel<float>, grid, dim3(kThreads), 0, st, static_cast<const float*>(src), ld_src,
                         rows, cols8, s, static_cast<float*>(dst), ld_dst);
  } else {
    dim3 grid((unsigned)((cols + kThreads - 1) / kThreads), gy);
    if (dtype == 1)
      hipLaunchKernelGGL(fold_any_kernel<uint16_t>, grid, dim3(kThreads), 0, st, static_cast<const uint16_t*>(src),
                         ld_src, rows, cols, s, static_cast<uint16_t*>(dst), ld_dst);
    else
      hipLaunchKernelGGL(fold_any_kernel<float>, grid, dim3(kThreads), 0, st, static_cast<const float*>(src), ld_src,
                         rows, cols, s, static_cast<float*>(dst), ld_dst);
  }
  return hipGetLastError();
}

hipError_t launch_export_fp16(const float* qscales, const int32_t* zeros, int64_t rows, int64_t n_groups,
                              uint16_t* steps_f16, uint8_t* zeros_u4, int32_t* counts, hipStream_t st) {
  const int64_t n = rows * ((n_groups + 1) / 2);
  hipLaunchKernelGGL(export_fp16_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     qscales, zeros, rows, n_groups, steps_f16, zeros_u4, counts);
  return hipGetLastError();
}

}  // namespace awq
