// a3: scale -> INT4 group quantize -> dequantize -> unscale -> delta, for many candidates;
// a6: the final quantize and nibble pack.
//
// The quantizer is gsyq.cn "AWQ 离群激活平滑实操", section 二 (pseudo_quantize_int4): groups of 128
// consecutive input channels of one row, step = max((max-min)/15, 1e-8), zero = round(-min/step),
// q = clamp(round(y/step) + zero, 0, 15), dequantized (q - zero) * step. The search scales the
// weights by s before quantizing and divides the dequantized values by s again (restored_w in
// the same listing; msModelSlim 缩放因子搜索流程). Codes are packed two per byte, even channel in
// the low nibble (bjdmk.com.cn AWQ article, section "GPU 硬件级反量化算子内联融合").
//
// Thread layout: 16 lanes hold one 128-channel group of a row, 8 consecutive channels each, so a
// wave covers four rows of one group per step and the block's four waves 16 consecutive rows.
// Each lane keeps its weights in registers for kRowsPerLane rows (rows 16 apart) and loops over
// the candidates, so W is read from HBM once however many candidates are evaluated, and each
// candidate's scales are read once per kRowsPerLane rows.
#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerLane = 8;
constexpr int kRowsPerBlock = 16 * kRowsPerLane;

template <typename T>
__device__ __forceinline__ const T* row_ptr(const WParts& w, int64_t o, int64_t d_in) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < w.n && o >= w.row_begin[i]) p = i;
  return static_cast<const T*>(w.ptr[p]) + (o - w.row_begin[p]) * d_in;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_delta_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                               const double* __restrict__ cand,
                                                               int n_cand, T* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane & 15;
  const int rs = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kGroup + gl * 8;
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerBlock + wave * 4 + rs;

  float wv[kRowsPerLane][8];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) {
    const int64_t o = row0 + 16 * i;
    if (o < d_out) {
      load8(row_ptr<T>(w, o, d_in) + c0, wv[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[i][j] = 0.f;
    }
  }

  for (int k = 0; k < n_cand; ++k) {
    const double* sk = cand + (int64_t)k * d_in + c0;
    double s[8], inv_s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s[j] = sk[j];
      inv_s[j] = 1.0 / s[j];
    }
    T* dk = delta + (int64_t)k * d_out * d_in + c0;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      double y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (double)wv[i][j] * s[j];
      const GroupStep g = group_step16(y);
      float d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double q = quant_code(y[j], g);
        const double w_hat = (q - g.zero) * g.step * inv_s[j];
        d[j] = (float)(w_hat - (double)wv[i][j]);
      }
      const int64_t o = row0 + 16 * i;
      if (o < d_out) store8(dk + o * d_in, d);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                                 const double* __restrict__ s_in,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ qscales,
                                                                 int32_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane & 15;
  const int rs = lane >> 4;
  const int64_t grp = blockIdx.x;
  const int64_t c0 = grp * kGroup + gl * 8;
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerBlock + wave * 4 + rs;
  const int64_t n_groups = d_in / kGroup;

  double s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = s_in[c0 + j];

#pragma unroll 2
  for (int i = 0; i < kRowsPerLane; ++i) {
    const int64_t o = row0 + 16 * i;
    const bool valid = o < d_out;
    float wv[8];
    if (valid) {
      load8(row_ptr<T>(w, o, d_in) + c0, wv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = 0.f;
    }
    double y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (double)wv[j] * s[j];
    const GroupStep g = group_step16(y);
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double q = quant_code(y[j], g);
      const uint32_t qi = (q >= 0.0 && q <= 15.0) ? (uint32_t)q : 0u;
      packed |= qi << (4 * j);
    }
    if (valid) {
      *reinterpret_cast<uint32_t*>(codes + o * (d_in / 2) + c0 / 2) = packed;
      if (gl == 0) {
        qscales[o * n_groups + grp] = (float)g.step;
        double z = g.zero;
        z = z > 2147483647.0 ? 2147483647.0 : (z < -2147483648.0 ? -2147483648.0 : z);
        zeros[o * n_groups + grp] = (z == z) ? (int32_t)z : 0;
      }
    }
  }
}

}  // namespace

hipError_t launch_quant_delta(const WParts& w, int dtype, int64_t d_in, const double* cand_scales,
                              int n_cand, void* delta, hipStream_t st) {
  const int64_t d_out = w.row_begin[w.n];
  dim3 grid((unsigned)(d_in / kGroup), (unsigned)((d_out + kRowsPerBlock - 1) / kRowsPerBlock));
  if (dtype == 1)
    hipLaunchKernelGGL(quant_delta_kernel<uint16_t>, grid, dim3(kThreads), 0, st, w, d_in, d_out,
                       cand_scales, n_cand, static_cast<uint16_t*>(delta));
  else
    hipLaunchKernelGGL(quant_delta_kernel<float>, grid, dim3(kThreads), 0, st, w, d_in, d_out,
                       cand_scales, n_cand, static_cast<float*>(delta));
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const WParts& w, int dtype, int64_t d_in, const double* s,
                                uint8_t* codes, float* qscales, int32_t* zeros, hipStream_t st) {
  const int64_t d_out = w.row_begin[w.n];
  dim3 grid((unsigned)(d_in / kGroup), (unsigned)((d_out + kRowsPerBlock - 1) / kRowsPerBlock));
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_pack_kernel<uint16_t>, grid, dim3(kThreads), 0, st, w, d_in, d_out, s,
                       codes, qscales, zeros);
  else
    hipLaunchKernelGGL(quantize_pack_kernel<float>, grid, dim3(kThreads), 0, st, w, d_in, d_out, s,
                       codes, qscales, zeros);
  return hipGetLastError();
}

}  // namespace awq
