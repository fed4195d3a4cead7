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
// Every decision (step, zero point, code) is taken in float64 and equals the float64
// definition: the fast path divides by multiplying with a reciprocal accurate to an ulp, which
// decides identically unless a value lies within 1e-6 of a rounding tie; a lane whose row
// segment has such a value (or whose group has a floored step) redoes it with exact divisions.
//
// Thread layout: 128 / kChans lanes hold one 128-channel group of a row, kChans consecutive
// channels each (by default 16 lanes x 8 channels); a wave covers 64 * kChans consecutive
// channels of kRows consecutive rows, the block's four waves 4 * kRows rows. Each lane keeps its weights in registers and loops over the
// candidates, so W is read from HBM once however many candidates are evaluated, and a
// candidate's scales are read once per kRows rows (prefetched one candidate ahead).
//
// delta = What - W is formed as -(t - round(t)) * step / s with t = y / step: in exact
// arithmetic (q - zero) * step / s - w = (round(t) - t) * step / s, and here the difference is
// about 1e-16 of |w|, far below the bfloat16 rounding of delta.
#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
#ifndef AWQ_QUANT_CHANS
#define AWQ_QUANT_CHANS 8
#endif
constexpr int kChans = AWQ_QUANT_CHANS;              // channels per lane (8 or 16)
constexpr int kLanesPerGroup = kGroup / kChans;      // lanes per 128-channel group
constexpr int kRows = 4;                             // rows per wave (per lane)
constexpr int kRowsPerBlock = 4 * kRows;
constexpr int kChansPerBlock = 64 * kChans;          // channels per wave (and per block)

template <typename T>
__device__ __forceinline__ const T* row_ptr(const WParts& w, int64_t o, int64_t d_in) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < w.n && o >= w.row_begin[i]) p = i;
  return static_cast<const T*>(w.ptr[p]) + (o - w.row_begin[p]) * d_in;
}

// A lane's E weights of one row, kept in their storage format (bf16 stays packed two per
// register) and widened on use.
template <typename T, int E>
struct RowE;
template <int E>
struct RowE<uint16_t, E> {
  uint32_t b[E / 2];
  __device__ __forceinline__ void load(const uint16_t* p) {
#pragma unroll
    for (int h = 0; h < E / 8; ++h) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + 8 * h);
      b[4 * h] = u.x; b[4 * h + 1] = u.y; b[4 * h + 2] = u.z; b[4 * h + 3] = u.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < E / 2; ++j) b[j] = 0u;
  }
  __device__ __forceinline__ float operator[](int j) const {
    return (j & 1) ? __uint_as_float(b[j >> 1] & 0xFFFF0000u) : __uint_as_float(b[j >> 1] << 16);
  }
};
template <int E>
struct RowE<float, E> {
  float v[E];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(p + 4 * h);
      v[4 * h] = u.x; v[4 * h + 1] = u.y; v[4 * h + 2] = u.z; v[4 * h + 3] = u.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = 0.f;
  }
  __device__ __forceinline__ float operator[](int j) const { return v[j]; }
};

template <typename T, int E>
__device__ __forceinline__ void storeE(T* p, const float (&v)[E]) {
#pragma unroll
  for (int h = 0; h < E / 8; ++h) {
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = v[8 * h + j];
    store8(p + 8 * h, a);
  }
}

template <int E>
__device__ __forceinline__ void load_scales(const double* p, bool ok, double (&s)[E]) {
  if (ok) {
#pragma unroll
    for (int j = 0; j < E; j += 2) {
      const double2 v = *reinterpret_cast<const double2*>(p + j);
      s[j] = v.x;
      s[j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) s[j] = 1.0;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_delta_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                               const double* __restrict__ cand,
                                                               int n_cand, T* __restrict__ delta) {
  constexpr int E = kChans;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kChansPerBlock + (lane / kLanesPerGroup) * kGroup +
                     (lane % kLanesPerGroup) * E;
  const bool col_ok = c0 < d_in;  // groups are whole, so all of the lane's channels are in range
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerBlock + wave * kRows;

  RowE<T, E> wv[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t o = row0 + i;
    if (col_ok && o < d_out)
      wv[i].load(row_ptr<T>(w, o, d_in) + c0);
    else
      wv[i].zero();
  }

  double s_next[E];
  load_scales(cand + c0, col_ok, s_next);
  for (int k = 0; k < n_cand; ++k) {
    double s[E], inv_s[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      s[j] = s_next[j];
      inv_s[j] = rcp_nr(s[j]);
    }
    if (k + 1 < n_cand) load_scales(cand + (int64_t)(k + 1) * d_in + c0, col_ok, s_next);
    T* dk = delta + (int64_t)k * d_out * d_in + c0;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      double y[E];
#pragma unroll
      for (int j = 0; j < E; ++j) y[j] = (double)wv[i][j] * s[j];
      double mn, mx;
      group_minmax<E>(y, mn, mx);
      const double step = group_step(mn, mx);
      const double inv = rcp_nr(step);
      const double zt = -mn * inv;
      const double ns = -step;
      double dmax = 0.0;
      float out[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const double t = y[j] * inv;
        const double d = t - rint(t);
        dmax = fmax(dmax, fabs(d));
        out[j] = (float)((d * ns) * inv_s[j]);
      }
      if (!(group_fast_ok(zt, rint(zt), step) && dmax <= kTieGuard)) {
        const double zero = rint(-mn / step);
#pragma unroll
        for (int j = 0; j < E; ++j)
          out[j] = (float)((exact_code(y[j], step, zero) - zero) * step * inv_s[j] - (double)wv[i][j]);
      }
      const int64_t o = row0 + i;
      if (col_ok && o < d_out) storeE<T, E>(dk + o * d_in, out);
      __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                                 const double* __restrict__ s_in,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ qscales,
                                                                 int32_t* __restrict__ zeros) {
  constexpr int E = kChans;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kChansPerBlock + (lane / kLanesPerGroup) * kGroup +
                     (lane % kLanesPerGroup) * E;
  const bool col_ok = c0 < d_in;
  const int64_t grp = c0 / kGroup;
  const int64_t n_groups = d_in / kGroup;
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerBlock + wave * kRows;

  double s[E];
  load_scales(s_in + c0, col_ok, s);
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t o = row0 + i;
    const bool ok = col_ok && o < d_out;
    RowE<T, E> wv;
    if (ok)
      wv.load(row_ptr<T>(w, o, d_in) + c0);
    else
      wv.zero();
    double y[E];
#pragma unroll
    for (int j = 0; j < E; ++j) y[j] = (double)wv[j] * s[j];
    double mn, mx;
    group_minmax<E>(y, mn, mx);
    const double step = group_step(mn, mx);
    const double inv = rcp_nr(step);
    const double zt = -mn * inv;
    double zero = rint(zt);
    double q[E];
    double dmax = 0.0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const double t = y[j] * inv;
      const double r = rint(t);
      dmax = fmax(dmax, fabs(t - r));
      q[j] = r + zero;
    }
    if (!(group_fast_ok(zt, zero, step) && dmax <= kTieGuard)) {
      zero = rint(-mn / step);
#pragma unroll
      for (int j = 0; j < E; ++j) q[j] = exact_code(y[j], step, zero);
    }
    uint32_t pk[E / 8];
#pragma unroll
    for (int h = 0; h < E / 8; ++h) {
      pk[h] = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double v = q[8 * h + j];
        pk[h] |= ((v >= 0.0 && v <= 15.0) ? (uint32_t)v : 0u) << (4 * j);
      }
    }
    if (ok) {
      if constexpr (E == 16) {
        uint2 v;
        v.x = pk[0];
        v.y = pk[1];
        *reinterpret_cast<uint2*>(codes + o * (d_in / 2) + c0 / 2) = v;
      } else {
        *reinterpret_cast<uint32_t*>(codes + o * (d_in / 2) + c0 / 2) = pk[0];
      }
      if (lane % kLanesPerGroup == 0) {
        qscales[o * n_groups + grp] = (float)step;
        double z = zero;
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
  dim3 grid((unsigned)((d_in + kChansPerBlock - 1) / kChansPerBlock),
            (unsigned)((d_out + kRowsPerBlock - 1) / kRowsPerBlock));
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
  dim3 grid((unsigned)((d_in + kChansPerBlock - 1) / kChansPerBlock),
            (unsigned)((d_out + kRowsPerBlock - 1) / kRowsPerBlock));
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_pack_kernel<uint16_t>, grid, dim3(kThreads), 0, st, w, d_in, d_out, s,
                       codes, qscales, zeros);
  else
    hipLaunchKernelGGL(quantize_pack_kernel<float>, grid, dim3(kThreads), 0, st, w, d_in, d_out, s,
                       codes, qscales, zeros);
  return hipGetLastError();
}

}  // namespace awq
