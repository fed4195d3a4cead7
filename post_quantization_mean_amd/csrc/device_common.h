// Device helpers shared by the quantize->delta and pack kernels: storage conversions and
// the INT4 group quantizer of gsyq.cn "AWQ 离群激活平滑实操", section 二 (pseudo_quantize_int4),
// evaluated in float64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Loads 8 consecutive elements (bf16 bit patterns or float) starting at p as floats.
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_to_f32(u.x & 0xFFFFu); v[1] = bf16_to_f32(u.x >> 16);
  v[2] = bf16_to_f32(u.y & 0xFFFFu); v[3] = bf16_to_f32(u.y >> 16);
  v[4] = bf16_to_f32(u.z & 0xFFFFu); v[5] = bf16_to_f32(u.z >> 16);
  v[6] = bf16_to_f32(u.w & 0xFFFFu); v[7] = bf16_to_f32(u.w >> 16);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  u.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  u.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
  u.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4 a = {v[0], v[1], v[2], v[3]};
  f32x4 b = {v[4], v[5], v[6], v[7]};
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Step, zero point and reciprocal step of one 128-channel group. The 16 lanes of a row
// slice (lanes 16j .. 16j+15 of a wave) each hold 8 consecutive values y of the group.
struct GroupStep {
  double step, zero, inv;
};

__device__ __forceinline__ GroupStep group_step16(const double (&y)[8]) {
  double mn = y[0], mx = y[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fmin(mn, y[j]);
    mx = fmax(mx, y[j]);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, m, 16));
    mx = fmax(mx, __shfl_xor(mx, m, 16));
  }
  GroupStep g;
  double st = (mx - mn) / 15.0;       // 16 levels between the group's extremes
  g.step = st < 1e-8 ? 1e-8 : st;     // floor on the step (NaN passes through)
  g.zero = rint(-mn / g.step);        // zero point, round half to even, not clamped
  g.inv = 1.0 / g.step;
  return g;
}

// Code of one value: clip(round(y / step) + zero, 0, 15), round half to even. y * (1/step)
// is within two ulps of the correctly rounded quotient, so it decides every value that is
// not within 1e-6 of a half-integer; those few use the exactly rounded y / step, which makes
// the result identical to evaluating the definition in float64.
__device__ __forceinline__ double quant_code(double y, const GroupStep& g) {
  double t = y * g.inv;
  double r = rint(t);
  if (fabs(t - r) > 0.5 - 1e-6) r = rint(y / g.step);
  double q = r + g.zero;
  q = q < 0.0 ? 0.0 : q;
  q = q > 15.0 ? 15.0 : q;
  return q;
}

}  // namespace awq
