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

// Two floats -> two bfloat16 (round to nearest even) in one register, first in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4 a = {v[0], v[1], v[2], v[3]};
  f32x4 b = {v[4], v[5], v[6], v[7]};
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// ---- the quantizer on one row of one 128-channel group held by 16 lanes x 8 channels
// (or 8 lanes x 16 channels)

// 64-bit lane exchange inside groups of 8 lanes (DPP quad permutes and the half-row mirror).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes

constexpr int kDppRowMirror = 0x140;  // lane i <-> 15-i within each 16 lanes

// Minimum and maximum of the group's 128 values, held as E values per lane by 128/E
// consecutive lanes (all 64 lanes must execute this).
template <int E>
__device__ __forceinline__ void group_minmax(const double (&y)[E], double& mn, double& mx) {
  static_assert(E == 8 || E == 16, "8 or 16 channels per lane");
  mn = y[0];
  mx = y[0];
#pragma unroll
  for (int j = 1; j < E; ++j) {
    mn = fmin(mn, y[j]);
    mx = fmax(mx, y[j]);
  }
  mn = fmin(mn, dpp_f64<kDppXor1>(mn));
  mx = fmax(mx, dpp_f64<kDppXor1>(mx));
  mn = fmin(mn, dpp_f64<kDppXor2>(mn));
  mx = fmax(mx, dpp_f64<kDppXor2>(mx));
  mn = fmin(mn, dpp_f64<kDppHalfMirror>(mn));
  mx = fmax(mx, dpp_f64<kDppHalfMirror>(mx));
  if constexpr (E == 8) {
    mn = fmin(mn, dpp_f64<kDppRowMirror>(mn));
    mx = fmax(mx, dpp_f64<kDppRowMirror>(mx));
  }
}

// 1/x to within an ulp: hardware estimate plus one Newton step.
__device__ __forceinline__ double rcp_nr(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return fma(r, fma(-x, r, 1.0), r);
}

// The group's step (max - min)/15 floored at 1e-8, exactly as the definition divides.
__device__ __forceinline__ double group_step(double mn, double mx) {
  const double st = (mx - mn) / 15.0;
  return st < 1e-8 ? 1e-8 : st;  // NaN passes through
}

// How far the quantizer's decisions may be from a rounding tie before the fast path, which
// uses y * (1/step) instead of y / step, is no longer guaranteed to decide like the exact
// float64 quotient (the two differ by a few ulps; the fast path is only taken for values of
// magnitude below about 1e6, where that is below 1e-9).
constexpr double kTieGuard = 0.5 - 1e-6;

// Fast-path preconditions for a group: the zero point -min/step is not within 1e-6 of a
// half-integer, is below 1e6 in magnitude, and the step is not the floor. Then every code round(y/step) + zero lies in
// [0, 15] without clamping (the minimum maps to 0 and the maximum to 15 or less), so
// q - zero = round(t) for every element.
__device__ __forceinline__ bool group_fast_ok(double zt, double zr, double step) {
  return fabs(zt - zr) <= kTieGuard && step > 1e-8 && fabs(zt) < 1e6;
}

// Exact codes of the definition: clip(round(y / step) + zero, 0, 15), zero = round(-min/step).
__device__ __forceinline__ double exact_code(double y, double step, double zero) {
  double q = rint(y / step) + zero;
  q = q < 0.0 ? 0.0 : q;
  q = q > 15.0 ? 15.0 : q;
  return q;
}

}  // namespace awq
