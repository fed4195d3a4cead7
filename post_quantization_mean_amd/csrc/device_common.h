// Device helpers of the quantize->delta and pack kernels: storage conversions, lane exchanges,
// and the float64 pieces of the INT4 group quantizer of gsyq.cn "AWQ 离群激活平滑实操", section 二
// (pseudo_quantize_int4) used by their exact paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

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

// 64-bit lane exchange by a DPP pattern (quad permutes, the half-row and row mirrors).
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

// The group's step (max - min)/15 floored at 1e-8, exactly as the definition divides.
__device__ __forceinline__ double group_step(double mn, double mx) {
  const double st = (mx - mn) / 15.0;
  return st < 1e-8 ? 1e-8 : st;  // NaN passes through
}

// Exact codes of the definition: clip(round(y / step) + zero, 0, 15), zero = round(-min/step).
__device__ __forceinline__ double exact_code(double y, double step, double zero) {
  double q = rint(y / step) + zero;
  q = q < 0.0 ? 0.0 : q;
  q = q > 15.0 ? 15.0 : q;
  return q;
}

}  // namespace awq
