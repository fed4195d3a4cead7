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
// Every decision (step, zero point, code) equals the float64 definition.
//
// quant_delta (every candidate) evaluates the quantizer in float32: 8 lanes hold one 128-channel
// group of a row, 16 consecutive channels each; a wave covers 1024 channels of kRows rows and
// the block's four waves 4 * kRows rows. Each lane keeps its weights in registers and loops
// over the candidates, so W is read from HBM once however many candidates are evaluated. The
// block converts a candidate's float64 scales to float32 (with -1/s) once, in LDS. Each element
// takes r = round(y / step) and the residual e = y - r * step, which gives
// delta = What - W = (r * step - y) / s = -e / s directly (in exact arithmetic
// (q - zero) * step / s - w with q - zero = r, as no code is clipped when the zero point lies in
// [0, 15]). The residual also proves the decision: |e| <= (0.5 - 2^-16) * step means r equals
// the float64 definition's round(y / step) (error bound at kGuard32); the zero point is checked
// the same way. A group that fails a check (a value within 2^-16 of a rounding tie, a zero point
// outside [-0.5, 15.5], a step near the 1e-8 floor, a non-finite value) is recomputed by the
// whole wave in float64 with exact divisions, as the definition is written. The float32 delta
// -e * (-1/s) is within 1e-5 * step / s of the float64 value: 8.6e-6 * step / s from e (bound at
// kGuard32) plus two float32 roundings (of -1/s and of the product) on |e| / s <= step / (2 s).
// That is below the bfloat16 rounding of delta for all but the smallest elements.
//
// quantize_pack (the final export, one scale vector) uses the same layout, float32 fast path and
// proof: its codes are r + zero, and flagged groups are redone by the whole wave in float64.
#include <algorithm>

#include <cfloat>

#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;               // rows per wave (per lane)
constexpr int kRowsPerBlock = 4 * kRows;
#ifndef AWQ_PACK_ROWS
#define AWQ_PACK_ROWS 1
#endif
#ifndef AWQ_PACK_NT
#define AWQ_PACK_NT 1  // the pack reads W once: non-temporal loads (measured 6-9 % faster on large layers)
#endif
#ifndef AWQ_PACK_GRID
#define AWQ_PACK_GRID 1024
#endif
#ifndef AWQ_PACK_DEPTH
#define AWQ_PACK_DEPTH 1
#endif
constexpr int kPackRows = AWQ_PACK_ROWS;    // pack: rows per wave per row block
constexpr int kPackDepth = AWQ_PACK_DEPTH;  // pack: row blocks in flight ahead of the current one

// Layout of both kernels: 16 channels per lane, 8 lanes per group, 1024 channels per wave; a
// quant_delta block's four waves take different rows of one 1024-channel slice, a pack block's
// four waves up to four adjacent slices of the same rows
constexpr int kChans = 16;
constexpr int kChansPerBlock = 64 * kChans;

// The float32 fast path. With y32 = fl(w * fl(s)) (relative error 2^-23), the group's
// min/max taken on y32, step32 = fl(fl(max - min) * fl(1/15)) (relative error 2^-22 A/R +
// 3 * 2^-24, A = max |y| of the group, R = max - min) and r = round(y32 * rcp(step32)), the
// kernel forms e = fl(y32 - r * step32) with one rounding. A zero point -min/step in [-0.5, 15.5]
// bounds |y| and |r| by 15.5 step and A/R by 1.04, so e is within 15.5 * (2^-23 + 2^-22 * 1.04 +
// 3 * 2^-24) step < 8.6e-6 step of y - r * step in float64. Hence |e| <= (0.5 - kGuard32) step32
// proves |y/step - r| < 0.5, i.e. r is the float64 definition's round(y/step); the zero point
// -min * rcp(step32) is within 1.2e-5 of the float64 one and is checked the same way.
// The pack checks in units of the step instead: t = fl(y32 * inv32 + zero) (one rounding, inv32 =
// rcp(step32) within 2^-23 relative) is within 15.5 * (2^-23 + 2^-22 * 1.04 + 3 * 2^-24 + 2^-23)
// + 2^-21 < 1.1e-5 of y / step + zero, so |t - round(t)| <= 0.5 - kGuard32 proves that round(t) is
// the definition's round(y / step) + zero (no tie within reach, zero an integer).
constexpr float kGuard32 = 1.0f / 65536.0f;
constexpr float kHalfGuard32 = 0.5f - kGuard32;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const WParts& w, int64_t o, int64_t d_in) {
  // stacked rows fit in 32 bits (the C ABI caps d_out); the part search stays in scalar
  // registers when o is wave-uniform
  const int o32 = (int)o;
  if (w.n == 1) return static_cast<const T*>(w.ptr[0]) + (int64_t)o32 * d_in;
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < w.n && o32 >= (int)w.row_begin[i]) p = i;
  return static_cast<const T*>(w.ptr[p]) + (int64_t)(o32 - (int)w.row_begin[p]) * d_in;
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
  __device__ __forceinline__ void set(int h, const uint4& u) {
    b[4 * h] = u.x; b[4 * h + 1] = u.y; b[4 * h + 2] = u.z; b[4 * h + 3] = u.w;
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
  __device__ __forceinline__ void set(int h, const uint4& u) {
    v[4 * h] = __uint_as_float(u.x); v[4 * h + 1] = __uint_as_float(u.y);
    v[4 * h + 2] = __uint_as_float(u.z); v[4 * h + 3] = __uint_as_float(u.w);
  }
};

// A wave's 1024-channel slice of one row loaded with consecutive lanes on consecutive 16 bytes
// (whole cache lines per instruction; a lane stride of 32 bytes reads about 30 % slower), then
// regrouped through the wave's LDS slot into each lane's 16 consecutive channels.
template <typename T, int E>
struct RawRow {
  static constexpr int NV = E * (int)sizeof(T) / 16;  // 16-byte words per lane
  uint4 u[NV];
  __device__ __forceinline__ void load(const T* row_slice, int valid16, int lane) {
#if AWQ_PACK_NT
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v* q = reinterpret_cast<const u32x4v*>(row_slice);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      u[v] = make_uint4(0u, 0u, 0u, 0u);
      if (v * 64 + lane < valid16) {
        const u32x4v t = __builtin_nontemporal_load(q + v * 64 + lane);
        u[v] = make_uint4(t.x, t.y, t.z, t.w);
      }
    }
#else
    const uint4* q = reinterpret_cast<const uint4*>(row_slice);
#pragma unroll
    for (int v = 0; v < NV; ++v) u[v] = (v * 64 + lane < valid16) ? q[v * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
#endif
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int v = 0; v < NV; ++v) u[v] = make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ void regroup(uint4* slot, int lane, RowE<T, E>& dst) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) slot[v * 64 + lane] = u[v];
#pragma unroll
    for (int h = 0; h < NV; ++h) dst.set(h, slot[lane * NV + h]);
  }
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

// Float32 quantizer parameters of one row's group, whose 128 values y are held by 8 lanes x 16:
// min/max over the group, step = (max - min) / 15, its reciprocal and the zero point -min/step.
// `ok` holds when the zero point is at least kGuard32 from a rounding tie and lies in
// [-0.5, 15.5], and the step is normal and above the floor (false for NaN).
struct FastGroup {
  float step, inv, zt;
  bool ok;
};
// The group's extremes with NaN-propagating minimum / maximum (v_minimum3_f32 / v_maximum3_f32,
// IEEE 754-2019): a NaN weight (or scale) makes the step NaN, an infinity makes it infinite, and
// either fails the step test below, so the group is redone in float64, where the definition's max
// and min propagate NaN too. (IEEE minNum / maxNum, fminf / fmaxf, would drop a NaN and quantize the
// rest of the group with a finite step.)
__device__ __forceinline__ float lane_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float lane_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <int E>
__device__ __forceinline__ FastGroup fast_group(const float (&y)[E]) {
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int j = 1; j < E; ++j) {
    mn = lane_min(mn, y[j]);
    mx = lane_max(mx, y[j]);
  }
  mn = lane_min(mn, dpp_f32<kDppXor1>(mn));
  mx = lane_max(mx, dpp_f32<kDppXor1>(mx));
  mn = lane_min(mn, dpp_f32<kDppXor2>(mn));
  mx = lane_max(mx, dpp_f32<kDppXor2>(mx));
  mn = lane_min(mn, dpp_f32<kDppHalfMirror>(mn));
  mx = lane_max(mx, dpp_f32<kDppHalfMirror>(mx));
  FastGroup g;
  g.step = (mx - mn) * (1.0f / 15.0f);
  g.inv = __builtin_amdgcn_rcpf(g.step);
  g.zt = -mn * g.inv;
  g.ok = fabsf(g.zt - rintf(g.zt)) <= kHalfGuard32 && g.step >= 2e-8f && g.step <= 1e30f && g.zt >= -0.5f &&
         g.zt <= 15.5f;
  return g;
}

// One group of one row by a whole wave, in float64 exactly as the definition is written, 2
// channels per lane (w0, w1 with scales s_lds[0..1]): y = w s, step = max((max-min)/15, 1e-8),
// zero = round(-min/step), q = clip(round(y/step) + zero, 0, 15), What = (q - zero) step / s,
// and delta = What - w is stored at dst[0..1].
__device__ __forceinline__ void store_pair(uint16_t* p, double a, double b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2((float)a, (float)b);
}
__device__ __forceinline__ void store_pair(float* p, double a, double b) {
  *reinterpret_cast<float2*>(p) = make_float2((float)a, (float)b);
}

// Float16 output of delta scaled by sc (a power of two, exact) for the Gram form of the loss.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
// E float32 values as float16 (round to nearest even; one v_cvt_pk_f16_f32 per pair)
template <int E>
__device__ __forceinline__ void storeE_f16(uint16_t* p, const float (&v)[E]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  uint32_t u[E / 2];
#pragma unroll
  for (int j = 0; j < E / 2; ++j) {
    const f2 pair = {v[2 * j], v[2 * j + 1]};
    u[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, h2));
  }
#pragma unroll
  for (int h = 0; h < E / 8; ++h)
    *reinterpret_cast<uint4*>(p + 8 * h) = make_uint4(u[4 * h], u[4 * h + 1], u[4 * h + 2], u[4 * h + 3]);
}

// Extends a lane mask to whole groups of 8 lanes: any lane of a group set -> all of them.
__device__ __forceinline__ uint64_t group_mask(uint64_t b) {
  b |= b >> 1;
  b |= b >> 2;
  b |= b >> 4;
  b &= 0x0101010101010101ull;
  b |= b << 1;
  b |= b << 2;
  b |= b << 4;
  return b;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Minimum and maximum over the whole wave: within rows of 16 lanes, then across the 4 rows.
// Group minimum and maximum over the wave's 128 values (two per lane), propagating NaN as the
// definition's max / min do (fmin / fmax alone would drop a NaN operand): a group holding a NaN
// gets a NaN step, hence NaN restored values and codes (stored as 0).
__device__ __forceinline__ void wave_minmax_f64(double& mn, double& mx);
__device__ __forceinline__ void group_minmax_f64(double y0, double y1, double& mn, double& mx) {
  mn = fmin(y0, y1);
  mx = fmax(y0, y1);
  wave_minmax_f64(mn, mx);
  if (__ballot(y0 != y0 || y1 != y1)) mn = mx = __builtin_nan("");
}

__device__ __forceinline__ void wave_minmax_f64(double& mn, double& mx) {
  mn = fmin(mn, dpp_f64<kDppXor1>(mn));
  mx = fmax(mx, dpp_f64<kDppXor1>(mx));
  mn = fmin(mn, dpp_f64<kDppXor2>(mn));
  mx = fmax(mx, dpp_f64<kDppXor2>(mx));
  mn = fmin(mn, dpp_f64<kDppHalfMirror>(mn));
  mx = fmax(mx, dpp_f64<kDppHalfMirror>(mx));
  mn = fmin(mn, dpp_f64<kDppRowMirror>(mn));
  mx = fmax(mx, dpp_f64<kDppRowMirror>(mx));
  mn = fmin(fmin(readlane_f64(mn, 0), readlane_f64(mn, 16)), fmin(readlane_f64(mn, 32), readlane_f64(mn, 48)));
  mx = fmax(fmax(readlane_f64(mx, 0), readlane_f64(mx, 16)), fmax(readlane_f64(mx, 32), readlane_f64(mx, 48)));
}

template <typename T, bool F16 = false>
__device__ __forceinline__ void exact_group(float wa, float wb, const double* s_lds, T* dst, float sc = 1.f) {
  const double w0 = wa, w1 = wb;
  const double s0 = s_lds[0], s1 = s_lds[1];
  const double y0 = w0 * s0, y1 = w1 * s1;
  double mn, mx;
  group_minmax_f64(y0, y1, mn, mx);
  const double st = group_step(mn, mx);
  const double zero = rint(-mn / st);
  const double q0 = exact_code(y0, st, zero), q1 = exact_code(y1, st, zero);
  const double d0 = (q0 - zero) * st / s0 - w0, d1 = (q1 - zero) * st / s1 - w1;
  if constexpr (F16)
    *reinterpret_cast<uint32_t*>(dst) = pack_f16x2((float)d0 * sc, (float)d1 * sc);
  else
    store_pair(dst, d0, d1);
}

// With F16 (bfloat16 weights only) delta is written as float16 of delta * 2^dexp[k] instead of in
// the weights' type.
template <typename T, bool F16 = false>
__global__ __launch_bounds__(kThreads) void quant_delta_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                               const double* __restrict__ cand,
                                                               int n_cand, T* __restrict__ delta,
                                                               const int32_t* __restrict__ dexp = nullptr) {
  constexpr int E = kChans;
  __shared__ __attribute__((aligned(16))) float sc_s[2][kChansPerBlock];
  __shared__ __attribute__((aligned(16))) float sc_i[2][kChansPerBlock];  // -1/s (F16: times 2^dexp[k])
  __shared__ __attribute__((aligned(16))) double sc_d[2][kChansPerBlock];  // for the exact path
  __shared__ __attribute__((aligned(16))) float xpose[4][kGroup];  // per wave: one group's weights
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: row math stays scalar
  const int64_t cb = (int64_t)blockIdx.x * kChansPerBlock;
  const int cl = lane * E;  // group lane/8, 16-channel slice lane%8: channels cb + 16*lane ..
  const int64_t c0 = cb + cl;
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

  // Each thread converts 4 of the block's 1024 scales of a candidate (fetched one candidate
  // ahead) into the LDS buffer of that candidate.
  const int64_t cs = cb + 4 * tid;
  const bool cs_ok = cs < d_in;
  double2 p0 = {1.0, 1.0}, p1 = {1.0, 1.0};
  auto fetch = [&](int k) {
    if (cs_ok) {
      const double2* p = reinterpret_cast<const double2*>(cand + (int64_t)k * d_in + cs);
      p0 = p[0];
      p1 = p[1];
    }
  };
  // F16: -1/s is stored times the candidate's 2^dexp, which scales every fast-path delta exactly
  // (a power of two, far from float32's limits)
  auto stage = [&](int buf, int kk) {
    const f32x4 sv = {(float)p0.x, (float)p0.y, (float)p1.x, (float)p1.y};
    const float m = F16 ? -ldexpf(1.f, dexp[kk]) : -1.f;
    const f32x4 iv = {m * __builtin_amdgcn_rcpf(sv.x), m * __builtin_amdgcn_rcpf(sv.y), m * __builtin_amdgcn_rcpf(sv.z),
                      m * __builtin_amdgcn_rcpf(sv.w)};
    *reinterpret_cast<f32x4*>(&sc_s[buf][4 * tid]) = sv;
    *reinterpret_cast<f32x4*>(&sc_i[buf][4 * tid]) = iv;
    *reinterpret_cast<double2*>(&sc_d[buf][4 * tid]) = p0;
    *reinterpret_cast<double2*>(&sc_d[buf][4 * tid + 2]) = p1;
  };
  fetch(0);
  stage(0, 0);
  if (n_cand > 1) fetch(1);

  uint64_t bad[kRows];  // per row: the lanes of the flagged groups (wave-uniform)
  for (int k = 0; k < n_cand; ++k) {
    __syncthreads();  // buffer k&1 is complete; nobody reads buffer (k+1)&1 any more
    float s[E], nis[E];
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sc_s[k & 1][cl + 4 * h]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&sc_i[k & 1][cl + 4 * h]);
      s[4 * h] = a.x; s[4 * h + 1] = a.y; s[4 * h + 2] = a.z; s[4 * h + 3] = a.w;
      nis[4 * h] = b.x; nis[4 * h + 1] = b.y; nis[4 * h + 2] = b.z; nis[4 * h + 3] = b.w;
    }
    if (k + 1 < n_cand) stage((k + 1) & 1, k + 1);
    if (k + 2 < n_cand) fetch(k + 2);
    T* dk = delta + (int64_t)k * d_out * d_in + c0;
    float sc = 1.f;
    if constexpr (F16) sc = ldexpf(1.f, dexp[k]);
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      float y[E];
#pragma unroll
      for (int j = 0; j < E; ++j) y[j] = wv[i][j] * s[j];
      const FastGroup fg = fast_group<E>(y);
      const float step = fg.step, inv = fg.inv;
      // r = round(y / step); e = y - r step (one rounding); delta = (r step - y) / s = e * (-1/s)
      // (F16: delta * 2^dexp[k])
      float em = 0.f;
      float out[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float e = fmaf(-rintf(y[j] * inv), step, y[j]);
        em = j == 0 ? fabsf(e) : fmaxf(em, fabsf(e));
        out[j] = e * nis[j];
      }
      // every test is false for NaN; the group decides as a whole (its 8 lanes agree); lanes
      // past the last row or channel never take the exact path
      const int64_t o = row0 + i;
      const bool live = col_ok && o < d_out;
      const bool ok = fg.ok && em <= kHalfGuard32 * step;
      bad[i] = group_mask(__ballot(live && !ok));
      if (live && !((bad[i] >> lane) & 1)) {
        if constexpr (F16)
          storeE_f16<E>(dk + o * d_in, out);
        else
          storeE<T, E>(dk + o * d_in, out);
      }
      __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
    }
    // The flagged groups (rare: near a rounding tie, or unusual ranges), each by the whole wave
    // in float64 as the definition is written: 2 channels per lane.
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      uint64_t m = bad[i];
      while (m) {
        const int g = __builtin_ctzll(m) >> 3;  // a flagged group's 8 lanes are all set
        m &= ~(0xFFull << (8 * g));
        if ((lane >> 3) == g) {  // the group's owners hand its 128 weights over through LDS
#pragma unroll
          for (int h = 0; h < E / 4; ++h) {
            const f32x4 v = {wv[i][4 * h], wv[i][4 * h + 1], wv[i][4 * h + 2], wv[i][4 * h + 3]};
            *reinterpret_cast<f32x4*>(&xpose[wave][(lane & 7) * E + 4 * h]) = v;
          }
        }
        const float2 wp = *reinterpret_cast<const float2*>(&xpose[wave][2 * lane]);
        const int64_t c = cb + g * kGroup + 2 * lane;
        exact_group<T, F16>(wp.x, wp.y, &sc_d[k & 1][g * kGroup + 2 * lane],
                            delta + ((int64_t)k * d_out + row0 + i) * d_in + c, sc);
      }
    }
  }
}

// The exact path of the pack for one group of one row, by the whole wave (2 channels per lane,
// w0/w1 with scales s[0..1]): codes of the float64 definition into one byte (even channel in the
// low nibble), and lane 0 writes the group's step (as float32) and zero point (saturated to int32).
__device__ __forceinline__ void exact_pack_group(float wa, float wb, const double* s, uint8_t* code, float* qs,
                                                 int32_t* zp, int lane) {
  const double y0 = (double)wa * s[0], y1 = (double)wb * s[1];
  double mn, mx;
  group_minmax_f64(y0, y1, mn, mx);
  const double st = group_step(mn, mx);
  const double zero = rint(-mn / st);
  double q0 = exact_code(y0, st, zero), q1 = exact_code(y1, st, zero);
  q0 = q0 == q0 ? q0 : 0.0;  // a NaN code (non-finite input) packs as 0
  q1 = q1 == q1 ? q1 : 0.0;
  *code = (uint8_t)((uint32_t)q0 | ((uint32_t)q1 << 4));
  if (lane == 0) {
    *qs = (float)st;
    double z = zero;
    z = z > 2147483647.0 ? 2147483647.0 : (z < -2147483648.0 ? -2147483648.0 : z);
    *zp = (z == z) ? (int32_t)z : 0;
  }
}

// a6: codes of W * s packed two per byte, with each group's step and zero point. The lane layout
// and float32 fast path of quant_delta (one scale vector, so no candidate loop): q = round(y / step)
// + zero, proved equal to the float64 definition by the residual and zero-point checks; flagged
// groups are redone by the whole wave in float64. A block's four waves take four adjacent
// 1024-channel slices of the same row (spb = 4), so each row block reads 8 KiB of one row and
// writes 2 KiB of its codes and 128 bytes each of its steps and zero points (for bf16 weights: 12 %
// faster on the 70B layers than four waves on four rows of one slice, with the codes' non-temporal
// stores). When the row's slice count is not a multiple of 4, spb = 2 or 1 slices per block with
// 2 or 4 rows per row block, so that no wave is idle.
template <typename T, int SPB>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                                 const double* __restrict__ s_in,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ qscales,
                                                                 int32_t* __restrict__ zeros) {
  constexpr int E = kChans;
  __shared__ __attribute__((aligned(16))) float xpose[4][kGroup];  // per wave: one group's weights
  __shared__ uint4 slot[4][RawRow<T, E>::NV * 64];                 // per wave: one row slice
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: row math stays scalar
  // this wave's 1024-channel slice (wave % SPB of the block's SPB slices; SPB divides the row's
  // slice count, so a slice past d_in occurs only in a single-slice row narrower than 1024) and its
  // rows (wave / SPB of the row block's 4 / SPB row sets); compile-time SPB keeps this arithmetic
  // scalar
  const int sw = SPB == 4 ? wave : wave % SPB, rw = SPB == 4 ? 0 : wave / SPB;  // wave < 4
  constexpr int rows_rb = (4 / SPB) * kPackRows;
  const int64_t cb = ((int64_t)blockIdx.x * SPB + sw) * kChansPerBlock;
  const int64_t c0 = cb + lane * E;
  const bool col_ok = c0 < d_in;
  const int64_t n_groups = d_in / kGroup;
  const int64_t n_rb = (d_out + rows_rb - 1) / rows_rb;
  // Row blocks blockIdx.y, blockIdx.y + gridDim.y, ...; the weights of the next kPackDepth row
  // blocks are in flight while the current one is quantized.
  const int valid16 =
      (int)((std::max<int64_t>(0, std::min<int64_t>(d_in - cb, kChansPerBlock)) * (int64_t)sizeof(T)) / 16);
  auto load_rows = [&](RawRow<T, E>(&dst)[kPackRows], int64_t rb) {
#pragma unroll
    for (int i = 0; i < kPackRows; ++i) {
      const int64_t o = rb * rows_rb + rw * kPackRows + i;
      if (o < d_out)
        dst[i].load(row_ptr<T>(w, o, d_in) + cb, valid16, lane);
      else
        dst[i].zero();
    }
  };
  RawRow<T, E> raw[kPackDepth + 1][kPackRows];
#pragma unroll
  for (int d = 0; d <= kPackDepth; ++d) {
    const int64_t rb = blockIdx.y + (int64_t)d * gridDim.y;
    if (d < kPackDepth && rb < n_rb) load_rows(raw[d], rb);
  }
  float s[E];
#pragma unroll
  for (int j = 0; j < E; j += 2) {
    double2 v = {1.0, 1.0};
    if (col_ok) v = *reinterpret_cast<const double2*>(s_in + c0 + j);
    s[j] = (float)v.x;
    s[j + 1] = (float)v.y;
  }

  for (int64_t rb = blockIdx.y; rb < n_rb; rb += gridDim.y) {
    const int64_t row0 = rb * rows_rb + rw * kPackRows;
    RowE<T, E> wv[kPackRows];
#pragma unroll
    for (int i = 0; i < kPackRows; ++i) raw[0][i].regroup(slot[wave], lane, wv[i]);
    if (rb + (int64_t)kPackDepth * gridDim.y < n_rb) load_rows(raw[kPackDepth], rb + (int64_t)kPackDepth * gridDim.y);
    uint64_t bad[kPackRows];
#pragma unroll
    for (int i = 0; i < kPackRows; ++i) {
      float y[E];
#pragma unroll
      for (int j = 0; j < E; ++j) y[j] = wv[i][j] * s[j];
      const FastGroup fg = fast_group<E>(y);
      const float z = rintf(fg.zt);
      // t = y / step + zero with one rounding, q = round(t) (the code: the zero point is an integer,
      // so away from ties round(y / step) + zero = round(t)), d = t - q exactly; the codes of the
      // even and odd channels go into the bytes of two words (v_cvt_pk_u8_f32, exact for the
      // integers 0..15), which one shift-or turns into nibble pairs.
      float em = 0.f;
      uint32_t ev[E / 8], od[E / 8];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float t = fmaf(y[j], fg.inv, z);
        const float q = rintf(t);
        em = j == 0 ? fabsf(t - q) : fmaxf(em, fabsf(t - q));
        uint32_t& dst = (j & 1) ? od[j / 8] : ev[j / 8];
        dst = __builtin_amdgcn_cvt_pk_u8_f32(q, (j % 8) / 2, (j % 8) < 2 ? 0u : dst);
      }
      const int64_t o = row0 + i;
      const bool live = col_ok && o < d_out;
      const bool ok = fg.ok && em <= kHalfGuard32;
      bad[i] = group_mask(__ballot(live && !ok));
      if (live && !((bad[i] >> lane) & 1)) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {ev[0] | (od[0] << 4), ev[1] | (od[1] << 4)};  // q in [0, 15] when the checks pass
        // row bases are wave-uniform (scalar registers), the lane offsets 32-bit; the block's four
        // waves write 2 KiB of one row's codes, non-temporal (written once, not read again here)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(codes + (o * (d_in / 2) + cb / 2) + (uint32_t)(lane * (E / 2))));
        if ((lane & 7) == 0) {
          const int64_t gb = o * n_groups + cb / kGroup;
          qscales[gb + (uint32_t)(lane >> 3)] = fg.step;
          zeros[gb + (uint32_t)(lane >> 3)] = (int32_t)z;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < kPackRows; ++i) {
      uint64_t m = bad[i];
      const int64_t o = row0 + i;
      while (m) {
        const int g = __builtin_ctzll(m) >> 3;
        m &= ~(0xFFull << (8 * g));
        if ((lane >> 3) == g) {
#pragma unroll
          for (int h = 0; h < E / 4; ++h) {
            const f32x4 v = {wv[i][4 * h], wv[i][4 * h + 1], wv[i][4 * h + 2], wv[i][4 * h + 3]};
            *reinterpret_cast<f32x4*>(&xpose[wave][(lane & 7) * E + 4 * h]) = v;
          }
        }
        const float2 wp = *reinterpret_cast<const float2*>(&xpose[wave][2 * lane]);
        const int64_t c = cb + g * kGroup + 2 * lane;
        const int64_t gi = o * n_groups + (cb + g * kGroup) / kGroup;
        exact_pack_group(wp.x, wp.y, s_in + c, codes + o * (d_in / 2) + c / 2, qscales + gi, zeros + gi, lane);
      }
    }
#pragma unroll
    for (int d = 0; d < kPackDepth; ++d)
#pragma unroll
      for (int i = 0; i < kPackRows; ++i) raw[d][i] = raw[d + 1][i];
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

hipError_t launch_quant_delta_f16(const WParts& w, int64_t d_in, const double* cand_scales, int n_cand,
                                  uint16_t* delta, const int32_t* dexp, hipStream_t st) {
  const int64_t d_out = w.row_begin[w.n];
  dim3 grid((unsigned)((d_in + kChansPerBlock - 1) / kChansPerBlock),
            (unsigned)((d_out + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((quant_delta_kernel<uint16_t, true>), grid, dim3(kThreads), 0, st, w, d_in, d_out,
                     cand_scales, n_cand, delta, dexp);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const WParts& w, int dtype, int64_t d_in, const double* s,
                                uint8_t* codes, float* qscales, int32_t* zeros, hipStream_t st) {
  const int64_t d_out = w.row_begin[w.n];
  // four resident blocks per compute unit (4 waves per SIMD at the kernel's register use), each
  // looping over row blocks
  const int64_t slices = (d_in + kChansPerBlock - 1) / kChansPerBlock;
  const int spb = slices % 4 == 0 ? 4 : (slices % 2 == 0 ? 2 : 1);  // slices per block
  const int64_t col_blocks = slices / spb;
  const int64_t row_blocks = (d_out + (4 / spb) * kPackRows - 1) / ((4 / spb) * kPackRows);
  const int64_t ry = std::max<int64_t>(1, std::min<int64_t>(row_blocks, AWQ_PACK_GRID / col_blocks));
  dim3 grid((unsigned)col_blocks, (unsigned)ry);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, st, w, d_in, d_out, s, codes, qscales, zeros);
  };
  if (dtype == 1)
    launch(spb == 4 ? quantize_pack_kernel<uint16_t, 4>
                    : (spb == 2 ? quantize_pack_kernel<uint16_t, 2> : quantize_pack_kernel<uint16_t, 1>));
  else
    launch(spb == 4 ? quantize_pack_kernel<float, 4>
                    : (spb == 2 ? quantize_pack_kernel<float, 2> : quantize_pack_kernel<float, 1>));
  return hipGetLastError();
}

}  // namespace awq
