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
// is within 1e-5 * step / s of the float64 value (below the bfloat16 rounding of delta for all
// but the smallest elements).
//
// quantize_pack (the final export) evaluates the quantizer in float64: 16 lanes x 8 channels
// per group, the fast path dividing by multiplying with a reciprocal accurate to an ulp, which
// decides identically unless a value lies within 1e-6 of a rounding tie; a lane whose row
// segment has such a value (or whose group has a floored step) redoes it with exact divisions.
#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;               // rows per wave (per lane)
constexpr int kRowsPerBlock = 4 * kRows;

// quant_delta layout: 16 channels per lane, 8 lanes per group, 1024 channels per block
constexpr int kDeltaChans = 16;
constexpr int kDeltaChansPerBlock = 64 * kDeltaChans;

// quantize_pack layout: 8 channels per lane, 16 lanes per group, 512 channels per block
constexpr int kPackChans = 8;
constexpr int kPackLanesPerGroup = kGroup / kPackChans;
constexpr int kPackChansPerBlock = 64 * kPackChans;

// Float32 fast path of quant_delta. With y32 = fl(w * fl(s)) (relative error 2^-23), the group's
// min/max taken on y32, step32 = fl(fl(max - min) * fl(1/15)) (relative error 2^-22 A/R +
// 3 * 2^-24, A = max |y| of the group, R = max - min) and r = round(y32 * rcp(step32)), the
// kernel forms e = fl(y32 - r * step32) with one rounding. A zero point -min/step in [-0.5, 15.5]
// bounds |y| and |r| by 15.5 step and A/R by 1.04, so e is within 15.5 * (2^-23 + 2^-22 * 1.04 +
// 3 * 2^-24) step < 8.6e-6 step of y - r * step in float64. Hence |e| <= (0.5 - kGuard32) step32
// proves |y/step - r| < 0.5, i.e. r is the float64 definition's round(y/step); the zero point
// -min * rcp(step32) is within 1.2e-5 of the float64 one and is checked the same way.
constexpr float kGuard32 = 1.0f / 65536.0f;
constexpr float kHalfGuard32 = 0.5f - kGuard32;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float elem_f32(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float elem_f32(const float* p) { return *p; }
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return (uint16_t)f32_to_bf16(v); }
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }

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

template <typename T>
__device__ __forceinline__ void exact_group(float wa, float wb, const double* s_lds, T* dst) {
  const double w0 = wa, w1 = wb;
  const double s0 = s_lds[0], s1 = s_lds[1];
  const double y0 = w0 * s0, y1 = w1 * s1;
  double mn = fmin(y0, y1), mx = fmax(y0, y1);
  // minimum and maximum over the wave: within rows of 16 lanes, then across the 4 rows
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
  const double st = group_step(mn, mx);
  const double zero = rint(-mn / st);
  const double q0 = exact_code(y0, st, zero), q1 = exact_code(y1, st, zero);
  store_pair(dst, (q0 - zero) * st / s0 - w0, (q1 - zero) * st / s1 - w1);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_delta_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                               const double* __restrict__ cand,
                                                               int n_cand, T* __restrict__ delta) {
  constexpr int E = kDeltaChans;
  __shared__ __attribute__((aligned(16))) float sc_s[2][kDeltaChansPerBlock];
  __shared__ __attribute__((aligned(16))) float sc_i[2][kDeltaChansPerBlock];  // -1/s
  __shared__ __attribute__((aligned(16))) double sc_d[2][kDeltaChansPerBlock];  // for the exact path
  __shared__ __attribute__((aligned(16))) float xpose[4][kGroup];  // per wave: one group's weights
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t cb = (int64_t)blockIdx.x * kDeltaChansPerBlock;
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
  auto stage = [&](int buf) {
    const f32x4 sv = {(float)p0.x, (float)p0.y, (float)p1.x, (float)p1.y};
    const f32x4 iv = {-__builtin_amdgcn_rcpf(sv.x), -__builtin_amdgcn_rcpf(sv.y), -__builtin_amdgcn_rcpf(sv.z),
                      -__builtin_amdgcn_rcpf(sv.w)};
    *reinterpret_cast<f32x4*>(&sc_s[buf][4 * tid]) = sv;
    *reinterpret_cast<f32x4*>(&sc_i[buf][4 * tid]) = iv;
    *reinterpret_cast<double2*>(&sc_d[buf][4 * tid]) = p0;
    *reinterpret_cast<double2*>(&sc_d[buf][4 * tid + 2]) = p1;
  };
  fetch(0);
  stage(0);
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
    if (k + 1 < n_cand) stage((k + 1) & 1);
    if (k + 2 < n_cand) fetch(k + 2);
    T* dk = delta + (int64_t)k * d_out * d_in + c0;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      float y[E];
#pragma unroll
      for (int j = 0; j < E; ++j) y[j] = wv[i][j] * s[j];
      float mn = y[0], mx = y[0];
#pragma unroll
      for (int j = 1; j < E; ++j) {
        mn = fminf(mn, y[j]);
        mx = fmaxf(mx, y[j]);
      }
      mn = fminf(mn, dpp_f32<kDppXor1>(mn));
      mx = fmaxf(mx, dpp_f32<kDppXor1>(mx));
      mn = fminf(mn, dpp_f32<kDppXor2>(mn));
      mx = fmaxf(mx, dpp_f32<kDppXor2>(mx));
      mn = fminf(mn, dpp_f32<kDppHalfMirror>(mn));
      mx = fmaxf(mx, dpp_f32<kDppHalfMirror>(mx));
      const float step = (mx - mn) * (1.0f / 15.0f);
      const float inv = __builtin_amdgcn_rcpf(step);
      const float zt = -mn * inv;
      // r = round(y / step); e = y - r step (one rounding); delta = (r step - y) / s = e * (-1/s)
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
      const bool ok = em <= kHalfGuard32 * step && fabsf(zt - rintf(zt)) <= kHalfGuard32 && step >= 2e-8f &&
                      step <= 1e30f && zt >= -0.5f && zt <= 15.5f;
      bad[i] = group_mask(__ballot(live && !ok));
      if (live && !((bad[i] >> lane) & 1)) storeE<T, E>(dk + o * d_in, out);
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
        exact_group<T>(wp.x, wp.y, &sc_d[k & 1][g * kGroup + 2 * lane],
                       delta + ((int64_t)k * d_out + row0 + i) * d_in + c);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                                 const double* __restrict__ s_in,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ qscales,
                                                                 int32_t* __restrict__ zeros) {
  constexpr int E = kPackChans;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kPackChansPerBlock + (lane / kPackLanesPerGroup) * kGroup +
                     (lane % kPackLanesPerGroup) * E;
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
      if (lane % kPackLanesPerGroup == 0) {
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
  dim3 grid((unsigned)((d_in + kDeltaChansPerBlock - 1) / kDeltaChansPerBlock),
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
  dim3 grid((unsigned)((d_in + kPackChansPerBlock - 1) / kPackChansPerBlock),
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
