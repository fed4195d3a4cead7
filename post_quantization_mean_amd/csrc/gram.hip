// The loss of every ratio through the Gram matrix of the activations.
//
// A ratio's loss is mean((X W^T - X What^T)^2) over the N x d_out outputs (gsyq.cn "AWQ 离群激活
// 平滑实操", section 二; bjdmk.com.cn AWQ article, L(s) in "数学等价变换与通道自适应缩放"). With
// delta = What - W that is sum_o ||X delta[o]^T||^2 / (N d_out), and ||X v||^2 = v (X^T X) v^T, so
// with G = X^T X ([d_in, d_in], formed once per layer) the loss is the quadratic form
// sum_o delta[o] G delta[o]^T / (N d_out): 2 d_out d_in^2 flops per ratio instead of 2 N d_in d_out,
// fewer whenever there are more calibration tokens than input channels.
//
// G is accumulated in float32 by the matrix cores from the bfloat16 activations (exact products)
// and both operands of the quadratic form are float16 (11-bit significands, against bfloat16's 8),
// each scaled by a power of two into float16's range: G by 2^gexp with its largest entry (on the
// diagonal, by Cauchy-Schwarz) at most 2^14, delta_k by 2^dexp[k] from a bound on |delta_k|. The
// scales are exact and removed exactly from each tile's float64 sum.
//
// Kernels here: the transpose of X into X^T (the GEMM wants both operands contiguous along the
// contraction, which for G is the token index), the choice of G's scale and its float16 form, and
// the per-ratio scale of delta. The GEMMs themselves are the error GEMM's (err_gemm.hip).
#include <stdint.h>

#include <algorithm>

#include "internal.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kTT = 64;  // transpose tile: 64 tokens x 64 channels

// X [n_tokens, ld_x] bf16 -> X^T [d_in, n_pad] bf16, zero for tokens >= n_tokens. A 64 x 64 tile
// through LDS: reads of 128 contiguous bytes of X rows, writes of 128 contiguous bytes of X^T rows.
__global__ __launch_bounds__(kThreads) void transpose_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                             int64_t n_tokens, int64_t d_in,
                                                             uint16_t* __restrict__ xt, int64_t n_pad) {
  __shared__ uint16_t t[kTT][kTT + 2];  // +2: the column reads of 8 rows fall in different banks
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kTT;  // channels
  const int64_t t0 = (int64_t)blockIdx.y * kTT;  // tokens
  // load: 64 token rows x 8 chunks of 8 channels; thread -> (row tid / 8 + 32 h, chunk tid % 8)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h, ch = tid & 7;
    const int64_t tok = t0 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (tok < n_tokens && c0 + 8 * ch < d_in) v = *reinterpret_cast<const uint4*>(x + tok * ld_x + c0 + 8 * ch);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t[r][8 * ch + 2 * q] = (uint16_t)(w[q] & 0xFFFFu);
      t[r][8 * ch + 2 * q + 1] = (uint16_t)(w[q] >> 16);
    }
  }
  __syncthreads();
  // store: 64 channel rows x 8 chunks of 8 tokens
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = (tid >> 3) + 32 * h, ch = tid & 7;
    if (c0 + c >= d_in) continue;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)t[8 * ch + 2 * q][c] | ((uint32_t)t[8 * ch + 2 * q + 1][c] << 16);
    *reinterpret_cast<uint4*>(xt + (c0 + c) * n_pad + t0 + 8 * ch) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// 14 - e for the smallest e with v < 2^e: a power-of-two scale that takes v to at most 2^14 (and
// float16's largest finite value is 65504 > 2^15). 0 for zero or a non-finite v.
__device__ __forceinline__ int32_t scale_exp(double v) {
  if (!(v > 0.0) || !(v <= 1.7976931348623157e308)) return 0;
  int e;
  (void)frexp(v, &e);  // v = m 2^e, 0.5 <= m < 1
  const int s = 14 - e;
  return s < -120 ? -120 : (s > 120 ? 120 : s);
}

// G's scale: its largest entry is on the diagonal (|G_ij| <= sqrt(G_ii G_jj)). One block.
__global__ __launch_bounds__(1024) void gram_exp_kernel(const float* __restrict__ g, int64_t d_in,
                                                        int32_t* __restrict__ gexp) {
  __shared__ float red[32];
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < d_in; i += blockDim.x) m = fmaxf(m, g[i * (d_in + 1)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) v = fmaxf(v, red[w]);
    // a NaN diagonal (non-finite activations) leaves the scale at 1; the loss is NaN either way
    gexp[0] = scale_exp((double)v);
  }
}

// float16(G * 2^gexp) in 64 x 64 blocks. The float32 G holds the 256-tiles on and above the diagonal;
// a block below them reads its mirror image (rows and columns swapped) and transposes it through LDS,
// so reads and writes are rows of 64 contiguous values either way.
__global__ __launch_bounds__(kThreads) void gram_f16_kernel(const float* __restrict__ g, int64_t d_in,
                                                            const int32_t* __restrict__ gexp,
                                                            uint16_t* __restrict__ g16) {
  __shared__ float t[kTT][kTT + 1];
  const float sc = ldexpf(1.f, gexp[0]);
  const int64_t i0 = (int64_t)blockIdx.y * kTT, j0 = (int64_t)blockIdx.x * kTT;
  const bool mirror = i0 / 256 > j0 / 256;  // below the stored tiles
  const int tid = threadIdx.x;
  // 64 rows x 16 float4; thread -> (row tid / 16 + 16 h, float4 tid % 16)
  const int64_t r0 = mirror ? j0 : i0, c0 = mirror ? i0 : j0;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int r = (tid >> 4) + 16 * h, q = tid & 15;
    const float4 v = *reinterpret_cast<const float4*>(g + (r0 + r) * d_in + c0 + 4 * q);
    if (mirror) {
      t[4 * q][r] = v.x; t[4 * q + 1][r] = v.y; t[4 * q + 2][r] = v.z; t[4 * q + 3][r] = v.w;
    } else {
      t[r][4 * q] = v.x; t[r][4 * q + 1] = v.y; t[r][4 * q + 2] = v.z; t[r][4 * q + 3] = v.w;
    }
  }
  __syncthreads();
  // 64 rows x 8 chunks of 8 halves; in a diagonal 256-block each float16 value is then multiplied
  // by 1/2 in float16 (exact in float16's normal range): the quadratic form's K loop takes G's
  // diagonal blocks halved and doubles each tile's sum, with no per-step scaling
  const _Float16 hm = i0 / 256 == j0 / 256 ? (_Float16)0.5f : (_Float16)1.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h, ch = tid & 7;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)((_Float16)(t[r][8 * ch + 2 * q] * sc) * hm)) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)((_Float16)(t[r][8 * ch + 2 * q + 1] * sc) * hm)) << 16);
    *reinterpret_cast<uint4*>(g16 + (i0 + r) * d_in + j0 + 8 * ch) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void set_u32_kernel(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

// max |w| over the stacked bf16 rows, as float bits (non-negative floats order as their bits; NaN
// compares above every finite value and infinity) into *slot: each block takes whole rows (row r,
// r + gridDim.x, ...), reduces in registers, across its waves in LDS, and then issues one atomic
__global__ __launch_bounds__(kThreads) void absmax_kernel(WParts w, int64_t d_in, int64_t d_out,
                                                          uint32_t* __restrict__ slot) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t n16 = d_in / 8;  // 16-byte words per row
  uint32_t m = 0u;
  for (int64_t r = blockIdx.x; r < d_out; r += gridDim.x) {
    int p = 0;
    while (r >= w.row_begin[p + 1]) ++p;
    const uint4* row = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w.ptr[p]) +
                                                      (r - w.row_begin[p]) * d_in);
    for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) {
      const uint4 v = row[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        m = max(m, (u[q] & 0x7FFFu) << 16);
        m = max(m, u[q] & 0x7FFF0000u);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
    atomicMax(slot, m);
  }
}

// The scale of ratio k's delta, from a bound on |delta| = |What - W| <= |What| + max|W|, with
// |What| <= (1.5 max|W| max(s_k) + b) / min(s_k) since |y| <= max|W| max(s_k):
// * group INT4: a reconstructed value is (q - zero) step / s, and the codes span the group's range to
//   within half a step, so |(q - zero) step| <= max|y| + step / 2 with step = max((max y - min y) /
//   15, 1e-8) <= max(2 max|y| / 15, 1e-8): at most 1.5 max|y| + 1e-8 (b = 1e-8);
// * row INT4: q = round(y / (step + 1e-6)), |q step| <= |y| + step / 2 <= (1 + 1/15) max|y| (b = 1e-8);
// * row INT8 symmetric: |q| <= 127 and step = max(max|y| / 127, 1e-8), |q step| <= max(max|y|, 1.27e-6)
//   (b = 1.27e-6).
// One block per ratio; dexp[n_cand] holds max|W| (absmax_kernel).
__global__ __launch_bounds__(kThreads) void delta_exp_kernel(const double* __restrict__ cand, int64_t d_in,
                                                             int n_cand, double b, int32_t* __restrict__ dexp) {
  __shared__ double rmx[kThreads / 64], rmn[kThreads / 64];
  const int k = blockIdx.x;
  const double* s = cand + (int64_t)k * d_in;
  double mx = 0.0, mn = 1.7976931348623157e308;
  for (int64_t c = threadIdx.x; c < d_in; c += blockDim.x) {
    mx = fmax(mx, s[c]);
    mn = fmin(mn, s[c]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmax(mx, __shfl_xor(mx, o, 64));
    mn = fmin(mn, __shfl_xor(mn, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    rmx[threadIdx.x >> 6] = mx;
    rmn[threadIdx.x >> 6] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) {
      mx = fmax(mx, rmx[w]);
      mn = fmin(mn, rmn[w]);
    }
    mx = fmax(mx, rmx[0]);
    mn = fmin(mn, rmn[0]);
    const double wmax = (double)__uint_as_float(reinterpret_cast<const uint32_t*>(dexp)[n_cand]);
    dexp[k] = scale_exp((1.5 * wmax * mx + b) / mn + wmax);
  }
}

__global__ void fill_f64_kernel(double* __restrict__ p, int64_t n, double v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

int64_t gram_n_pad(int64_t n_tokens) { return (n_tokens + kTT - 1) / kTT * kTT; }

hipError_t launch_gram(const void* x, int64_t ld_x, int64_t n_tokens, int64_t d_in, uint16_t* xt, float* g32,
                       uint16_t* g16, int32_t* gexp, hipStream_t st) {
  const int64_t n_pad = gram_n_pad(n_tokens);
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((d_in + kTT - 1) / kTT), (unsigned)(n_pad / kTT)),
                     dim3(kThreads), 0, st, static_cast<const uint16_t*>(x), ld_x, n_tokens, d_in, xt, n_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gram_store(xt, n_pad, d_in, g32, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gram_exp_kernel, dim3(1), dim3(1024), 0, st, g32, d_in, gexp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned nb = (unsigned)(d_in / kTT);  // d_in is a multiple of 128
  hipLaunchKernelGGL(gram_f16_kernel, dim3(nb, nb), dim3(kThreads), 0, st, g32, d_in, gexp, g16);
  return hipGetLastError();
}

hipError_t launch_delta_exp(const WParts& w, int64_t d_in, const double* cand_scales, int n_cand, double b,
                            int32_t* dexp, hipStream_t st) {
  const int64_t d_out = w.row_begin[w.n];
  uint32_t* slot = reinterpret_cast<uint32_t*>(dexp + n_cand);
  hipLaunchKernelGGL(set_u32_kernel, dim3(1), dim3(64), 0, st, slot, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)std::min<int64_t>(d_out, 1024)), dim3(kThreads), 0, st, w, d_in,
                     d_out, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(delta_exp_kernel, dim3((unsigned)n_cand), dim3(kThreads), 0, st, cand_scales, d_in, n_cand, b,
                     dexp);
  return hipGetLastError();
}

hipError_t launch_fill_f64(double* p, int64_t n, double v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f64_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, p, n,
                     v);
  return hipGetLastError();
}

}  // namespace awq
