// a1: per-input-channel mean of |X| over the calibration tokens
// (bjdmk.com.cn AWQ article, section "显著权重的识别", S_X(i) = (1/N) sum_j |X_{j,i}|;
//  msModelSlim "AWQ：激活感知权重量化算法说明", 原理 / 算法公式, act_mean = mean(abs(act))).
//
// HBM-bound column reduction. Each lane owns 16 bytes of a row (8 bf16 or 4 f32 channels);
// `lanes_per_row` lanes cover a row slice, so a wave reads 64/lanes_per_row rows per load
// instruction and the block's four waves read consecutive rows. Every lane accumulates in
// float64 (exact for the magnitudes of bf16 inputs, no drift over 65536 tokens); row slots of
// a wave are folded with cross-lane shuffles, the four waves through LDS, and each row chunk
// writes one float64 partial per channel. A second kernel adds the partials in chunk order
// and divides by n_tokens, so the result does not depend on scheduling.
#include "internal.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int LC>
__global__ __launch_bounds__(kThreads) void act_stats_partial_kernel(
    const T* __restrict__ x, int64_t ld, int64_t n_tokens, int64_t d_in, int64_t rows_per_chunk,
    double* __restrict__ partial) {
  constexpr int VEC = 16 / sizeof(T);  // channels per lane
  constexpr int RW = 64 / LC;          // row slots per wave
  constexpr int RB = RW * (kThreads / 64);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cl = lane % LC;
  const int rs = lane / LC;
  const int64_t col = (int64_t)blockIdx.x * (LC * VEC) + cl * VEC;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r_end = min(n_tokens, r_begin + rows_per_chunk);

  double acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.0;

  auto add = [&](const u32x4& u) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += (double)fabsf(bf16_to_f32(w[j] & 0xFFFFu));
        acc[2 * j + 1] += (double)fabsf(bf16_to_f32(w[j] >> 16));
      }
    } else {
      acc[0] += (double)fabsf(__uint_as_float(u.x));
      acc[1] += (double)fabsf(__uint_as_float(u.y));
      acc[2] += (double)fabsf(__uint_as_float(u.z));
      acc[3] += (double)fabsf(__uint_as_float(u.w));
    }
  };

  const T* base = x + col;
  int64_t r = r_begin + wave * RW + rs;
  for (; r + (kUnroll - 1) * RB < r_end; r += kUnroll * RB) {
    u32x4 u[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      u[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (r + i * RB) * ld));
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) add(u[i]);
  }
  for (; r < r_end; r += RB) add(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + r * ld)));

  // fold the row slots of the wave (lanes that share cl)
#pragma unroll
  for (int m = LC; m < 64; m <<= 1) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] += __shfl_xor(acc[j], m, 64);
  }

  __shared__ double red[kThreads / 64][LC * VEC];
  if (rs == 0) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) red[wave][cl * VEC + j] = acc[j];
  }
  __syncthreads();
  double* out = partial + (int64_t)blockIdx.y * d_in + (int64_t)blockIdx.x * (LC * VEC);
  for (int i = threadIdx.x; i < LC * VEC; i += kThreads) {
    double s = red[0][i];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) s += red[w][i];
    out[i] = s;
  }
}

// One block per 64 channels: wave w adds the chunks w, w+4, w+8, ... of its lane's channel
// (independent loads, eight in flight), then the four waves are added in order.
// With `accumulate`, out[c] += sum (a running sum over calibration batches); otherwise
// out[c] = sum / n_tokens.
__global__ __launch_bounds__(kThreads) void act_stats_finalize_kernel(
    const double* __restrict__ partial, int64_t n_chunks, int64_t d_in, int64_t n_tokens,
    double* __restrict__ act_mean, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  double s = 0.0;
  if (c < d_in) {
    int64_t k = wave;
    for (; k + 28 < n_chunks; k += 32) {
      double v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = partial[(k + 4 * i) * d_in + c];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; k < n_chunks; k += 4) s += partial[k * d_in + c];
  }
  __shared__ double red[kThreads / 64][64];
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && c < d_in) {
    const double t = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    act_mean[c] = accumulate ? act_mean[c] + t : t / (double)n_tokens;
  }
}

__global__ __launch_bounds__(kThreads) void act_mean_from_sums_kernel(const double* sums, int64_t d_in,
                                                                       int64_t total_tokens, double* act_mean) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c < d_in) act_mean[c] = sums[c] / (double)total_tokens;
}

template <typename T, int LC>
hipError_t launch_partial(const void* x, int64_t ld, int64_t n, int64_t d_in, double* partial,
                          const ActStatsPlan& p, hipStream_t st) {
  dim3 grid((unsigned)p.col_blocks, (unsigned)p.row_chunks);
  hipLaunchKernelGGL((act_stats_partial_kernel<T, LC>), grid, dim3(kThreads), 0, st,
                     static_cast<const T*>(x), ld, n, d_in, p.rows_per_chunk, partial);
  return hipGetLastError();
}

}  // namespace

namespace {

ActStatsPlan plan_with(int lanes_per_row, int vec, int64_t n_tokens, int64_t d_in) {
  ActStatsPlan p{};
  p.lanes_per_row = lanes_per_row;
  p.col_blocks = d_in / (p.lanes_per_row * vec);
  const int64_t rows_per_iter = (64 / p.lanes_per_row) * (kThreads / 64);
  // At most 1024 blocks (4 per CU, all resident at once: a second, partial round of blocks
  // would leave a tail), every block >= 64 rows. Measured on the 7B/70B activation shapes,
  // this beats 2048 or 4096 blocks and 256-byte or 1 KB slices.
  const int64_t min_rows = rows_per_iter * kUnroll > 64 ? rows_per_iter * kUnroll : 64;
  const int64_t max_chunks = (n_tokens + min_rows - 1) / min_rows;
  int64_t chunks = 1024 / p.col_blocks;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  int64_t rpc = (n_tokens + chunks - 1) / chunks;
  rpc = (rpc + rows_per_iter - 1) / rows_per_iter * rows_per_iter;
  if (rpc < 1) rpc = rows_per_iter;
  p.rows_per_chunk = rpc;
  p.row_chunks = (n_tokens + rpc - 1) / rpc;
  if (p.row_chunks < 1) p.row_chunks = 1;
  return p;
}

}  // namespace

ActStatsPlan act_stats_plan(int dtype, int64_t n_tokens, int64_t d_in) {
  const int vec = dtype == 1 ? 8 : 4;
  const int64_t vec_lanes = d_in / vec;
  // 512-byte row slices (two rows per wave load); 256 bytes when d_in only divides that way, or
  // when blocks would get fewer than 128 rows (a short input: narrower slices give twice the blocks
  // along d_in and half the row chunks; 4096 x 4096 bf16 measured 15 -> 13 us)
  if (vec_lanes % 32 == 0) {
    const ActStatsPlan p = plan_with(32, vec, n_tokens, d_in);
    if (p.rows_per_chunk >= 128) return p;
  }
  return plan_with(16, vec, n_tokens, d_in);
}

hipError_t launch_act_stats(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                            double* act_mean, double* partial, const ActStatsPlan& p,
                            hipStream_t st, bool accumulate) {
  hipError_t e;
  if (dtype == 1) {
    e = p.lanes_per_row == 32 ? launch_partial<uint16_t, 32>(x, ld_x, n_tokens, d_in, partial, p, st)
                              : launch_partial<uint16_t, 16>(x, ld_x, n_tokens, d_in, partial, p, st);
  } else {
    e = p.lanes_per_row == 32 ? launch_partial<float, 32>(x, ld_x, n_tokens, d_in, partial, p, st)
                              : launch_partial<float, 16>(x, ld_x, n_tokens, d_in, partial, p, st);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(act_stats_finalize_kernel, dim3((unsigned)((d_in + 63) / 64)),
                     dim3(kThreads), 0, st, partial, p.row_chunks, d_in, n_tokens, act_mean, accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_act_mean_from_sums(const double* sums, int64_t d_in, int64_t total_tokens, double* act_mean,
                                     hipStream_t st) {
  hipLaunchKernelGGL(act_mean_from_sums_kernel, dim3((unsigned)((d_in + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, st, sums, d_in, total_tokens, act_mean);
  return hipGetLastError();
}

}  // namespace awq
