// The inference consumer of the export: Y = X * W_hat^T with W_hat dequantized on the fly from the
// deployment form (4-bit codes two per byte, float16 per-group steps, 4-bit zero points), as the
// bjdmk.com.cn AWQ article describes in "GPU 硬件级反量化算子内联融合": wide loads of the packed
// weights, low/high 4-bit unpack, conversion and per-group scale/offset, then the matrix units,
// without ever writing 16-bit weights to memory.
//
// Dequantization (qqiyuan.cn "基于awq 4-bit量化技术的大模型推理优化实战", dequantize): a code q of
// group g of row o gives (q - zero[o, g]) * step[o, g]. With the float16 step that product is exact
// in float32 (a 5-bit integer times an 11-bit mantissa), formed as fma(q, step, -zero * step), and is
// rounded once, to nearest even, to the activations' type (bfloat16 or float16), which both matrix
// operands share. Products are accumulated in float32 by v_mfma_f32_16x16x32_{bf16,f16}.
//
// Operand layout of the 16x16x32 instruction: lane l supplies row (l mod 16) of A (a token) and
// column (l mod 16) of B (an output row), each with 8 consecutive k of the lane group l / 16. Any
// assignment of the contraction index to (lane group, element) works as long as A and B use the same
// one; here lane group kq of sub-step t of a 128-wide group holds k = 32 kq + 8 t + e, so that a lane's
// codes for a whole group are one 16-byte load (32 nibbles) and its activations 64 contiguous bytes.
#include "w4a16.h"
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;          // small-M kernel: groups whose codes a wave loads at once
constexpr int kBigTokens = 128;    // large-M kernel: tokens per block (8 tiles of 16)
constexpr int kBigRowsPerWave = 64;  // 4 tiles of 16 output rows per wave
constexpr int kBigRows = 4 * kBigRowsPerWave;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b, int kind) {
  if (kind == 0) return pack_bf16x2(a, b);
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// 8 codes (one dword, element e in bits 4e..4e+3) -> 8 operands, two per register.
template <int KIND>
__device__ __forceinline__ uint4 dequant8(uint32_t w, float st, float nzs) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fmaf((float)((w >> (4 * e)) & 15u), st, nzs);
  return make_uint4(pack2(v[0], v[1], KIND), pack2(v[2], v[3], KIND), pack2(v[4], v[5], KIND),
                    pack2(v[6], v[7], KIND));
}

template <int KIND>
__device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, const f32x4& c) {
  if constexpr (KIND == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
}

template <typename OutT>
__device__ __forceinline__ OutT to_out(float v, int kind);
template <>
__device__ __forceinline__ float to_out<float>(float v, int) { return v; }
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float v, int kind) {
  return (uint16_t)(pack2(v, 0.f, kind) & 0xFFFFu);
}

// The step and the negated offset of group g of a row.
__device__ __forceinline__ void group_params(const uint16_t* srow, const uint8_t* zrow, int g, float& st,
                                             float& nzs) {
  const float s = (float)__builtin_bit_cast(_Float16, srow[g]);
  const int z = (zrow[g >> 1] >> ((g & 1) * 4)) & 15;
  st = s;
  nzs = -(float)z * s;  // exact: 4-bit integer times an 11-bit mantissa
}

// Few tokens (decode): a block computes 16 tokens x 16 output rows; its four waves take four
// contiguous ranges of the groups and their partial products are added in wave order. The
// weights, read once per 16 tokens, dominate the traffic: each wave has the codes of up to
// kBatch groups in flight before it starts on them.
template <int KIND, typename OutT>
__global__ __launch_bounds__(kThreads) void w4a16_small_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                              const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ steps,
                                                              const uint8_t* __restrict__ zeros, int n_tokens,
                                                              int d_in, int d_out, OutT* __restrict__ y,
                                                              int64_t ld_y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int row = blockIdx.x * 16 + n;
  const int tok = blockIdx.y * 16 + n;
  const int G = d_in / kGroup, GZ = (G + 1) / 2;
  const bool row_ok = row < d_out, tok_ok = tok < n_tokens;
  const int g_begin = (G * wave) / 4, g_end = (G * (wave + 1)) / 4;
  const uint8_t* crow = codes + (int64_t)row * (d_in / 2) + kq * 16;
  const uint16_t* srow = steps + (int64_t)row * G;
  const uint8_t* zrow = zeros + (int64_t)row * GZ;
  const uint16_t* xrow = x + (int64_t)tok * ld_x + kq * 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int gb = g_begin; gb < g_end; gb += kBatch) {
    const int nb = min(kBatch, g_end - gb);
    uint4 cw[kBatch];
    float st[kBatch], nzs[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      cw[i] = make_uint4(0, 0, 0, 0);
      st[i] = 0.f;
      nzs[i] = 0.f;
      if (i < nb && row_ok) {
        cw[i] = *reinterpret_cast<const uint4*>(crow + (int64_t)(gb + i) * (kGroup / 2));
        group_params(srow, zrow, gb + i, st[i], nzs[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < nb) {
        uint4 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          a[t] = tok_ok ? *reinterpret_cast<const uint4*>(xrow + (gb + i) * kGroup + t * 8) : make_uint4(0, 0, 0, 0);
        const uint32_t wt[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = mma<KIND>(a[t], dequant8<KIND>(wt[t], st[i], nzs[i]), acc);
      }
    }
  }
  __shared__ f32x4 red[4][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4 s = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    // C layout of the 16x16 result: lane l holds rows 4 (l / 16) .. +3 of column l mod 16
    const int orow = blockIdx.x * 16 + (lane & 15);
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t2 = blockIdx.y * 16 + 4 * (lane >> 4) + i;
      if (orow < d_out && t2 < n_tokens) y[(int64_t)t2 * ld_y + orow] = to_out<OutT>(sv[i], KIND);
    }
  }
}

// Many tokens (prefill): a block computes 128 tokens x 256 output rows, each wave 128 tokens x 64
// rows. Per group the block stages the 128 x 128 activations in LDS (16-byte chunks of a token row
// XOR-swizzled by the token, so that the 16 lanes of a read phase hit distinct banks) and every
// wave dequantizes its own rows' codes in registers. The next group's activations and codes are
// loaded while the current one is multiplied.
template <int KIND, typename OutT>
__global__ __launch_bounds__(kThreads) void w4a16_big_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                            const uint8_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ steps,
                                                            const uint8_t* __restrict__ zeros, int n_tokens,
                                                            int d_in, int d_out, OutT* __restrict__ y,
                                                            int64_t ld_y) {
  __shared__ __attribute__((aligned(16))) uint4 xs[2][kBigTokens * 16];  // 2 x 32 KiB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int G = d_in / kGroup, GZ = (G + 1) / 2;
  const int tok0 = blockIdx.y * kBigTokens;
  const int row0 = blockIdx.x * kBigRows + wave * kBigRowsPerWave;

  // activations: thread t moves chunks t, t + 256, ... (token = chunk / 16, 16-byte piece = chunk % 16)
  uint4 xa[8];
  auto load_x = [&](int g) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = threadIdx.x + kThreads * j;
      const int tk = tok0 + (c >> 4);
      xa[j] = tk < n_tokens ? *reinterpret_cast<const uint4*>(x + (int64_t)tk * ld_x + g * kGroup + (c & 15) * 8)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = threadIdx.x + kThreads * j;
      const int tr = c >> 4;
      xs[buf][tr * 16 + ((c & 15) ^ (tr & 15))] = xa[j];
    }
  };
  // codes of the wave's 4 row tiles: lane (n, kq) holds 32 codes of row row0 + 16 j + n
  uint4 cw[4];
  float st[4], nzs[4];
  auto load_w = [&](int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + 16 * j + n;
      cw[j] = make_uint4(0, 0, 0, 0);
      st[j] = 0.f;
      nzs[j] = 0.f;
      if (r < d_out) {
        cw[j] = *reinterpret_cast<const uint4*>(codes + (int64_t)r * (d_in / 2) + g * (kGroup / 2) + kq * 16);
        group_params(steps + (int64_t)r * G, zeros + (int64_t)r * GZ, g, st[j], nzs[j]);
      }
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_x(0);
  load_w(0);
  store_x(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const uint4 cur[4] = {cw[0], cw[1], cw[2], cw[3]};
    const float cst[4] = {st[0], st[1], st[2], st[3]};
    const float cnz[4] = {nzs[0], nzs[1], nzs[2], nzs[3]};
    if (g + 1 < G) {
      load_x(g + 1);
      load_w(g + 1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wj[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
        b[j] = dequant8<KIND>(wj[t], cst[j], cnz[j]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int tr = 16 * m + n;
        const uint4 a = xs[buf][tr * 16 + ((4 * kq + t) ^ (tr & 15))];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = mma<KIND>(a, b[j], acc[m][j]);
      }
    }
    if (g + 1 < G) store_x(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int orow = row0 + 16 * j + (lane & 15);
      const float sv[4] = {acc[m][j].x, acc[m][j].y, acc[m][j].z, acc[m][j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t2 = tok0 + 16 * m + 4 * (lane >> 4) + i;
        if (orow < d_out && t2 < n_tokens) y[(int64_t)t2 * ld_y + orow] = to_out<OutT>(sv[i], KIND);
      }
    }
  }
}

template <int KIND, typename OutT>
hipError_t launch_kind(const void* x, int64_t ld_x, const uint8_t* codes, const uint16_t* steps,
                       const uint8_t* zeros, int n_tokens, int d_in, int d_out, void* y, int64_t ld_y, bool big,
                       hipStream_t st) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  OutT* yp = static_cast<OutT*>(y);
  if (big) {
    const dim3 grid((unsigned)((d_out + kBigRows - 1) / kBigRows), (unsigned)((n_tokens + kBigTokens - 1) / kBigTokens));
    hipLaunchKernelGGL((w4a16_big_kernel<KIND, OutT>), grid, dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros,
                       n_tokens, d_in, d_out, yp, ld_y);
  } else {
    const dim3 grid((unsigned)((d_out + 15) / 16), (unsigned)((n_tokens + 15) / 16));
    hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT>), grid, dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros,
                       n_tokens, d_in, d_out, yp, ld_y);
  }
  return hipGetLastError();
}

}  // namespace

bool w4a16_uses_big_kernel(int64_t n_tokens) { return n_tokens > kW4a16SmallMaxTokens; }

hipError_t launch_w4a16_gemm(const void* x, int64_t ld_x, int kind, const uint8_t* codes, const uint16_t* steps_f16,
                             const uint8_t* zeros_u4, int64_t n_tokens, int64_t d_in, int64_t d_out, void* y,
                             int64_t ld_y, bool y_f32, hipStream_t st) {
  const bool big = w4a16_uses_big_kernel(n_tokens);
  const int nt = (int)n_tokens, di = (int)d_in, dout = (int)d_out;
  if (kind == 0)
    return y_f32 ? launch_kind<0, float>(x, ld_x, codes, steps_f16, zeros_u4, nt, di, dout, y, ld_y, big, st)
                 : launch_kind<0, uint16_t>(x, ld_x, codes, steps_f16, zeros_u4, nt, di, dout, y, ld_y, big, st);
  return y_f32 ? launch_kind<1, float>(x, ld_x, codes, steps_f16, zeros_u4, nt, di, dout, y, ld_y, big, st)
               : launch_kind<1, uint16_t>(x, ld_x, codes, steps_f16, zeros_u4, nt, di, dout, y, ld_y, big, st);
}

}  // namespace awq
