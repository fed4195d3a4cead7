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
#include <type_traits>

#include "w4a16.h"
#include "device_common.h"
#include "lds_dma.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 2;   // small-M kernel: groups whose codes a wave loads at once
constexpr int kXSub = 2;    // small-M kernel: groups whose activations are loaded at once
constexpr int kSmallWaves = 8;  // small-M kernel: waves per block, each 1/8 of the groups (a 4096-input
                                // layer's codes then fit one batch per wave)
// small-M kernel: layers with at least this many rows take two 16-row tiles per wave (each
// activation fragment then feeds both, halving the activation loads, whose scattered cache lines
// limit the kernel at 16 tokens); smaller layers take one, which keeps at least 256 blocks
constexpr int kSmallWideRows = 8192;
constexpr int kBigTokens = 128;    // large-M kernel: tokens per block (8 tiles of 16)
// many-token kernel: NJ tiles of 16 output rows per wave (4 for prefill; 1 for a few hundred tokens,
// where 4 would leave too few blocks to fill the chip)
constexpr int kBigNJ = 4, kMidNJ = 1;
constexpr int64_t kMidMaxTokens = 512;

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

// The step and the negated offset of a group from its raw float16 step and zero-point byte.
__device__ __forceinline__ void group_params(uint32_t step_bits, uint32_t zbyte, int g, float& st, float& nzs) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)step_bits);
  const int z = (zbyte >> ((g & 1) * 4)) & 15;
  st = s;
  nzs = -(float)z * s;  // exact: 4-bit integer times an 11-bit mantissa
}

// Few tokens (decode): a block computes 16 MT tokens x 16 NT output rows (MT = 2 for 17-32 tokens,
// so that each dequantized weight fragment feeds both token tiles and the weights are read once);
// its eight waves take eight contiguous ranges of the groups and their partial products are added
// in wave order. The weights dominate the HBM traffic; each activation fragment is used for NT row
// tiles, which divides the activations' re-reads from L2. Loads are unconditional
// (rows and tokens past the end read the last valid one, whose results are never stored) so that a
// batch's loads all go out back to back; the codes of the next batch are in flight while the
// current one is multiplied.
template <int KIND, typename OutT, int NT, int MT>
__global__ __launch_bounds__(64 * kSmallWaves) void w4a16_small_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                              const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ steps,
                                                              const uint8_t* __restrict__ zeros, int n_tokens,
                                                              int d_in, int d_out, OutT* __restrict__ y,
                                                              int64_t ld_y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int G = d_in / kGroup, GZ = (G + 1) / 2;
  const int g_begin = (G * wave) / kSmallWaves, g_end = (G * (wave + 1)) / kSmallWaves;
  const uint8_t* crow[NT];
  const uint16_t* srow[NT];
  const uint8_t* zrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int row = min(blockIdx.x * (16 * NT) + 16 * j + n, d_out - 1);
    crow[j] = codes + (int64_t)row * (d_in / 2) + kq * 16;
    srow[j] = steps + (int64_t)row * G;
    zrow[j] = zeros + (int64_t)row * GZ;
  }
  const uint16_t* xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xrow[m] = x + (int64_t)min(blockIdx.y * (16 * MT) + 16 * m + n, n_tokens - 1) * ld_x + kq * 32;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 cw[kBatch][NT];
  uint32_t sr[kBatch][NT], zr[kBatch][NT];
  auto load_w = [&](int gb) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int g = min(gb + i, g_end - 1);  // a short last batch re-reads its last group (unused)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        cw[i][j] = *reinterpret_cast<const uint4*>(crow[j] + (int64_t)g * (kGroup / 2));
        sr[i][j] = srow[j][g];
        zr[i][j] = zrow[j][g >> 1];
      }
    }
  };
  if (g_begin < g_end) load_w(g_begin);
  for (int gb = g_begin; gb < g_end; gb += kBatch) {
    uint4 cur[kBatch][NT];
    float st[kBatch][NT], nzs[kBatch][NT];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        cur[i][j] = cw[i][j];
        group_params(sr[i][j], zr[i][j], gb + i, st[i][j], nzs[i][j]);
      }
    if (gb + kBatch < g_end) load_w(gb + kBatch);
#pragma unroll
    for (int h = 0; h < kBatch; h += kXSub) {
      if (gb + h < g_end) {  // wave-uniform
        uint4 a[MT][kXSub][4];
#pragma unroll
        for (int i = 0; i < kXSub; ++i) {
          const int g = min(gb + h + i, g_end - 1);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t) a[m][i][t] = *reinterpret_cast<const uint4*>(xrow[m] + g * kGroup + t * 8);
        }
#pragma unroll
        for (int i = 0; i < kXSub; ++i) {
          if (gb + h + i < g_end) {  // wave-uniform
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const uint32_t wt[4] = {cur[h + i][j].x, cur[h + i][j].y, cur[h + i][j].z, cur[h + i][j].w};
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const uint4 b = dequant8<KIND>(wt[t], st[h + i][j], nzs[h + i][j]);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m][j] = mma<KIND>(a[m][i][t], b, acc[m][j]);
              }
            }
          }
        }
      }
    }
  }
  __shared__ f32x4 red[kSmallWaves][MT * NT][64];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][m * NT + j][lane] = acc[m][j];
  __syncthreads();
  if (wave < MT * NT) {  // wave m NT + j adds the partials of token tile m, row tile j
    const int m = wave / NT, j = wave % NT;
    f32x4 s = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) s += red[w][wave][lane];
    // C layout of the 16x16 result: lane l holds rows 4 (l / 16) .. +3 of column l mod 16
    const int orow = blockIdx.x * (16 * NT) + 16 * j + (lane & 15);
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t2 = blockIdx.y * (16 * MT) + 16 * m + 4 * (lane >> 4) + i;
      if (orow < d_out && t2 < n_tokens) y[(int64_t)t2 * ld_y + orow] = to_out<OutT>(sv[i], KIND);
    }
  }
}

// One token (decode): the weights stream through in contiguous 1 KiB windows, one output row at a
// time per wave. Lane l of a window holds the row's codes 32 l .. 32 l + 31 (one 16-byte load, all in
// group l / 4 of the window's 16), so each wave load reads 1 KiB of consecutive bytes. The token's
// activations sit in LDS, chunk t (8 values) of lane l's 32 at t KiB + 16 l of the window's 4 KiB, so
// that the four reads of a window are conflict-free. Products use v_mfma_f32_16x16x32 with the lane's
// activations as A and its dequantized weights as B: the diagonal C[i][i] collects the products of
// the lanes i, i + 16, i + 32, i + 48, so the sum of the diagonal over all windows is the row's dot
// product (the off-diagonal entries are discarded). Dequantization per 8 codes: (q, q') pairs of
// nibbles e and e + 4 are placed in the mantissas of two float16 values 1024 + q (one and-or), and
// fma(1024 + q, step, -(1024 + zero) * step) = (q - zero) * step exactly in float32 (both products
// need at most 22 bits), rounded once to the operand type: the same values the other kernels form.
constexpr int kGemvWaves = 8;
constexpr int kGemvDepth = 8;         // windows in flight per wave
constexpr int kGemvMaxIn = 32768;     // the LDS copy of the activations (64 KiB)
constexpr int kGemvBlocks = 512;      // two blocks per compute unit

// (h & mask) | magic in one instruction: VOP3 takes no literal operand on this architecture, so the
// mask comes in a scalar register and the float16 exponent pattern in a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t h, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(h), "s"(mask), "v"(magic));
  return r;
}

// Per-lane constants of a group: fma(1024 + q, st, c0) and fma(1024 + 16 q, st16, c16) both give
// (q - zero) * step exactly.
struct MixParams {
  float st, c0, st16, c16;
};

template <int KIND>
__device__ __forceinline__ uint4 dequant8_mix(uint32_t w, const MixParams& p, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const f16x2_t h0 = __builtin_bit_cast(f16x2_t, and_or(w, 0x000F000Fu, magic));   // nibbles 0, 4
  const f16x2_t h1 = __builtin_bit_cast(f16x2_t, and_or(w, 0x00F000F0u, magic));   // 1, 5 (times 16)
  const f16x2_t h2 = __builtin_bit_cast(f16x2_t, and_or(w8, 0x000F000Fu, magic));  // 2, 6
  const f16x2_t h3 = __builtin_bit_cast(f16x2_t, and_or(w8, 0x00F000F0u, magic));  // 3, 7 (times 16)
  const float v0 = fmaf((float)h0.x, p.st, p.c0), v4 = fmaf((float)h0.y, p.st, p.c0);
  const float v1 = fmaf((float)h1.x, p.st16, p.c16), v5 = fmaf((float)h1.y, p.st16, p.c16);
  const float v2 = fmaf((float)h2.x, p.st, p.c0), v6 = fmaf((float)h2.y, p.st, p.c0);
  const float v3 = fmaf((float)h3.x, p.st16, p.c16), v7 = fmaf((float)h3.y, p.st16, p.c16);
  return make_uint4(pack2(v0, v1, KIND), pack2(v2, v3, KIND), pack2(v4, v5, KIND), pack2(v6, v7, KIND));
}

template <int KIND, typename OutT>
__global__ __launch_bounds__(64 * kGemvWaves) void w4a16_gemv_kernel(const uint16_t* __restrict__ x,
                                                                     const uint8_t* __restrict__ codes,
                                                                     const uint16_t* __restrict__ steps,
                                                                     const uint8_t* __restrict__ zeros, int d_in,
                                                                     int d_out, int rows_per_wave,
                                                                     OutT* __restrict__ y) {
  extern __shared__ uint4 xs[];  // windows x 4 KiB
  constexpr int D = kGemvDepth;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = d_in / kGroup, GZ = (G + 1) / 2, W = (G + 15) / 16;
  // 64-bit until clamped: near the largest d_out the last wave's row range ends past 2^31
  const int64_t r0l = ((int64_t)blockIdx.x * kGemvWaves + wave) * rows_per_wave;
  const int r0 = (int)min(r0l, (int64_t)d_out);
  const int r1 = (int)min(r0l + rows_per_wave, (int64_t)d_out);
  const int n_items = r1 > r0 ? (r1 - r0) * W : 0;
  const int lg = lane >> 2;  // the lane's group within a window

  uint4 cw[D];
  // the narrow loads stay in their own types: a zero extension at the loop's back edge would wait for
  // every load in flight
  uint16_t sr[D];
  uint8_t zr[D];
  int lrow = r0, lwin = 0, lcount = 0;  // next item to load
  // items past the wave's last re-load its last one (the same cache lines; never used); a wave
  // without rows has r1 = d_out and re-reads the last row
  auto load_item = [&](int u) {
    const bool in = lcount < n_items;
    const int64_t o = in ? lrow : r1 - 1;
    const int g = min((in ? lwin : W - 1) * 16 + lg, G - 1);  // lanes past the row's last group re-read it
    cw[u] = *reinterpret_cast<const uint4*>(codes + o * (d_in / 2) + (int64_t)g * (kGroup / 2) + (lane & 3) * 16);
    sr[u] = steps[o * G + g];
    zr[u] = zeros[o * GZ + (g >> 1)];
    ++lcount;
    if (++lwin == W) lwin = 0, ++lrow;
    // keep the slots' loads in slot order, as the waits assume
    __builtin_amdgcn_sched_barrier(0);
  };

  // the activations into LDS, window by window, chunk c of a window (8 values, c = 4 l + t) at
  // t KiB + 16 l, past d_in zeros. Their loads go out first, then the ring's first loads, so that the
  // stores wait only for the activations.
  {
    constexpr int kIters = kGemvMaxIn / 8 / (64 * kGemvWaves);
    uint4 v[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {  // every load issued before the first store
      const int c = threadIdx.x + i * 64 * kGemvWaves;
      v[i] = make_uint4(0, 0, 0, 0);
      if (c * 8 < d_in) v[i] = *reinterpret_cast<const uint4*>(x + (int64_t)c * 8);
    }
    // unconditional, so that the count of loads in flight is the same in every wave
#pragma unroll
    for (int u = 0; u < D; ++u) load_item(u);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int c = threadIdx.x + i * 64 * kGemvWaves, cc = c & 255;
      if (c < W * 256) xs[(c >> 8) * 256 + (cc & 3) * 64 + (cc >> 2)] = v[i];
    }
  }
  __syncthreads();

  const uint32_t magic = 0x64006400u;  // float16 1024 in both halves
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int crow = r0, cwin = 0;  // next item to consume
  auto consume = [&](int u) {
    const int g = cwin * 16 + lg;
    const float s = (float)__builtin_bit_cast(_Float16, sr[u]);
    const int z = __builtin_amdgcn_ubfe(zr[u], (lg & 1) * 4, 4);
    MixParams p;
    p.st = s;
    p.c0 = -(float)(1024 + z) * s;  // exact: 11-bit integer times an 11-bit mantissa
    p.st16 = s * 0.0625f;
    p.c16 = -(float)(64 + z) * s;
    if (g >= G) p.st = p.c0 = p.st16 = p.c16 = 0.f;  // past the row's end: weight 0 (the LDS holds zeros there)
    const uint4* xw = xs + cwin * 256 + lane;
    const uint32_t wt[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = mma<KIND>(xw[64 * t], dequant8_mix<KIND>(wt[t], p, magic), acc);
    if (++cwin == W) {
      // the diagonal: lane l holds C[4 (l / 16) + i][l mod 16] in acc[i]
      const int i = (lane & 15) - 4 * (lane >> 4);
      float d = (i == 0) ? acc.x : (i == 1) ? acc.y : (i == 2) ? acc.z : (i == 3) ? acc.w : 0.f;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) d += __shfl_xor(d, m);
      if (lane == 0) y[crow] = to_out<OutT>(d, KIND);
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      cwin = 0;
      ++crow;
    }
  };
  // a slot is consumed, then refilled with the item D places later; the loads are unconditional so
  // that every wait counts a fixed number of loads in flight, except in the last round, which loads
  // nothing
  for (int base = 0; base < n_items; base += D) {
    if (base + D < n_items) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (base + u < n_items) consume(u);  // wave-uniform
        load_item(u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < D; ++u)
        if (base + u < n_items) consume(u);
    }
  }
}

// Many tokens (prefill): a block computes 128 tokens x 64 NJ output rows, each wave 128 tokens x
// 16 NJ rows (NJ = 4 for prefill, 1 up to a few hundred tokens). Per group the block's activations (128 tokens x 128 inputs, 32 KiB) go global -> LDS by
// DMA, 16-byte chunks of a token row XOR-swizzled by the token so that the 16 lanes of a fragment
// read hit distinct banks; tokens past the end lie outside the buffer range and read as zero. Every
// wave dequantizes its own rows' codes in registers. The next group's activations and codes are in
// flight while the current group is multiplied (two LDS stages, two register sets of codes).
template <int KIND, typename OutT, int NJ>
__global__ __launch_bounds__(kThreads, 2) void w4a16_big_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                               const uint8_t* __restrict__ codes,
                                                               const uint16_t* __restrict__ steps,
                                                               const uint8_t* __restrict__ zeros, int n_tokens,
                                                               int d_in, int d_out, OutT* __restrict__ y,
                                                               int64_t ld_y) {
  __shared__ __attribute__((aligned(1024))) uint4 xs[2][kBigTokens * 16];  // 2 x 32 KiB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int G = d_in / kGroup, GZ = (G + 1) / 2;
  const int tok0 = blockIdx.y * kBigTokens;
  constexpr int kRowsPerWave = 16 * NJ;
  const int row0 = blockIdx.x * (4 * kRowsPerWave) + wave * kRowsPerWave;

  // activations: wave w fills LDS chunks p = 512 w + 64 j + lane (token p / 16, slot p % 16) with
  // the global chunk (p % 16) ^ (token % 16) of that token's 256-byte group slice. The buffer range
  // check covers the per-lane offset only, not the scalar one, so the token's row offset is in the
  // per-lane offset (a token past the end then reads zero) and the scalar offset holds only the group's
  // position inside the row (g * 256 + 16 <= d_in * 2 <= ld_x * 2, so a valid token stays in its row).
  const int valid_tok = min(kBigTokens, n_tokens - tok0);
  const i32x4 xr = make_rsrc(x + (int64_t)tok0 * ld_x, (uint32_t)valid_tok * (uint32_t)ld_x * 2u);
  int xoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tr = 32 * wave + 16 * (j >> 2) + 4 * (j & 3) + (lane >> 4);
    xoff[j] = tr * (int)ld_x * 2 + (((lane & 15) ^ (tr & 15)) * 16);
  }
  auto load_x = [&](int g, int buf) {
    const uint32_t base = lds_address(&xs[buf][512 * wave]);
#pragma unroll
    for (int j = 0; j < 8; ++j) dma_load16(xr, base + 1024 * j, xoff[j], g * (kGroup * 2));
  };
  // codes, steps and zero points of the wave's rows through buffer descriptors whose range ends at
  // the last valid row; rows past it read zero and their results are not stored. Lane (n, kq) holds
  // the 32 codes k = 32 kq .. 32 kq + 31 of group g of row row0 + 16 j + n. As for the activations,
  // the row (16 j + n) is in the per-lane offset, which the range check covers, and the scalar offset
  // holds only the group's position inside the row.
  const int vrows = max(0, min(kRowsPerWave, d_out - row0));
  const int64_t r0 = min(row0, d_out - 1);
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(codes + r0 * (d_in / 2)), (short)0, vrows * (d_in / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t sres =
      __builtin_amdgcn_make_buffer_rsrc((void*)(steps + r0 * G), (short)0, vrows * G * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t zres =
      __builtin_amdgcn_make_buffer_rsrc((void*)(zeros + r0 * GZ), (short)0, vrows * GZ, 0x00020000);
  const int c_off = n * (d_in / 2) + kq * 16, s_off = n * G * 2, z_off = n * GZ;
  uint4 cw[2][NJ];
  uint32_t sr[2][NJ], zr[2][NJ];
  auto load_w = [&](int g, int set) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      cw[set][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 cr, c_off + 16 * j * (d_in / 2), g * (kGroup / 2), 0));
      sr[set][j] = __builtin_amdgcn_raw_buffer_load_b16(sres, s_off + 16 * j * G * 2, g * 2, 0);
      zr[set][j] = __builtin_amdgcn_raw_buffer_load_b8(zres, z_off + 16 * j * GZ, g >> 1, 0);
    }
  };

  f32x4 acc[8][NJ];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int g, int buf) {
    // buf is also the codes register set of group g
    if (g + 1 < G) {
      load_x(g + 1, buf ^ 1);
      load_w(g + 1, buf ^ 1);
    }
    float st[NJ], nz[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) group_params(sr[buf][j], zr[buf][j], g, st[j], nz[j]);
    auto dq = [&](int t, uint4(&b)[NJ]) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t wj[4] = {cw[buf][j].x, cw[buf][j].y, cw[buf][j].z, cw[buf][j].w};
        b[j] = dequant8<KIND>(wj[t], st[j], nz[j]);
      }
    };
    // software pipeline: sub-step t's MFMAs run while sub-step t+1's operands are dequantized and
    // the next token tile's fragment is read from LDS
    uint4 bcur[NJ], bnext[NJ];
    dq(0, bcur);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 a = xs[buf][n * 16 + ((4 * kq + t) ^ n)];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint4 an;
        if (m + 1 < 8) {
          const int tr = 16 * (m + 1) + n;
          an = xs[buf][tr * 16 + ((4 * kq + t) ^ (tr & 15))];
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[m][j] = mma<KIND>(a, bcur[j], acc[m][j]);
        if (t + 1 < 4 && m < NJ) {
          // one row tile of the next sub-step's dequantization per token tile (j = m)
          const uint32_t wj[4] = {cw[buf][m].x, cw[buf][m].y, cw[buf][m].z, cw[buf][m].w};
          bnext[m] = dequant8<KIND>(wj[t + 1], st[m], nz[m]);
        }
        a = an;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) bcur[j] = bnext[j];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };

  load_x(0, 0);
  load_w(0, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  int g = 0;
  for (; g + 1 < G; g += 2) {
    step(g, 0);
    step(g + 1, 1);
  }
  if (g < G) step(g, 0);

#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
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

// Prefill at scale (thousands of tokens): the error GEMM's tiling with the weight operand produced in
// LDS. A block computes 256 tokens x 256 output rows; four waves as 2 x 2, each 128 x 128 as 4 x 4
// accumulators of v_mfma_f32_32x32x16_{bf16,f16}. A K step is 64 inputs: the activations (256 rows
// x 128 bytes) move global -> LDS by buffer DMA, and the weights are dequantized by the block's
// threads, one output row each (64 codes, the group's float16 step and zero point), into the same
// swizzled LDS layout, so every weight is dequantized once per 256 tokens and read by two waves.
// Two LDS stages: the activations of step kt+2 are loaded into the stage step kt has just freed, and
// its weights dequantized there, spread over the four sub-steps that follow (half a chunk of eight
// weights per four MFMAs); each step's codes are requested a step before their dequantization
// begins. Tiles in the super-block order of the error GEMM (one block per compute unit at a time).
constexpr int kTileTok = 256, kTileRows = 256, kTileKB = 128;
constexpr int kTileStage = (kTileTok + kTileRows) * kTileKB;  // 64 KiB
constexpr int64_t kTileMinTokens = 1024;

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int KIND, bool ZC>
__device__ __forceinline__ void mma32(const uint4& a, const uint4& b, f32x16& c) {
  const f32x16 zero = {};
  if constexpr (KIND == 0)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                ZC ? zero : c, 0, 0, 0);
  else
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                               ZC ? zero : c, 0, 0, 0);
}

// Byte j of a word as a float (v_cvt_f32_ubyte{j}: one instruction; written out because the compiler
// otherwise extracts the byte with a bit-field instruction first when it knows the upper bits are zero).
template <int J>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
  float f;
  if constexpr (J == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(w));
  else if constexpr (J == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(w));
  else if constexpr (J == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(w));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(w));
  return f;
}

// 8 codes (one word: element 2j in the low nibble of byte j, 2j+1 in the high one) -> 8 operands,
// (q - zero) * step rounded once to the 16-bit type; the low and high nibbles are masked four at a
// time and each byte converted directly.
template <int KIND>
__device__ __forceinline__ uint4 dequant8_bytes(uint32_t w, float st, float nzs) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const float v[8] = {fmaf(ubyte_f32<0>(lo), st, nzs), fmaf(ubyte_f32<0>(hi), st, nzs),
                      fmaf(ubyte_f32<1>(lo), st, nzs), fmaf(ubyte_f32<1>(hi), st, nzs),
                      fmaf(ubyte_f32<2>(lo), st, nzs), fmaf(ubyte_f32<2>(hi), st, nzs),
                      fmaf(ubyte_f32<3>(lo), st, nzs), fmaf(ubyte_f32<3>(hi), st, nzs)};
  return make_uint4(pack2(v[0], v[1], KIND), pack2(v[2], v[3], KIND), pack2(v[4], v[5], KIND),
                    pack2(v[6], v[7], KIND));
}

// group_params reading only the zero-point byte's low 8 bits (one byte-to-float conversion, the nibble
// then split off in exact float arithmetic): a byte loaded in one loop iteration and used in the next
// then needs no zero extension, which the compiler would otherwise place at the loop head and wait
// there for the load in flight
__device__ __forceinline__ void tile_group_params(uint32_t step_bits, uint32_t zbyte, int g, float& st, float& nzs) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)step_bits);
  const float zb = (float)(zbyte & 0xFFu);           // 0 .. 255
  const float zhi = __builtin_floorf(zb * 0.0625f);  // high nibble (exact)
  const float z = (g & 1) ? zhi : __builtin_fmaf(-16.f, zhi, zb);
  st = s;
  nzs = -z * s;  // exact: 4-bit integer times an 11-bit mantissa
}

template <int KIND, typename OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void w4a16_tile_kernel(const uint16_t* __restrict__ x, int64_t ld_x, const uint8_t* __restrict__ codes,
                       const uint16_t* __restrict__ steps, const uint8_t* __restrict__ zeros, int n_tokens,
                       int d_in, int d_out, OutT* __restrict__ y, int64_t ld_y, int tiles_m, int tiles_n) {
  constexpr int FM = 4, FN = 4, NR = 8, KB = kTileKB, BM = kTileTok;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kTileStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTileTok, n0 = (int64_t)tn * kTileRows;
  const int G = d_in / kGroup, GZ = (G + 1) / 2;
  const int k_steps = d_in / 64;  // >= 2

  // activations: DMA load j of wave w covers token rows (4 j + w) * 8 .. + 7 (as the error GEMM's A);
  // tokens past the end lie outside the descriptor's range and read as zero (their rows are not stored)
  const int lda_bytes = (int)ld_x * 2;
  const int rows_a = (int)min((int64_t)kTileTok, (int64_t)n_tokens - m0);
  const i32x4 ra = make_rsrc(x + m0 * ld_x, (uint32_t)((rows_a - 1) * lda_bytes + d_in * 2));
  int voff_a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (4 * j + wave) * 8 + (lane >> 3);
    voff_a[j] = row * lda_bytes + (((lane & 7) ^ swz(row)) << 4);
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_address(lds));
  auto dma_a = [&](uint32_t stage, int j, int kstep) {
    dma_load16(ra, __builtin_amdgcn_readfirstlane(stage + (4 * j + wave) * 8 * KB), voff_a[j], kstep * KB);
  };

  // weights: thread t dequantizes output row n0 + t; rows past d_out read zero codes, steps and zero
  // points through range-checked descriptors (the row offset is in the range-checked per-lane offset)
  const int vrows = (int)max((int64_t)0, min((int64_t)kTileRows, (int64_t)d_out - n0));
  const int64_t r0 = min(n0, (int64_t)d_out - 1);
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + r0 * (d_in / 2)), (short)0, vrows * (d_in / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void*)(steps + r0 * G), (short)0,
                                                                     vrows * G * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc((void*)(zeros + r0 * GZ), (short)0,
                                                                     vrows * GZ, 0x00020000);
  const int c_off = tid * (d_in / 2), s_off = tid * G * 2, z_off = tid * GZ;
  uint4 cw[2][2];           // codes of two K steps (64 each) in flight / in use
  uint32_t sw[2], zw[2];    // their group's raw float16 step and zero-point byte
  auto load_codes = [&](int set, int kstep) {
    cw[set][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(cr, c_off, kstep * 32, 0));
    cw[set][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(cr, c_off + 16, kstep * 32, 0));
    sw[set] = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off, (kstep >> 1) * 2, 0);
    zw[set] = __builtin_amdgcn_raw_buffer_load_b8(zr, z_off, kstep >> 2, 0);
  };
  // chunk c (inputs 8 c .. 8 c + 7 of the step) of this thread's row, into the stage's weight rows
  const uint32_t brow = BM * KB + tid * KB;
  auto code_word = [&](int set, int c) -> uint32_t {
    const uint4 u = cw[set][c >> 2];
    return (c & 3) == 0 ? u.x : (c & 3) == 1 ? u.y : (c & 3) == 2 ? u.z : u.w;
  };
  float gst[2], gnzs[2];  // the group's step and -zero * step for the step whose codes are in set 0 / 1
  auto params = [&](int set, int kstep) { tile_group_params(sw[set], zw[set], kstep >> 1, gst[set], gnzs[set]); };
  auto dequant_chunk = [&](char* stage, int set, int c) {
    *reinterpret_cast<uint4*>(stage + brow + ((c ^ swz(tid)) << 4)) =
        dequant8_bytes<KIND>(code_word(set, c), gst[set], gnzs[set]);
  };
  // the same as a pipeline of eight parts of at most four VALU instructions, one part after each MFMA
  // (a chunk per eight MFMAs): the parts' dependency chains span several MFMAs instead of stalling
  // the issue of the next one; part 7 writes the chunk to LDS
  uint32_t dlo = 0, dhi = 0, dq[4];
  float dv[4];
  auto dequant_part = [&](char* stage, int set, int c, int m) {
    const float st = gst[set], nzs = gnzs[set];
    if (m == 0) {
      const uint32_t wd = code_word(set, c);
      dlo = wd & 0x0F0F0F0Fu;
      dhi = (wd >> 4) & 0x0F0F0F0Fu;
    } else if (m == 1) {
      dv[0] = fmaf(ubyte_f32<0>(dlo), st, nzs);
      dv[1] = fmaf(ubyte_f32<0>(dhi), st, nzs);
    } else if (m == 2) {
      dq[0] = pack2(dv[0], dv[1], KIND);
      dv[2] = ubyte_f32<1>(dlo);
      dv[3] = ubyte_f32<1>(dhi);
    } else if (m == 3) {
      dq[1] = pack2(fmaf(dv[2], st, nzs), fmaf(dv[3], st, nzs), KIND);
    } else if (m == 4) {
      dv[0] = fmaf(ubyte_f32<2>(dlo), st, nzs);
      dv[1] = fmaf(ubyte_f32<2>(dhi), st, nzs);
    } else if (m == 5) {
      dq[2] = pack2(dv[0], dv[1], KIND);
      dv[2] = ubyte_f32<3>(dlo);
      dv[3] = ubyte_f32<3>(dhi);
    } else if (m == 6) {
      dq[3] = pack2(fmaf(dv[2], st, nzs), fmaf(dv[3], st, nzs), KIND);
    } else {
      *reinterpret_cast<uint4*>(stage + brow + ((c ^ swz(tid)) << 4)) = make_uint4(dq[0], dq[1], dq[2], dq[3]);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  const int ra_off = (wm * 128 + fr) * KB;
  const int rb_off = BM * KB + (wn * 128 + fr) * KB;
  int slot[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) slot[q] = ((2 * q + fh) ^ swz(fr)) << 4;
  f32x16 acc[FM][FN];
  auto frag = [&](const char* stage, int sl, int r) -> uint4 {
    const int off = r < FM ? ra_off + r * 32 * KB : rb_off + (r - FM) * 32 * KB;
    return *reinterpret_cast<const uint4*>(stage + off + sl);
  };
  // one sub-step: 16 MFMAs on `use` while the next sub-step's fragments are read (if `reads`); after
  // MFMA i of the 16, aux(i): at most one load, one LDS write or half a chunk of dequantization
  auto substep = [&](auto zc, const uint4 (&use)[NR], uint4 (&nxt)[NR], const char* src, int sl, bool reads,
                     auto aux) {
    constexpr bool ZC = decltype(zc)::value;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1, fn = (g & 1) * 2;
      mma32<KIND, ZC>(use[fm], use[FM + fn], acc[fm][fn]);
      __builtin_amdgcn_sched_barrier(0);
      aux(2 * g);
      if (reads) nxt[g] = frag(src, sl, g);
      __builtin_amdgcn_sched_barrier(0);
      mma32<KIND, ZC>(use[fm], use[FM + fn + 1], acc[fm][fn + 1]);
      __builtin_amdgcn_sched_barrier(0);
      aux(2 * g + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::false_type acc_in{};
  const std::true_type acc_zero{};
  auto none = [](int) {};

  // prologue: stage 0 (activations and weights) into buffer 0; stage 1's activations and the first
  // half of its weights into buffer 1 (the second half is done by step 0's first two sub-steps); the
  // codes of step 2 requested
  char* const buf[2] = {lds, lds + kTileStage};
  const uint32_t bufa[2] = {lds_base, lds_base + kTileStage};
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_a(bufa[0], j, 0);
  load_codes(0, 0);
  load_codes(1, 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  params(0, 0);
#pragma unroll
  for (int c = 0; c < 8; ++c) dequant_chunk(buf[0], 0, c);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_a(bufa[1], j, 1);
  params(1, 1);
#pragma unroll
  for (int c = 0; c < 4; ++c) dequant_chunk(buf[1], 1, c);
  // (past the last step the last step's codes are loaded again and not used: the loads stay
  // unconditional, so no register is carried around the loop by a branch and copied while in flight)
  load_codes(0, min(2, k_steps - 1));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  uint4 f0[NR], f1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) f0[r] = frag(buf[0], slot[0], r);
  substep(acc_zero, f0, f1, buf[0], slot[1], true, none);

  // step kt: B C | barrier | D A'. The weights of step kt+1 are finished (chunks 4..7) in B and C,
  // into its stage (read only after the barrier); D loads the activations of step kt+2 into the stage
  // of step kt (freed by the barrier), and D and A' dequantize chunks 0..3 of step kt+2's weights into
  // it; A' requests the codes of step kt+3 (into the register set B and C have just finished with).
  // Codes are thus requested before the barrier that precedes their first use, whose wait covers
  // them: the load counter completes in issue order, so a wait for codes requested after an
  // activation DMA would also wait for that DMA, long before its barrier needs it.
  // The parity of kt (buffer and codes register set) is a template argument: register arrays indexed
  // at run time would be placed in scratch memory.
  auto step = [&](int kt, auto parity) {
    constexpr int P = decltype(parity)::value;
    char* cur = buf[P];
    char* nxt = buf[P ^ 1];
    const bool pre2 = kt + 2 < k_steps;
    // a part of a chunk after every MFMA: B chunks 4, 5 and C chunks 6, 7 of step kt+1
    substep(acc_in, f1, f0, cur, slot[2], true, [&](int i) { dequant_part(nxt, P ^ 1, 4 + (i >> 3), i & 7); });
    substep(acc_in, f0, f1, cur, slot[3], true, [&](int i) { dequant_part(nxt, P ^ 1, 6 + (i >> 3), i & 7); });
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // D: step kt+2's activations into the freed stage (a load per pair of MFMAs) and its weight
    // chunks 0, 1; A': the codes of step kt+3 and chunks 2, 3
    substep(acc_in, f1, f0, nxt, slot[0], true, [&](int i) {
      if (pre2 && (i & 1) == 0) dma_a(bufa[P], i >> 1, kt + 2);
      if (pre2 && i == 0) params(P, kt + 2);
      if (pre2) dequant_part(cur, P, i >> 3, i & 7);
    });
    substep(acc_in, f0, f1, nxt, slot[1], true, [&](int i) {
      if (i == 0) load_codes(P ^ 1, min(kt + 3, k_steps - 1));
      if (pre2) dequant_part(cur, P, 2 + (i >> 3), i & 7);
    });
  };
  const std::integral_constant<int, 0> even{};
  const std::integral_constant<int, 1> odd{};
  // k_steps = d_in / 64 is even: steps 0 .. k_steps - 2 in pairs and one, then the last (odd) one
  int kt = 0;
  for (; kt + 2 < k_steps - 1; kt += 2) {
    step(kt, even);
    step(kt + 1, odd);
  }
  step(kt, even);
  {  // the last step (k_steps - 1, odd): B C D
    const char* cur = buf[1];
    substep(acc_in, f1, f0, cur, slot[2], true, none);
    substep(acc_in, f0, f1, cur, slot[3], true, none);
    substep(acc_in, f1, f0, cur, slot[0], false, none);
  }

  // element e of accumulator (i, j) in lane l: token 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 of the
  // wave's 128, output row 32 j + l % 32 of its 128
  const int64_t t_w = m0 + wm * 128, f_w = n0 + wn * 128;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t f = f_w + 32 * j + fr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = t_w + 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3);
        if (t < n_tokens && f < d_out) y[t * ld_y + f] = to_out<OutT>(acc[i][j][e], KIND);
      }
    }
}

template <int KIND, typename OutT>
hipError_t launch_kind(const void* x, int64_t ld_x, const uint8_t* codes, const uint16_t* steps,
                       const uint8_t* zeros, int n_tokens, int d_in, int d_out, void* y, int64_t ld_y, bool big,
                       hipStream_t st) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  OutT* yp = static_cast<OutT*>(y);
  const int64_t tiles64 =
      ((int64_t)(n_tokens + kTileTok - 1) / kTileTok) * ((int64_t)(d_out + kTileRows - 1) / kTileRows);
  if (big && n_tokens >= kTileMinTokens && tiles64 <= 0x7FFFFFFF) {
    const int tiles_m = (n_tokens + kTileTok - 1) / kTileTok, tiles_n = (d_out + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL((w4a16_tile_kernel<KIND, OutT>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, st,
                       xp, ld_x, codes, steps, zeros, n_tokens, d_in, d_out, yp, ld_y, tiles_m, tiles_n);
  } else if (big) {
    const unsigned gy = (unsigned)((n_tokens + kBigTokens - 1) / kBigTokens);
    if (n_tokens > kMidMaxTokens)
      hipLaunchKernelGGL((w4a16_big_kernel<KIND, OutT, kBigNJ>), dim3((unsigned)((d_out + 64 * kBigNJ - 1) / (64 * kBigNJ)), gy),
                         dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
    else
      hipLaunchKernelGGL((w4a16_big_kernel<KIND, OutT, kMidNJ>), dim3((unsigned)((d_out + 64 * kMidNJ - 1) / (64 * kMidNJ)), gy),
                         dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
  } else if (n_tokens == 1 && d_in <= kGemvMaxIn) {
    // about kGemvBlocks blocks of kGemvWaves waves, each wave a run of whole rows
    const int W = (d_in / kGroup + 15) / 16;
    const int64_t per = (int64_t)kGemvWaves * kGemvBlocks;
    const int rpw = (int)(((int64_t)d_out + per - 1) / per);
    const unsigned blocks = (unsigned)(((int64_t)d_out + (int64_t)kGemvWaves * rpw - 1) / ((int64_t)kGemvWaves * rpw));
    hipLaunchKernelGGL((w4a16_gemv_kernel<KIND, OutT>), dim3(blocks), dim3(64 * kGemvWaves), W * 4096, st, xp, codes,
                       steps, zeros, d_in, d_out, rpw, yp);
  } else {
    // 17-32 tokens: both 16-token tiles in one block, so each weight fragment is dequantized once
    const bool wide = d_out >= kSmallWideRows, two = n_tokens > 16;
    const dim3 grid((unsigned)((d_out + (wide ? 31 : 15)) / (wide ? 32 : 16)), 1);
    if (wide && two)
      hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT, 2, 2>), grid, dim3(64 * kSmallWaves), 0, st, xp, ld_x, codes,
                         steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
    else if (wide)
      hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT, 2, 1>), grid, dim3(64 * kSmallWaves), 0, st, xp, ld_x, codes,
                         steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
    else if (two)
      hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT, 1, 2>), grid, dim3(64 * kSmallWaves), 0, st, xp, ld_x, codes,
                         steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
    else
      hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT, 1, 1>), grid, dim3(64 * kSmallWaves), 0, st, xp, ld_x, codes,
                         steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
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
