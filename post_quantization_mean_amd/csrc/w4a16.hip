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
#include "lds_dma.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;   // small-M kernel: groups whose codes a wave loads at once
constexpr int kXSub = 4;    // small-M kernel: groups whose activations are loaded at once
constexpr int kSmallWaves = 8;  // small-M kernel: waves per block, each 1/8 of the groups (a 4096-input
                                // layer's codes then fit one batch per wave)
constexpr int kSmallNT = 1; // small-M kernel: 16-row tiles per wave (more cut the activations' L2
                            // re-reads but leave too few blocks for layers of 4096 rows)
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

// Few tokens (decode): a block computes 16 tokens x (16 kSmallNT) output rows; its eight waves take
// eight contiguous ranges of the groups and their partial products are added in wave order. The
// weights, read once per 16 tokens, dominate the HBM traffic; each activation fragment is used for
// kSmallNT row tiles, which divides the activations' re-reads from L2. Loads are unconditional
// (rows and tokens past the end read the last valid one, whose results are never stored) so that a
// batch's loads all go out back to back; the codes of the next batch are in flight while the
// current one is multiplied.
template <int KIND, typename OutT>
__global__ __launch_bounds__(64 * kSmallWaves) void w4a16_small_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                              const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ steps,
                                                              const uint8_t* __restrict__ zeros, int n_tokens,
                                                              int d_in, int d_out, OutT* __restrict__ y,
                                                              int64_t ld_y) {
  constexpr int NT = kSmallNT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int tok = min(blockIdx.y * 16 + n, n_tokens - 1);
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
  const uint16_t* xrow = x + (int64_t)tok * ld_x + kq * 32;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        uint4 a[kXSub][4];
#pragma unroll
        for (int i = 0; i < kXSub; ++i) {
          const int g = min(gb + h + i, g_end - 1);
#pragma unroll
          for (int t = 0; t < 4; ++t) a[i][t] = *reinterpret_cast<const uint4*>(xrow + g * kGroup + t * 8);
        }
#pragma unroll
        for (int i = 0; i < kXSub; ++i) {
          if (gb + h + i < g_end) {  // wave-uniform
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const uint32_t wt[4] = {cur[h + i][j].x, cur[h + i][j].y, cur[h + i][j].z, cur[h + i][j].w};
#pragma unroll
              for (int t = 0; t < 4; ++t)
                acc[j] = mma<KIND>(a[i][t], dequant8<KIND>(wt[t], st[h + i][j], nzs[h + i][j]), acc[j]);
            }
          }
        }
      }
    }
  }
  __shared__ f32x4 red[kSmallWaves][NT][64];
#pragma unroll
  for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  if (wave < NT) {
    const int j = wave;
    f32x4 s = red[0][j][lane];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) s += red[w][j][lane];
    // C layout of the 16x16 result: lane l holds rows 4 (l / 16) .. +3 of column l mod 16
    const int orow = blockIdx.x * (16 * NT) + 16 * j + (lane & 15);
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t2 = blockIdx.y * 16 + 4 * (lane >> 4) + i;
      if (orow < d_out && t2 < n_tokens) y[(int64_t)t2 * ld_y + orow] = to_out<OutT>(sv[i], KIND);
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

template <int KIND, typename OutT>
hipError_t launch_kind(const void* x, int64_t ld_x, const uint8_t* codes, const uint16_t* steps,
                       const uint8_t* zeros, int n_tokens, int d_in, int d_out, void* y, int64_t ld_y, bool big,
                       hipStream_t st) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  OutT* yp = static_cast<OutT*>(y);
  if (big) {
    const unsigned gy = (unsigned)((n_tokens + kBigTokens - 1) / kBigTokens);
    if (n_tokens > kMidMaxTokens)
      hipLaunchKernelGGL((w4a16_big_kernel<KIND, OutT, kBigNJ>), dim3((unsigned)((d_out + 64 * kBigNJ - 1) / (64 * kBigNJ)), gy),
                         dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
    else
      hipLaunchKernelGGL((w4a16_big_kernel<KIND, OutT, kMidNJ>), dim3((unsigned)((d_out + 64 * kMidNJ - 1) / (64 * kMidNJ)), gy),
                         dim3(kThreads), 0, st, xp, ld_x, codes, steps, zeros, n_tokens, d_in, d_out, yp, ld_y);
  } else {
    const dim3 grid((unsigned)((d_out + 16 * kSmallNT - 1) / (16 * kSmallNT)), (unsigned)((n_tokens + 15) / 16));
    hipLaunchKernelGGL((w4a16_small_kernel<KIND, OutT>), grid, dim3(64 * kSmallWaves), 0, st, xp, ld_x, codes, steps, zeros,
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
