// The block-level objective for the gate/up pair of a gated MLP: the error is measured at the MLP's
// output y = down(act(x gate^T) * (x up^T)), the lowest common ancestor of the two searched linears
// (msModelSlim "AWQ：激活感知权重量化算法说明", 关键特性 and 缩放因子搜索流程: block-level error on
// the ancestor module, float reference with the original weights).
//
// By linearity of the down projection, y_ref - y_k = (h_ref - h_k) down^T with h = act(g) * u, so
// the candidate's loss is the error GEMM's sum of squares of dh_k down^T. This file forms dh_k:
//   reference pass: G = X Wg^T and U = X Wu^T in float32 (once per search);
//   candidate pass: Eg = X dWg^T, Eu = X dWu^T (dW = What - W, as the quantize -> delta step writes
//   it), and in the epilogue dh = act(G) U - act(G + Eg) (U + Eu), rounded to bfloat16.
//
// The GEMM is the error GEMM's pipeline (256 x 256 tiles, four waves of 128 x 128, 32x32x16 bf16
// matrix-core instructions, operands global -> LDS by buffer DMA with XOR-swizzled 16-byte chunks,
// one DMA per MFMA pair, persistent workgroups walking the same super-block tile order). Its B tile
// is 128 gate rows followed by the same 128 up rows, so waves (wm, 0) and (wm, 1) hold the gate and
// up accumulators of the same 128 tokens x 128 hidden units. After the K loop each wave of the pair
// passes half of its accumulators to the other through LDS (same lane layout) and computes dh for the
// other half.
#include <algorithm>
#include <math.h>
#include <type_traits>

#include "block.h"
#include "lds_dma.h"

namespace awq {
namespace {

constexpr int BM = 256, BN = 256;  // tokens, B rows (128 gate + 128 up) per tile
constexpr int kHalf = 128;         // hidden units per tile
constexpr int KB = 128;
constexpr int kStageBytes = (BM + BN) * KB;  // 64 KiB
constexpr int kThreads = 256;
constexpr int kSplit = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool ZC>
__device__ __forceinline__ void mma_pair(const uint4& a, const uint4& b, f32x16& c) {
  const f32x16 zero = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                              ZC ? zero : c, 0, 0, 0);
}

struct TileOps {
  i32x4 ra, rg, ru;  // X rows, gate rows, up rows of the tile
  int tm, tn;
};

__device__ __forceinline__ TileOps tile_ops(int G, const uint16_t* x, int64_t ld_x, const uint16_t* wg,
                                            const uint16_t* wu, int64_t n_tokens, int64_t d_in, int64_t d_ff,
                                            int tiles_m, int tiles_n) {
  TileOps t;
  tile_of(G, tiles_m, tiles_n, t.tm, t.tn);
  const int64_t m0 = (int64_t)t.tm * BM, f0 = (int64_t)t.tn * kHalf;
  const int rows_a = (int)min((int64_t)BM, n_tokens - m0);
  const int rows_b = (int)min((int64_t)kHalf, d_ff - f0);
  const int lda_bytes = (int)(ld_x * 2), row_bytes = (int)(d_in * 2);
  t.ra = make_rsrc(x + m0 * ld_x, (rows_a - 1) * lda_bytes + row_bytes);
  t.rg = make_rsrc(wg + f0 * d_in, rows_b * row_bytes);
  t.ru = make_rsrc(wu + f0 * d_in, rows_b * row_bytes);
  return t;
}

template <int ACT>
__device__ __forceinline__ float act_f(float v) {
  if constexpr (ACT == kActRelu) return v > 0.f ? v : 0.f;
  else return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

// MODE kModeRef: g_out = X Wg^T, u_out = X Wu^T (float32, [n_tokens, d_ff]).
// MODE kModeDelta: wg/wu are dWg/dWu; dh = act(G) U - act(G + Eg)(U + Eu) with G, U read from
// g_ref / u_ref; bfloat16 [n_tokens, d_ff].
template <int MODE, int ACT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mlp_hidden_kernel(const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* __restrict__ wg,
                       const uint16_t* __restrict__ wu, int64_t n_tokens, int64_t d_in, int64_t d_ff, int tiles_m,
                       int tiles_n, float* __restrict__ g_io, float* __restrict__ u_io, uint16_t* __restrict__ dh) {
  constexpr int FM = 4, FN = 4, NR = 8;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = tiles_m * tiles_n;

  const int lda_bytes = (int)(ld_x * 2), row_bytes = (int)(d_in * 2);
  // 8 loads per operand per wave per stage: load j of wave w covers rows 8 (4 j + w) .. +7 of the
  // tile (B rows 0..127 gate, 128..255 up); lane i fills row 8 (4 j + w) + i / 8, slot i % 8,
  // which holds K chunk (i % 8) ^ swz(row)
  int voff_a[8], voff_b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (4 * j + wave) * 8 + (lane >> 3);
    const int sl = ((lane & 7) ^ swz(row)) << 4;
    voff_a[j] = row * lda_bytes + sl;
    voff_b[j] = (row & (kHalf - 1)) * row_bytes + sl;
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_address(lds));
  auto issue = [&](const TileOps& t, uint32_t stage, int i, int kbyte) {
    if (i < 8)
      dma_load16(t.ra, __builtin_amdgcn_readfirstlane(stage + (4 * i + wave) * 8 * KB), voff_a[i], kbyte);
    else
      dma_load16(i < 12 ? t.rg : t.ru, __builtin_amdgcn_readfirstlane(stage + BM * KB + (4 * (i - 8) + wave) * 8 * KB),
                 voff_b[i - 8], kbyte);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int ra_off = (wm * 128 + fr) * KB;
  // the up wave reads its four 32-row B fragments with the two halves swapped, so that in both
  // waves accumulators j = 0, 1 are the hidden units the wave finishes and j = 2, 3 those it passes
  // on: accumulator j of wave wn holds hidden units 32 (j ^ 2 wn) .. +31 of the tile
  const int rb_off = BM * KB + (wn * 128 + fr) * KB;
  const int rb_lo = rb_off + wn * 64 * KB, rb_hi = rb_off - wn * 64 * KB;
  int slot[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) slot[q] = ((2 * q + fh) ^ swz(fr)) << 4;
  const int k_steps = row_bytes / KB;

  f32x16 acc[FM][FN];
  auto frag = [&](const char* stage, int sl, int r) -> uint4 {
    const int off = r < FM ? ra_off + r * 32 * KB : (r < FM + 2 ? rb_lo : rb_hi) + (r - FM) * 32 * KB;
    return *reinterpret_cast<const uint4*>(stage + off + sl);
  };
  auto substep = [&](auto zc, const uint4(&use)[NR], uint4(&nxt)[NR], const char* src, int sl, bool reads,
                     const TileOps& lt, uint32_t fstage, int kbyte, int l0, int l1) {
    constexpr bool ZC = decltype(zc)::value;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1, fn = (g & 1) * 2;
      mma_pair<ZC>(use[fm], use[FM + fn], acc[fm][fn]);
      __builtin_amdgcn_sched_barrier(0);
      if (l0 + g < l1) issue(lt, fstage, l0 + g, kbyte);
      if (reads) nxt[g] = frag(src, sl, g);
      __builtin_amdgcn_sched_barrier(0);
      mma_pair<ZC>(use[fm], use[FM + fn + 1], acc[fm][fn + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::false_type acc_in{};
  const std::true_type acc_zero{};

  int G = blockIdx.x;
  if (G >= nblk) return;
  for (;;) {
    const TileOps cur_t = tile_ops(G, x, ld_x, wg, wu, n_tokens, d_in, d_ff, tiles_m, tiles_n);
    // every wave has passed the previous tile's final barrier: both buffers are free
#pragma unroll
    for (int i = 0; i < 16; ++i) issue(cur_t, lds_base, i, 0);
    uint4 f0[NR], f1[NR];
#pragma unroll
    for (int i = 0; i < kSplit; ++i) issue(cur_t, lds_base + kStageBytes, i, KB);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kSplit));
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) f0[r] = frag(lds, slot[0], r);
    substep(acc_zero, f0, f1, lds, slot[1], true, cur_t, lds_base + kStageBytes, KB, kSplit, 16);
    int kt = 0;
    for (; kt + 2 < k_steps; ++kt) {
      const int b = kt & 1;
      char* cur = lds + b * kStageBytes;
      char* nxt = lds + (b ^ 1) * kStageBytes;
      const uint32_t fre = lds_base + b * kStageBytes;  // stage kt's buffer, refilled with stage kt+2
      substep(acc_in, f1, f0, cur, slot[2], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, cur, slot[3], true, cur_t, 0, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // stage kt+1 has landed
      __syncthreads();                           // and every wave has read all of stage kt
      substep(acc_in, f1, f0, nxt, slot[0], true, cur_t, fre, (kt + 2) * KB, 0, kSplit);
      substep(acc_in, f0, f1, nxt, slot[1], true, cur_t, fre, (kt + 2) * KB, kSplit, 16);
    }
    {  // K step k_steps-2 (B C D) and the first sub-step of the last one
      const int b = kt & 1;
      char* cur = lds + b * kStageBytes;
      char* nxt = lds + (b ^ 1) * kStageBytes;
      substep(acc_in, f1, f0, cur, slot[2], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, cur, slot[3], true, cur_t, 0, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      substep(acc_in, f1, f0, nxt, slot[0], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, nxt, slot[1], true, cur_t, 0, 0, 0, 0);
      ++kt;
    }
    {  // K step k_steps-1: B C D
      const int b = kt & 1;
      char* cur = lds + b * kStageBytes;
      substep(acc_in, f1, f0, cur, slot[2], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, cur, slot[3], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f1, f0, cur, slot[0], false, cur_t, 0, 0, 0, 0);
    }

    // Element e of accumulator (i, j) in lane l is token 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 of
    // the wave's 128 and hidden unit 32 j + l % 32 of the tile's 128.
    const int64_t tok_w = (int64_t)cur_t.tm * BM + wm * 128;
    const int64_t f_w = (int64_t)cur_t.tn * kHalf;
    __syncthreads();  // every wave has read the last stage: LDS is free for the exchange
    if constexpr (MODE == kModeRef) {
      float* out = wn == 0 ? g_io : u_io;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t f = f_w + 32 * (j ^ (2 * wn)) + fr;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t t = tok_w + 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3);
            if (t < n_tokens && f < d_ff) out[t * d_ff + f] = acc[i][j][e];
          }
        }
    } else {
      // Both waves of a pair share the work: each finishes the hidden units of its accumulators
      // j = 0, 1 and passes j = 2, 3 to its partner through LDS (lane-major, 16 values per
      // accumulator); the partner's are the other operand for the same units. Reference values are
      // loaded unconditionally (clamped to the last valid token / unit; results outside are not stored).
      const int64_t tmax = n_tokens - 1, fmax = d_ff - 1;
      float* give = reinterpret_cast<float*>(lds) + (wm * 2 + wn) * (FM * 2 * 16 * 64);
      const float* take = reinterpret_cast<const float*>(lds) + (wm * 2 + (wn ^ 1)) * (FM * 2 * 16 * 64);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 w = {acc[i][2 + jj][4 * q], acc[i][2 + jj][4 * q + 1], acc[i][2 + jj][4 * q + 2],
                             acc[i][2 + jj][4 * q + 3]};
            *reinterpret_cast<f32x4*>(give + (((i * 2 + jj) * 4 + q) * 64 + lane) * 4) = w;
          }
      const bool is_gate = wn == 0;
      // the reference values of four accumulator groups are in flight (one or two exposed the loads'
      // latency group by group); the first four go out before the exchange's barrier
      constexpr int D = 4;
      float gv[D][16], uv[D][16];
      auto load_ref = [&](int n, int b) {
        const int i = n >> 1, jj = n & 1;
        const int64_t fc = min(f_w + 32 * (jj + 2 * wn) + fr, fmax);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = min(tok_w + 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3), tmax);
          gv[b][e] = g_io[t * d_ff + fc];
          uv[b][e] = u_io[t * d_ff + fc];
        }
      };
#pragma unroll
      for (int n = 0; n < D; ++n) load_ref(n, n);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int n = i * 2 + jj;
          const int64_t f = f_w + 32 * (jj + 2 * wn) + fr;
          const float (&gn)[16] = gv[n % D];
          const float (&un)[16] = uv[n % D];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 oth = *reinterpret_cast<const f32x4*>(take + ((n * 4 + q) * 64 + lane) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = 4 * q + r;
              const float own = acc[i][jj][e];
              const float eg = is_gate ? own : oth[r];
              const float eu = is_gate ? oth[r] : own;
              const float d = act_f<ACT>(gn[e]) * un[e] - act_f<ACT>(gn[e] + eg) * (un[e] + eu);
              const int64_t t = tok_w + 32 * i + 8 * q + 4 * fh + r;
              if (t < n_tokens && f < d_ff) dh[t * d_ff + f] = (uint16_t)(pack_bf16x2(d, 0.f) & 0xFFFFu);
            }
          }
          if (n + D < FM * 2) load_ref(n + D, n % D);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();  // LDS is free again for the next tile's stages
    G += (int)gridDim.x;
    if (G >= nblk) break;
  }
}

int compute_units() {
  // compute units of the current device, looked up once per device and thread
  static thread_local int cus_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cus_of[dev];
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cus_of[dev] = cus;
  }
  return cus;
}

}  // namespace

hipError_t launch_mlp_hidden(int mode, int act, const void* x, int64_t ld_x, const void* wg, const void* wu,
                             int64_t n_tokens, int64_t d_in, int64_t d_ff, float* g_io, float* u_io, void* dh,
                             hipStream_t st) {
  const int tiles_m = (int)((n_tokens + BM - 1) / BM);
  const int tiles_n = (int)((d_ff + kHalf - 1) / kHalf);
  const int64_t nblk = (int64_t)tiles_m * tiles_n;
  const unsigned grid = (unsigned)std::min<int64_t>(nblk, compute_units());
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* gp = static_cast<const uint16_t*>(wg);
  const uint16_t* up = static_cast<const uint16_t*>(wu);
  uint16_t* hp = static_cast<uint16_t*>(dh);
  if (mode == kModeRef)
    hipLaunchKernelGGL((mlp_hidden_kernel<kModeRef, kActSilu>), dim3(grid), dim3(kThreads), 0, st, xp, ld_x, gp, up,
                       n_tokens, d_in, d_ff, tiles_m, tiles_n, g_io, u_io, hp);
  else if (act == kActRelu)
    hipLaunchKernelGGL((mlp_hidden_kernel<kModeDelta, kActRelu>), dim3(grid), dim3(kThreads), 0, st, xp, ld_x, gp,
                       up, n_tokens, d_in, d_ff, tiles_m, tiles_n, g_io, u_io, hp);
  else
    hipLaunchKernelGGL((mlp_hidden_kernel<kModeDelta, kActSilu>), dim3(grid), dim3(kThreads), 0, st, xp, ld_x, gp,
                       up, n_tokens, d_in, d_ff, tiles_m, tiles_n, g_io, u_io, hp);
  return hipGetLastError();
}

}  // namespace awq
