// a4: the output error of every candidate, E_j = X * delta_j^T, squared and summed per tile
// without ever being written out.
//
// The loss of a ratio is mean((X W^T - X What^T)^2) (gsyq.cn "AWQ 离群激活平滑实操", section 二,
// target_out / actual_out; bjdmk.com.cn AWQ article, L(s) in "数学等价变换与通道自适应缩放").
// By linearity X W^T - X What^T = -X (What - W)^T, so one GEMM against delta = What - W gives
// the error directly (the two reference outputs are never formed), and the squared-error
// reduction runs in the GEMM epilogue on the accumulators.
//
// Both operands are K-contiguous ([rows, d_in] row-major): M = tokens, N = candidate rows
// (candidates stacked along N), K = d_in. Tiles are 256 x 256, four waves in a 2 x 2
// arrangement, each wave a 128 x 128 sub-tile held as 4 x 4 accumulators (256 AGPRs) of the
// 32x32 matrix-core instruction (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2_f32 for
// f32). A K step is 128 bytes of every row (64 bf16 / 32 f32), four 32-byte sub-steps.
//
// Operands move global -> LDS with buffer loads that write LDS directly (16 bytes per lane, 8
// lanes per 128-byte row segment, so every L1 request is a full cache line; with 64-byte row
// segments the texture unit was saturated by twice as many half-line requests). Rows past the
// end of X or of a candidate's delta lie outside the buffer descriptor's range and read as
// zero, which adds nothing to a sum of squares. Two 64 KiB LDS stages: a stage's loads go out
// right after the barrier that frees its buffer and have a whole K step of matrix work to land.
// The MFMAs of each sub-step run while the next sub-step's fragments are read from LDS, and
// the loads are placed between MFMA pairs. The 16-byte chunks of each LDS row are XOR-swizzled
// by row, which leaves the fragment reads free of bank conflicts.
//
// Tile order: the 256 concurrently running tiles form a 16 x 16 super-block, split 8 x 4 per XCD
// (tile_of in lds_dma.h), so operand K-slices are shared inside each XCD's L2 and across the XCDs in
// the memory-side cache.
#include <algorithm>
#include <type_traits>

#include "gemm.h"
#include "lds_dma.h"

namespace awq {
namespace {

constexpr int BM = kTileM, BN = kTileN;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One 16-byte fragment pair: a 32 x 32 x (16 bf16 | 8 f32) product into one accumulator; with ZC
// the accumulator's old value is not read (the matrix core adds to zero), which starts a tile
// without clearing 256 accumulator registers.
template <typename T, bool ZC = false>
__device__ __forceinline__ void mma_pair(const uint4& a, const uint4& b, f32x16& c) {
  const f32x16 zero = {};
  if constexpr (sizeof(T) == 2) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                ZC ? zero : c, 0, 0, 0);
  } else {
    // four K=2 steps; lane half h contributes K index 4h+e of the 8-wide chunk pair in step e,
    // identically for both operands
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), ZC ? zero : c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
}

constexpr int KB = 128;
constexpr int kStageBytes = (BM + BN) * KB;  // 64 KiB
constexpr int kThreads = 256;
// Of a stage's 16 loads per wave, kSplit go out in the last sub-step of the step two ahead of
// its use (right after the barrier that frees its buffer) and the rest in the first sub-step
// of the next step, so the texture unit sees no burst.
constexpr int kSplit = 8;

// Operand descriptors of one tile: A = its 256 token rows of X, B = its 256 rows of the
// candidate's delta, each a raw buffer whose range ends at the last valid row.
struct TileOps {
  i32x4 ra, rb;
  int idx;  // tile_sse index
};
template <typename T>
__device__ __forceinline__ TileOps tile_ops(int G, const T* x, int64_t ld_x, const T* delta, int64_t n_tokens,
                                            int64_t d_in, int64_t d_out, int tiles_m, int tiles_n, int n_cols) {
  int tm, col;
  tile_of(G, tiles_m, n_cols, tm, col);
  const int cand = col / tiles_n;
  const int tn = col % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, n_tokens - m0);
  const int rows_b = (int)min((int64_t)BN, d_out - n0);
  const int lda_bytes = (int)(ld_x * (int64_t)sizeof(T));
  const int row_bytes = (int)(d_in * (int64_t)sizeof(T));
  TileOps t;
  t.ra = make_rsrc(x + m0 * ld_x, (rows_a - 1) * lda_bytes + row_bytes);
  t.rb = make_rsrc(delta + ((int64_t)cand * d_out + n0) * d_in, (rows_b - 1) * row_bytes + row_bytes);
  t.idx = cand * tiles_m * tiles_n + tm * tiles_n + tn;
  return t;
}

// Persistent: one workgroup per compute unit walks tiles G = blockIdx.x, + gridDim.x, ... The
// next tile's first K stage is loaded into the free LDS buffer during the current tile's last K
// step, so its load latency hides behind that step and the epilogue.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void error_sse_kernel(const T* __restrict__ x, int64_t ld_x, const T* __restrict__ delta,
                      int64_t n_tokens, int64_t d_in, int64_t d_out, int tiles_m, int tiles_n,
                      int n_cols, double* __restrict__ tile_sse) {
  constexpr int FM = 4, FN = 4, NR = 8;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStageBytes];
  __shared__ double red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = tiles_m * n_cols;

  const int lda_bytes = (int)(ld_x * (int64_t)sizeof(T));
  const int row_bytes = (int)(d_in * (int64_t)sizeof(T));
  // 8 loads per operand per wave per stage: load j of wave w covers rows 8*(4j+w) .. +7; lane i
  // fills row 8*(4j+w) + i/8, slot i%8, which holds K chunk (i%8) ^ swz(row)
  int voff_a[8], voff_b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (4 * j + wave) * 8 + (lane >> 3);
    const int sl = ((lane & 7) ^ swz(row)) << 4;
    voff_a[j] = row * lda_bytes + sl;
    voff_b[j] = row * row_bytes + sl;
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_address(lds));
  // load i of 16 (8 of A, then 8 of B) of the stage at LDS address `stage`, K offset kbyte
  auto issue = [&](const TileOps& t, uint32_t stage, int i, int kbyte) {
    if (i < 8)
      dma_load16(t.ra, __builtin_amdgcn_readfirstlane(stage + (4 * i + wave) * 8 * KB), voff_a[i], kbyte);
    else
      dma_load16(t.rb, __builtin_amdgcn_readfirstlane(stage + BM * KB + (4 * (i - 8) + wave) * 8 * KB),
                 voff_b[i - 8], kbyte);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int ra_off = (wm * 128 + fr) * KB;
  const int rb_off = BM * KB + (wn * 128 + fr) * KB;
  int slot[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) slot[q] = ((2 * q + fh) ^ swz(fr)) << 4;
  const int k_steps = row_bytes / KB;  // >= 2: d_in is a positive multiple of 128

  f32x16 acc[FM][FN];
  auto frag = [&](const char* stage, int sl, int r) -> uint4 {
    const int off = r < FM ? ra_off + r * 32 * KB : rb_off + (r - FM) * 32 * KB;
    return *reinterpret_cast<const uint4*>(stage + off + sl);
  };
  // one sub-step: 16 MFMAs on `use`; between the two MFMAs of each of its 8 pairs, at most one
  // load (of [l0, l1), tile `lt`'s stage at LDS address `fstage`, K offset kbyte) and one of the
  // next sub-step's fragment reads (if `reads`). A load holds up the wave's issue for about as
  // long as the texture unit takes to accept its 64 addresses, so one per MFMA keeps the matrix
  // core fed (two back to back left it idle for ~10 % of the cycles).
  // (zc: the tile's first sub-step, which writes every accumulator once from zero)
  auto substep = [&](auto zc, const uint4 (&use)[NR], uint4 (&nxt)[NR], const char* src, int sl, bool reads,
                     const TileOps& lt, uint32_t fstage, int kbyte, int l0, int l1) {
    constexpr bool ZC = decltype(zc)::value;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1, fn = (g & 1) * 2;
      mma_pair<T, ZC>(use[fm], use[FM + fn], acc[fm][fn]);
      __builtin_amdgcn_sched_barrier(0);
      if (l0 + g < l1) issue(lt, fstage, l0 + g, kbyte);
      if (reads) nxt[g] = frag(src, sl, g);
      __builtin_amdgcn_sched_barrier(0);
      mma_pair<T, ZC>(use[fm], use[FM + fn + 1], acc[fm][fn + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::false_type acc_in{};
  const std::true_type acc_zero{};

  int G = blockIdx.x;
  if (G >= nblk) return;
  TileOps cur_t = tile_ops<T>(G, x, ld_x, delta, n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols);
  int par = 0;  // LDS buffer holding the tile's K stage 0
#pragma unroll
  for (int i = 0; i < 16; ++i) issue(cur_t, lds_base, i, 0);

  for (;;) {
    const int Gn = G + (int)gridDim.x;
    const bool has_next = Gn < nblk;
    const TileOps nxt_t =
        tile_ops<T>(has_next ? Gn : G, x, ld_x, delta, n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols);
    uint4 f0[NR], f1[NR];
    // stage 0 is in flight in buffer par; the first kSplit loads of stage 1 go to the other
    // buffer (free: every wave passed the previous tile's final barrier); wait for stage 0
#pragma unroll
    for (int i = 0; i < kSplit; ++i) issue(cur_t, lds_base + (par ^ 1) * kStageBytes, i, KB);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kSplit));
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) f0[r] = frag(lds + par * kStageBytes, slot[0], r);

    // A K step is four sub-steps A B C D on fragment slots 0..3 (each sub-step reads the next
    // one's fragments); the loop runs B C | barrier | D A', so that K step 0's A, which starts
    // the accumulators, stays outside it. Loads: the rest of stage kt+1 in A(kt), the first
    // kSplit of stage kt+2 in D(kt) into the buffer the barrier of step kt freed.
    substep(acc_zero, f0, f1, lds + par * kStageBytes, slot[1], true, cur_t, lds_base + (par ^ 1) * kStageBytes, KB,
            kSplit, 16);
    int kt = 0;
    for (; kt + 2 < k_steps; ++kt) {
      const int b = (kt + par) & 1;
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
    {  // K step k_steps-2 (B C D), then A of the last step, which starts the next tile's stage 0
      // in the buffer this step's barrier freed
      const int b = (kt + par) & 1;
      char* cur = lds + b * kStageBytes;
      char* nxt = lds + (b ^ 1) * kStageBytes;
      const uint32_t fre = lds_base + b * kStageBytes;
      const int nl = has_next ? 16 : 0;
      substep(acc_in, f1, f0, cur, slot[2], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, cur, slot[3], true, cur_t, 0, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();  // every wave has read all of stage k_steps-2: its buffer is free
      substep(acc_in, f1, f0, nxt, slot[0], true, cur_t, 0, 0, 0, 0);
      substep(acc_in, f0, f1, nxt, slot[1], true, nxt_t, fre, 0, 0, min(nl, 8));
      ++kt;
    }
    {  // K step k_steps-1: B C D
      const int b = (kt + par) & 1;
      char* cur = lds + b * kStageBytes;
      const uint32_t fre = lds_base + (b ^ 1) * kStageBytes;
      const int nl = has_next ? 16 : 0;
      substep(acc_in, f1, f0, cur, slot[2], true, nxt_t, fre, 0, 8, nl);
      substep(acc_in, f0, f1, cur, slot[3], true, nxt_t, 0, 0, 0, 0);
      substep(acc_in, f1, f0, cur, slot[0], false, nxt_t, 0, 0, 0, 0);
      par = b ^ 1;
    }

    // sum of squares: each accumulator's 16 values in float32 (relative error below 1e-6), the
    // 16 accumulators and then lanes, waves in float64
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float s32 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) s32 = fmaf(acc[i][j][e], acc[i][j][e], s32);
        ss += (double)s32;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();  // red is complete, and every wave has read the last stage
    if (threadIdx.x == 0) tile_sse[cur_t.idx] = (red[0] + red[1]) + (red[2] + red[3]);
    if (!has_next) break;
    G = Gn;
    cur_t = nxt_t;
  }
}

}  // namespace

hipError_t launch_error_sse(const void* x, int64_t ld_x, const void* delta, int dtype,
                            int64_t n_tokens, int64_t d_in, int64_t d_out, int n_cand,
                            double* tile_sse, hipStream_t st) {
  const int tiles_m = (int)((n_tokens + BM - 1) / BM);
  const int tiles_n = (int)((d_out + BN - 1) / BN);
  const int n_cols = tiles_n * n_cand;
  const int64_t nblk = (int64_t)tiles_m * n_cols;
  // one persistent workgroup per compute unit (the tile order assumes 8 XCDs dealt round-robin)
  // compute units of the current device, looked up once per device and thread
  static thread_local int cus_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cus_of[dev];
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cus_of[dev] = cus;
  }
  const unsigned grid = (unsigned)std::min<int64_t>(nblk, cus);
  if (dtype == 1)
    hipLaunchKernelGGL((error_sse_kernel<uint16_t>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(delta),
                       n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse);
  else
    hipLaunchKernelGGL((error_sse_kernel<float>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const float*>(x), ld_x, static_cast<const float*>(delta), n_tokens,
                       d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse);
  return hipGetLastError();
}

}  // namespace awq
