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
//
// The same data movement serves the Gram form of the loss (gram.hip): with A = B = X^T it stores
// the float32 tiles of G = X^T X on and above the diagonal (kStore; G is symmetric), and with A = G
// and B = the candidates' delta, both in float16, it sums products T[o, j] delta[o, j] per tile
// (kQuad), T = delta G over a K range, so that the tiles hold shares of the quadratic form
// delta G delta^T. With d_in cut into 256-blocks, the form is the sum over block pairs (I, J) of
// delta_I G_IJ delta_J^T, and G_JI = G_IJ^T makes the (J, I) term equal to the (I, J) one, so the
// form is sum_I (delta_I G_II delta_I^T + 2 sum_{J>I} delta_I G_IJ delta_J^T): row tile I runs K over
// the blocks J >= I, about half the matrix work of the full K range: G is stored with its diagonal
// blocks halved (gram.hip), and the tile's sum is doubled. The tiles' lengths fall with I, so a compute
// unit takes row tile I and then row tile R - 1 - I of the same column (R = ceil(d_in / 256) row
// tiles): every pair has the same length, the 256 units stay in step, and their 16 x 16
// super-blocks keep sharing operands in L2.
// The first tile of a pair walks K down from d_in and the second walks it up, so that at any
// moment the tiles of either kind read the same K slice.
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// epilogues: the tile's sum of squares, the float32 tile itself, the quadratic-form share
enum { kSse = 0, kStore = 1, kQuad = 2 };

template <typename T, bool ZC = false, bool F16 = false>
__device__ __forceinline__ void mma_pair(const uint4& a, const uint4& b, f32x16& c) {
  const f32x16 zero = {};
  if constexpr (F16) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                               ZC ? zero : c, 0, 0, 0);
  } else if constexpr (sizeof(T) == 2) {
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

// Operand descriptors of one tile: A = its 256 rows of the first operand (tokens of X; in the Gram
// form rows of X^T or of G), B = its 256 rows of the second (a candidate's delta; X^T), each a raw
// buffer that starts at the tile's first K element and whose range ends at the last valid row.
struct TileOps {
  i32x4 ra, rb;
  int idx;   // tile_sse index
  int m0, n0, cand;
  int k_steps;  // K steps of this tile (>= 2)
  int k_last;   // kQuad: byte offset of the last K step if K is walked downwards, else 0
};
// Tile G of the upper triangle tm <= tn of a tiles x tiles grid, row by row.
__device__ __forceinline__ void tri_of(int G, int tiles, int& tm, int& tn) {
  int r = 0, rem = G;
  while (rem >= tiles - r) {
    rem -= tiles - r;
    ++r;
  }
  tm = r;
  tn = r + rem;
}
// The same triangle in super-block rows of 16 tile rows: for the super-block row starting at tile
// row r0, its h(h+1)/2 tiles on the diagonal (row by row), then its h x (tiles - r0 - h) tiles right
// of them in tile_of's order, so that the tiles running together share operand panels inside each
// XCD's L2.
__device__ __forceinline__ void tri_tile(int G, int tiles, int& tm, int& tn) {
  int r0 = 0, rem = G;
  for (;;) {
    const int h = min(kSuper, tiles - r0), n_diag = h * (h + 1) / 2, n_right = h * (tiles - r0 - h);
    if (rem < n_diag) {
      tri_of(rem, h, tm, tn);
      tm += r0;
      tn += r0;
      return;
    }
    rem -= n_diag;
    if (rem < n_right) {
      tile_of(rem, h, tiles - r0 - h, tm, tn);
      tm += r0;
      tn += r0 + h;
      return;
    }
    rem -= n_right;
    r0 += kSuper;
  }
}

// kQuad work items: the R x n_cols tiles (R = tiles_m) in pairs of rows (I, R - 1 - I), see the
// file comment; with R odd the middle row comes last. Item G runs on unit G % grid as that unit's
// (G / grid)-th tile, so pair p of the top rows is taken by items that are grid apart: chunks of
// grid items alternate between first and second tiles (the last, partial chunk of pairs lists its
// first tiles, then their partners).
__device__ __forceinline__ void quad_tile(int G, int R, int n_cols, int grid, int& tm, int& col, bool& down) {
  const int n_pairs = (R / 2) * n_cols;
  if (G < 2 * n_pairs) {
    const int full = n_pairs / grid, rem = n_pairs - full * grid;
    int p, second;
    if (G < 2 * full * grid) {
      const int c = G / grid;
      p = (c >> 1) * grid + (G - c * grid);
      second = c & 1;
    } else {
      const int g = G - 2 * full * grid;
      second = g >= rem;
      p = full * grid + (second ? g - rem : g);
    }
    tile_of(p, R / 2, n_cols, tm, col);
    if (second) tm = R - 1 - tm;
    down = !second;
  } else {  // R odd: the middle row, its tiles all of one length
    tm = R / 2;
    col = G - 2 * n_pairs;
    down = false;
  }
}

template <typename T, int MODE>
__device__ __forceinline__ TileOps tile_ops(int G, const T* x, int64_t ld_x, const T* delta, int64_t n_tokens,
                                            int64_t d_in, int64_t d_out, int tiles_m, int tiles_n, int n_cols,
                                            int64_t cand_stride) {
  int tm, col;
  int64_t k0 = 0;  // K range [k0, d_in) in elements
  bool down = false;
  if constexpr (MODE == kStore) {
    tri_tile(G, tiles_m, tm, col);
  } else if constexpr (MODE == kQuad) {
    quad_tile(G, tiles_m, n_cols, (int)gridDim.x, tm, col, down);
    k0 = (int64_t)tm * BM;
  } else {
    tile_of(G, tiles_m, n_cols, tm, col);
  }
  const int cand = col / tiles_n;
  const int tn = col % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, n_tokens - m0);
  const int rows_b = (int)min((int64_t)BN, d_out - n0);
  const int lda_bytes = (int)(ld_x * (int64_t)sizeof(T));
  const int row_bytes = (int)(d_in * (int64_t)sizeof(T));
  const int kb0 = (int)(k0 * (int64_t)sizeof(T));  // both bases start at K element k0
  TileOps t;
  t.ra = make_rsrc(x + m0 * ld_x + k0, (rows_a - 1) * lda_bytes + row_bytes - kb0);
  t.rb = make_rsrc(delta + ((int64_t)cand * d_out + n0) * d_in + k0, (rows_b - 1) * row_bytes + row_bytes - kb0);
  t.idx = (int)(cand * cand_stride + (int64_t)tm * tiles_n + tn);
  t.m0 = (int)m0;
  t.n0 = (int)n0;
  t.cand = cand;
  t.k_steps = (int)((d_in - k0) * (int64_t)sizeof(T) / KB);
  t.k_last = down ? (t.k_steps - 1) * KB : 0;
  return t;
}

// Arguments of the kStore and kQuad epilogues.
struct Epi {
  float* c;                     // kStore: the float32 output, row pitch ld_c
  int64_t ld_c;
  const int32_t* dexp;          // kQuad: delta of candidate k is scaled by 2^dexp[k] ...
  const int32_t* gexp;          // ... and G by 2^gexp[0]
  int64_t cand_stride;          // tile_sse entries per candidate
};

// Persistent: one workgroup per compute unit walks tiles G = blockIdx.x, + gridDim.x, ... The
// next tile's first K stage is loaded into the free LDS buffer during the current tile's last K
// step, so its load latency hides behind that step and the epilogue.
template <typename T, int MODE = kSse>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void error_sse_kernel(const T* __restrict__ x, int64_t ld_x, const T* __restrict__ delta,
                      int64_t n_tokens, int64_t d_in, int64_t d_out, int tiles_m, int tiles_n,
                      int n_cols, double* __restrict__ tile_sse, Epi epi) {
  constexpr int FM = 4, FN = 4, NR = 8;
  constexpr bool F16 = MODE == kQuad;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStageBytes];
  __shared__ double red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // kStore (G = X^T X, symmetric): only the tiles with tm <= tn
  const int nblk = MODE == kStore ? tiles_m * (tiles_m + 1) / 2 : tiles_m * n_cols;

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
    if constexpr (MODE == kQuad) kbyte = t.k_last ? t.k_last - kbyte : kbyte;  // K step order
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
  auto substep = [&](auto zc, uint4 (&use)[NR], uint4 (&nxt)[NR], const char* src, int sl, bool reads,
                     const TileOps& lt, uint32_t fstage, int kbyte, int l0, int l1) {
    constexpr bool ZC = decltype(zc)::value;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1, fn = (g & 1) * 2;
      mma_pair<T, ZC, F16>(use[fm], use[FM + fn], acc[fm][fn]);
      __builtin_amdgcn_sched_barrier(0);
      if (l0 + g < l1) issue(lt, fstage, l0 + g, kbyte);
      if (reads) nxt[g] = frag(src, sl, g);
      __builtin_amdgcn_sched_barrier(0);
      mma_pair<T, ZC, F16>(use[fm], use[FM + fn + 1], acc[fm][fn + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::false_type acc_in{};
  const std::true_type acc_zero{};
  // kQuad: the epilogue's delta[o, j] (four consecutive j per 8 bytes), loaded while the tile's last
  // K steps run; element e of accumulator (i, j) in lane l is row 32 i + 8 (e / 4) + 4 (l / 32) +
  // e % 4 of the wave's 128 A rows and column 32 j + l % 32 of its 128 B rows. Here n_tokens = d_in
  // is a multiple of 128, so a wave's A rows are all inside or all outside G; loads outside either
  // matrix read a clamped address, and the epilogue skips their terms.
  uint2 dq[FM][FN][4];
  auto load_dq = [&](const TileOps& t) {
    if constexpr (MODE == kQuad) {
      const int64_t am = (int64_t)t.m0 + wm * 128 < n_tokens ? (int64_t)t.m0 + wm * 128 + 4 * fh : 0;
      const int64_t bn = (int64_t)t.n0 + wn * 128 + fr;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t o = min(bn + 32 * j, d_out - 1);  // row of this candidate's delta
        const uint2* drow =
            reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(delta) + ((int64_t)t.cand * d_out + o) * d_in + am);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) dq[i][j][q] = drow[8 * i + 2 * q];  // j index am + 32 i + 8 q
      }
    }
  };

  int G = blockIdx.x;
  if (G >= nblk) return;
  const int64_t cand_stride = MODE == kQuad ? epi.cand_stride : (int64_t)tiles_m * tiles_n;
  TileOps cur_t = tile_ops<T, MODE>(G, x, ld_x, delta, n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols, cand_stride);
  int par = 0;  // LDS buffer holding the tile's K stage 0
#pragma unroll
  for (int i = 0; i < 16; ++i) issue(cur_t, lds_base, i, 0);

  for (;;) {
    const int Gn = G + (int)gridDim.x;
    const bool has_next = Gn < nblk;
    const TileOps nxt_t =
        tile_ops<T, MODE>(has_next ? Gn : G, x, ld_x, delta, n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols,
                          cand_stride);
    const int k_steps = cur_t.k_steps;  // >= 2: K ranges are positive multiples of 128 elements
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
    substep(acc_zero, f0, f1, lds + par * kStageBytes, slot[1], true, cur_t,
            lds_base + (par ^ 1) * kStageBytes, KB,
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
      load_dq(cur_t);
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

    // element e of accumulator (i, j) in lane l: row 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 of the
    // wave's 128 A rows, column 32 j + l % 32 of its 128 B rows
    const int64_t am = (int64_t)cur_t.m0 + wm * 128 + 4 * fh, bn = (int64_t)cur_t.n0 + wn * 128 + fr;
    if constexpr (MODE == kStore) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t m = am + 32 * i + 8 * (e >> 2) + (e & 3), n = bn + 32 * j;
            if (m < n_tokens && n < d_out) epi.c[m * epi.ld_c + n] = acc[i][j][e];
          }
      __syncthreads();  // every wave has read the last stage
    } else {
      // kSse: sum of squares; kQuad: sum of acc * delta[o, j] (A row j, B row o; zero outside the
      // matrices). Each accumulator's 16 terms in float32, then accumulators, lanes and waves in
      // float64.
      double ss = 0.0;
      const bool rows_in = MODE != kQuad || am - 4 * fh < n_tokens;  // kQuad: wave-uniform
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float s32 = 0.f;
          if constexpr (MODE == kSse) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s32 = fmaf(acc[i][j][e], acc[i][j][e], s32);
          } else if (rows_in && bn + 32 * j < d_out) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f16x8 h = __builtin_bit_cast(f16x8, make_uint4(dq[i][j][q].x, dq[i][j][q].y, 0u, 0u));
#pragma unroll
              for (int r = 0; r < 4; ++r) s32 = fmaf(acc[i][j][4 * q + r], (float)h[r], s32);
            }
          }
          ss += (double)s32;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
      if (lane == 0) red[wave] = ss;
      __syncthreads();  // red is complete, and every wave has read the last stage
      if (threadIdx.x == 0) {
        double v = (red[0] + red[1]) + (red[2] + red[3]);
        // kQuad: doubled and unscaled, exactly
        if constexpr (MODE == kQuad) v = ldexp(v, 1 - (epi.gexp[0] + 2 * epi.dexp[cur_t.cand]));
        tile_sse[cur_t.idx] = v;
      }
    }
    if (!has_next) break;
    G = Gn;
    cur_t = nxt_t;
  }
}

}  // namespace

namespace {
// one persistent workgroup per compute unit (the tile order assumes 8 XCDs dealt round-robin);
// compute units of the current device, looked up once per device and thread
unsigned persistent_grid(int64_t nblk) {
  static thread_local int cus_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cus_of[dev];
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cus_of[dev] = cus;
  }
  return (unsigned)std::min<int64_t>(nblk, cus);
}
}  // namespace

hipError_t launch_error_sse(const void* x, int64_t ld_x, const void* delta, int dtype,
                            int64_t n_tokens, int64_t d_in, int64_t d_out, int n_cand,
                            double* tile_sse, hipStream_t st) {
  const int tiles_m = (int)((n_tokens + BM - 1) / BM);
  const int tiles_n = (int)((d_out + BN - 1) / BN);
  const int n_cols = tiles_n * n_cand;
  const unsigned grid = persistent_grid((int64_t)tiles_m * n_cols);
  const Epi epi = {};
  if (dtype == 1)
    hipLaunchKernelGGL((error_sse_kernel<uint16_t>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(delta),
                       n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse, epi);
  else
    hipLaunchKernelGGL((error_sse_kernel<float>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const float*>(x), ld_x, static_cast<const float*>(delta), n_tokens,
                       d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse, epi);
  return hipGetLastError();
}

hipError_t launch_gram_store(const uint16_t* xt, int64_t n_pad, int64_t d_in, float* g, hipStream_t st) {
  const int tiles = (int)((d_in + BM - 1) / BM);
  const unsigned grid = persistent_grid((int64_t)tiles * (tiles + 1) / 2);
  Epi epi = {};
  epi.c = g;
  epi.ld_c = d_in;
  // A = B = X^T ([d_in, n_pad], K = tokens): G[i, j] = sum_t x[t, i] x[t, j]
  hipLaunchKernelGGL((error_sse_kernel<uint16_t, kStore>), dim3(grid), dim3(kThreads), 0, st, xt, n_pad, xt,
                     d_in, n_pad, d_in, tiles, tiles, tiles, (double*)nullptr, epi);
  return hipGetLastError();
}

hipError_t launch_quad_sse(const uint16_t* g16, const int32_t* gexp, const uint16_t* delta16, const int32_t* dexp,
                           int n_cand, int64_t d_in, int64_t d_out, int64_t cand_stride, double* tile_sse,
                           hipStream_t st) {
  const int tiles_m = (int)((d_in + BM - 1) / BM);
  const int tiles_n = (int)((d_out + BN - 1) / BN);
  const int n_cols = tiles_n * n_cand;
  const unsigned grid = persistent_grid((int64_t)tiles_m * n_cols);
  Epi epi = {};
  epi.dexp = dexp;
  epi.gexp = gexp;
  epi.cand_stride = cand_stride;
  // A = G ([d_in, d_in], symmetric: its rows are its columns), B = the candidates' delta
  hipLaunchKernelGGL((error_sse_kernel<uint16_t, kQuad>), dim3(grid), dim3(kThreads), 0, st, g16, d_in, delta16,
                     d_in, d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse, epi);
  return hipGetLastError();
}

}  // namespace awq
