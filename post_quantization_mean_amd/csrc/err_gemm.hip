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
// (candidates stacked along N), K = d_in. Tiles are 256 x 256 with a K step of 64 bytes
// (32 bf16 / 16 f32), four waves in a 2 x 2 arrangement, each wave a 128 x 128 sub-tile held as
// 4 x 4 accumulators of the 32x32 matrix-core instruction (v_mfma_f32_32x32x16_bf16 for bf16,
// v_mfma_f32_32x32x2_f32 for f32). Operands move global -> LDS with buffer loads that write LDS
// directly (16 bytes per lane); rows past the end of X or of a candidate's delta lie outside the
// buffer's range and read as zero, which adds nothing to a sum of squares. A ring of five LDS
// stages (all 160 KiB) keeps four K steps of loads in flight while one is consumed, enough to
// cover the latency of the L2 / Infinity-cache / HBM path. The 16-byte chunks of each LDS row
// are XOR-swizzled by row so that any 16 consecutive lanes of a fragment read hit distinct banks.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so block ids are first mapped to
// a contiguous logical range per XCD, then that range walks groups of 8 token tiles across all
// candidate-row tiles; the concurrently running tiles of an XCD then share operand K-slices in
// its L2.
#include "internal.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kTileM, BN = kTileN;
constexpr int KB = 64;                       // bytes of K per LDS row per stage (32 bf16 / 16 f32)
constexpr int kStageBytes = (BM + BN) * KB;  // 32 KiB
#ifndef AWQ_GEMM_STAGES
#define AWQ_GEMM_STAGES 5
#endif
constexpr int kStages = AWQ_GEMM_STAGES;     // ring of stages; kStages - 1 in flight
constexpr int kLdsBytes = kStages * kStageBytes;  // 160 KiB: all of a CU's LDS
constexpr int kLoadsPerStage = 8;            // buffer->LDS loads per wave per stage (4 A + 4 B)
#ifndef AWQ_GEMM_P1LOADS
#define AWQ_GEMM_P1LOADS 4
#endif
constexpr int kLoadsPhase1 = AWQ_GEMM_P1LOADS;  // of those, issued before the mid-step barrier
#ifndef AWQ_GEMM_GROUP_M
#define AWQ_GEMM_GROUP_M 8
#endif
constexpr int kGroupM = AWQ_GEMM_GROUP_M;  // token tiles per group of the tile order
constexpr int kXcds = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16-byte slot of K chunk c in a 64-byte LDS row r is c ^ swz(r). With this choice the fragment
// reads below (lane l: row l%32, chunk 2s + l/32) show no LDS bank-conflict cycles on gfx950
// (SQ_LDS_BANK_CONFLICT = 0); the other permutations tried stall 50-75% of LDS cycles.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9 encoding;
// expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Per-lane byte offsets of the 4 buffer->LDS loads that fill one operand's 256 x 64-byte stage
// slice. Wave w, load j covers LDS rows 16*(4j+w) .. +15; lane i of it fills row 16*(4j+w) + i/4,
// 16-byte slot i%4, which holds K chunk (i%4) ^ swz(row). The K position of the stage is added
// as the scalar offset at issue time.
__device__ __forceinline__ void load_offsets(int ld_bytes, int wave, int lane, int (&voff)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * j + wave) * 16 + (lane >> 2);
    voff[j] = row * ld_bytes + (((lane & 3) ^ swz(row)) << 4);
  }
}

// One 16-byte-per-lane buffer load that writes LDS directly (M0 = the wave's LDS destination).
// It is issued from inline assembly so that the compiler does not treat it as a possible
// writer of every later LDS read and wait for it there: this kernel synchronises the stages
// itself (s_waitcnt vmcnt + barrier). The instruction has no register results. M0 is set in
// the same statement; nothing else in this kernel uses M0 (no LDS-DMA builtins, GWS or
// message sends), so the compiler holds no value there across it.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma_load16(i32x4 rsrc, uint32_t lds_addr, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// lds_stage: LDS byte address of the operand's slice in the stage (wave-uniform).
__device__ __forceinline__ void load_stage(i32x4 rsrc, uint32_t lds_stage, const int (&voff)[4], int k_byte,
                                           int wave) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    dma_load16(rsrc, __builtin_amdgcn_readfirstlane(lds_stage + (4 * j + wave) * 16 * KB), voff[j], k_byte);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, num_records bytes; reads at byte
// offsets >= num_records return zero. Word 3 selects 32-bit data format, no swizzle.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane(num_records);
  r.w = 0x00020000;
  return r;
}

// One 16-byte fragment pair: a 32 x 32 x (16 bf16 | 8 f32) product into one accumulator.
template <typename T>
__device__ __forceinline__ void mma_pair(const uint4& a, const uint4& b, f32x16& c) {
  if constexpr (sizeof(T) == 2) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                0, 0, 0);
  } else {
    // four K=2 steps; lane half h contributes K index 4h+e of the 8-wide chunk pair in step e,
    // identically for both operands
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ void mma_all(const uint4 (&a)[4], const uint4 (&b)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) mma_pair<T>(a[fm], b[fn], acc[fm][fn]);
}

// The 8 fragment reads of one 32-byte K sub-step (two per 64-byte stage row): rows f*32 + lane%32
// of the wave's A and B strips; pa / pb already hold the lane's row and swizzled slot, so each read is an immediate
// offset of f * 32 rows.
__device__ __forceinline__ void read_frags(const char* pa, const char* pb, uint4 (&a)[4], uint4 (&b)[4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a[f] = *reinterpret_cast<const uint4*>(pa + f * 32 * KB);
    b[f] = *reinterpret_cast<const uint4*>(pb + f * 32 * KB);
  }
}

// Scheduling hint: spread n_ds fragment reads evenly among n_mfma matrix instructions.
#define SCHED_INTERLEAVE(n_mfma, n_ds)                                 \
  _Pragma("unroll") for (int _i = 0; _i < (n_ds); ++_i) {              \
    __builtin_amdgcn_sched_group_barrier(0x008, (n_mfma) / (n_ds), 0); \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 \
  }

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void error_sse_kernel(const T* __restrict__ x, int64_t ld_x, const T* __restrict__ delta,
                      int64_t n_tokens, int64_t d_in, int64_t d_out, int tiles_m, int tiles_n,
                      int n_cols, double* __restrict__ tile_sse) {
  constexpr int MPP = sizeof(T) == 2 ? 1 : 4;  // matrix instructions per fragment pair
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- block id -> (candidate, token tile, row tile)
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, jx = bid / kXcds;
  const int qx = nblk / kXcds, rx = nblk % kXcds;
  const int L = xcd * qx + min(xcd, rx) + jx;
  const int span = kGroupM * n_cols;
  const int first_m = (L / span) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_g = L % span;
  const int tm = first_m + in_g % gsize;
  const int col = in_g / gsize;  // candidate-major column tile
  const int cand = col / tiles_n;
  const int tn = col % tiles_n;

  // ---- buffer descriptors clipped to the valid rows of this tile
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, n_tokens - m0);
  const int rows_b = (int)min((int64_t)BN, d_out - n0);
  const int lda_bytes = (int)(ld_x * (int64_t)sizeof(T));
  const int row_bytes = (int)(d_in * (int64_t)sizeof(T));
  const T* a_base = x + m0 * ld_x;
  const T* b_base = delta + ((int64_t)cand * d_out + n0) * d_in;
  const i32x4 ra = make_rsrc(a_base, (rows_a - 1) * lda_bytes + row_bytes);
  const i32x4 rb = make_rsrc(b_base, (rows_b - 1) * row_bytes + row_bytes);
  int voff_a[4], voff_b[4];
  load_offsets(lda_bytes, wave, lane, voff_a);
  load_offsets(row_bytes, wave, lane, voff_b);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // The lane's fragment row and swizzled 16-byte slot for sub-steps 0 and 1 of a stage: row
  // 32f + lane%32 of the wave's strip, K chunk 2s + lane/32. swz(row) depends only on
  // lane % 16, because fragment rows start at multiples of 32.
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int ra_off = (wm * 128 + fr) * KB;
  const int rb_off = BM * KB + (wn * 128 + fr) * KB;
  const int slot0 = ((0 + fh) ^ swz(fr)) << 4;
  const int slot1 = ((2 + fh) ^ swz(fr)) << 4;
  const int k_steps = row_bytes / KB;  // >= 4: d_in is a positive multiple of 128

  // Pipeline over a ring of kStages LDS stages, one K step (two 32 x 32 x 16 sub-steps) each.
  // Per K step kt:
  //   phase 1: sub-step 0's MFMAs run while sub-step 1's fragments are read from LDS;
  //   wait until stage kt+1 has landed (the kStages-3 younger stages already issued may stay in
  //   flight) and barrier, after which every wave is also done reading stage kt-1;
  //   phase 2: sub-step 1's MFMAs run while the loads of stage kt+kStages-1 go into that freed
  //   buffer and stage kt+1's first fragments are read.
  // So kStages-1 stages of loads are in flight while the matrix cores work, and no fragment
  // read is waited on. The loop without loads at the end waits for everything instead.
  uint4 fa0[4], fb0[4], fa1[4], fb1[4];
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_address(lds));
  static_assert(kStages >= 4 && kStages <= 5, "the prologue fills kStages-1 <= 4 <= k_steps stages");
#pragma unroll
  for (int q = 0; q < kStages - 1; ++q) {
    load_stage(ra, lds_base + q * kStageBytes, voff_a, q * KB, wave);
    load_stage(rb, lds_base + q * kStageBytes + BM * KB, voff_b, q * KB, wave);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoadsPerStage));  // stage 0 has landed
  __syncthreads();
  read_frags(lds + ra_off + slot0, lds + rb_off + slot0, fa0, fb0);

  int kt = 0;
  int buf = 0;  // kt % kStages
  for (; kt + kStages - 1 < k_steps; ++kt) {
    char* cur = lds + buf * kStageBytes;
    const int nbuf = buf + 1 == kStages ? 0 : buf + 1;
    const int fbuf = buf == 0 ? kStages - 1 : buf - 1;
    char* nxt = lds + nbuf * kStageBytes;
    const uint32_t fre = lds_base + fbuf * kStageBytes;
    const int kload = (kt + kStages - 1) * KB;
    // The 8 loads of stage kt+kStages-1 (its buffer was freed at the previous barrier): load i
    // fills A slice i (i < 4) or B slice i-4.
    auto issue_load = [&](int i) {
      if (i < 4)
        dma_load16(ra, __builtin_amdgcn_readfirstlane(fre + (4 * i + wave) * 16 * KB), voff_a[i], kload);
      else
        dma_load16(rb, __builtin_amdgcn_readfirstlane(fre + BM * KB + (4 * (i - 4) + wave) * 16 * KB),
                   voff_b[i - 4], kload);
    };
    // phase 1: sub-step 0's MFMAs; between MFMA pairs, sub-step 1's fragment reads and the first
    // kLoadsPhase1 loads (spread out: a burst of loads would stall MFMA issue)
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1;
      mma_pair<T>(fa0[fm], fb0[(g & 1) * 2], acc[fm][(g & 1) * 2]);
      mma_pair<T>(fa0[fm], fb0[(g & 1) * 2 + 1], acc[fm][(g & 1) * 2 + 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (g < kLoadsPhase1) issue_load(g);
      if (g < 4)
        fa1[g] = *reinterpret_cast<const uint4*>(cur + ra_off + slot1 + g * 32 * KB);
      else
        fb1[g - 4] = *reinterpret_cast<const uint4*>(cur + rb_off + slot1 + (g - 4) * 32 * KB);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stages kt+1 .. kt+kStages-2 and the phase-1 loads are in flight; kt+1 must have landed
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 3) * kLoadsPerStage + kLoadsPhase1));
    __syncthreads();
    // phase 2: sub-step 1's MFMAs; between MFMA pairs, the remaining loads and stage kt+1's
    // sub-step-0 fragment reads
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int fm = g >> 1;
      mma_pair<T>(fa1[fm], fb1[(g & 1) * 2], acc[fm][(g & 1) * 2]);
      mma_pair<T>(fa1[fm], fb1[(g & 1) * 2 + 1], acc[fm][(g & 1) * 2 + 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (kLoadsPhase1 + g < kLoadsPerStage) issue_load(kLoadsPhase1 + g);
      if (g < 4)
        fa0[g] = *reinterpret_cast<const uint4*>(nxt + ra_off + slot0 + g * 32 * KB);
      else
        fb0[g - 4] = *reinterpret_cast<const uint4*>(nxt + rb_off + slot0 + (g - 4) * 32 * KB);
      __builtin_amdgcn_sched_barrier(0);
    }
    buf = nbuf;
  }
  for (; kt < k_steps - 1; ++kt) {
    char* cur = lds + buf * kStageBytes;
    const int nbuf = buf + 1 == kStages ? 0 : buf + 1;
    char* nxt = lds + nbuf * kStageBytes;
    read_frags(cur + ra_off + slot1, cur + rb_off + slot1, fa1, fb1);
    mma_all<T>(fa0, fb0, acc);
    SCHED_INTERLEAVE(16 * MPP, 8)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    read_frags(nxt + ra_off + slot0, nxt + rb_off + slot0, fa0, fb0);
    mma_all<T>(fa1, fb1, acc);
    SCHED_INTERLEAVE(16 * MPP, 8)
    buf = nbuf;
  }
  {  // K step k_steps-1
    char* cur = lds + buf * kStageBytes;
    read_frags(cur + ra_off + slot1, cur + rb_off + slot1, fa1, fb1);
    mma_all<T>(fa0, fb0, acc);
    SCHED_INTERLEAVE(16 * MPP, 8)
    mma_all<T>(fa1, fb1, acc);
  }

  // ---- epilogue: sum of squares of the 128 x 128 wave tile, float64
  // one accumulator tile row at a time, so only 64 values leave the accumulator registers at once
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const double v = (double)acc[i][j][e];
        ss = fma(v, v, ss);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  __syncthreads();  // every wave is done reading the last stage before LDS is reused
  double* red = reinterpret_cast<double*>(lds);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double t = (red[0] + red[1]) + (red[2] + red[3]);
    tile_sse[(int64_t)cand * tiles_m * tiles_n + (int64_t)tm * tiles_n + tn] = t;
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
  if (dtype == 1)
    hipLaunchKernelGGL(error_sse_kernel<uint16_t>, dim3((unsigned)nblk), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(delta),
                       n_tokens, d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse);
  else
    hipLaunchKernelGGL(error_sse_kernel<float>, dim3((unsigned)nblk), dim3(kThreads), 0, st,
                       static_cast<const float*>(x), ld_x, static_cast<const float*>(delta), n_tokens,
                       d_in, d_out, tiles_m, tiles_n, n_cols, tile_sse);
  return hipGetLastError();
}

}  // namespace awq
