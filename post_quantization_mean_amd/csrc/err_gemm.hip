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
// (candidates stacked along N), K = d_in. Tiles are 256 x 256 with a K step of 128 bytes
// (64 bf16 / 32 f32), four waves in a 2 x 2 arrangement, each wave a 128 x 128 sub-tile held as
// 8 x 8 accumulators of the 16x16 matrix-core instruction (v_mfma_f32_16x16x32_bf16 for bf16,
// v_mfma_f32_16x16x4_f32 for f32). Operands move global -> LDS with buffer loads that write LDS
// directly (16 bytes per lane); rows past the end of X or of a candidate's delta lie outside the
// buffer's range and read as zero, which adds nothing to a sum of squares. Two LDS stages hold
// the next K step while the current one is consumed. The 16-byte chunks of each 128-byte LDS row
// are XOR-swizzled by row so that the 16 lanes of a fragment read hit distinct banks.
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
constexpr int KB = 128;                      // bytes of K per LDS row per stage
constexpr int kStageBytes = (BM + BN) * KB;  // 64 KiB
constexpr int kLdsBytes = 2 * kStageBytes;   // 128 KiB of the 160 KiB per CU
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Issue the 8 buffer->LDS loads that fill one operand's 256 x 128-byte stage slice.
// Wave w, load j covers LDS rows 8*(4j+w) .. +7; lane i of it fills row 8*(4j+w) + i/8,
// 16-byte slot i%8, which holds K chunk (i%8) ^ swz(row).
template <int ESZ>
__device__ __forceinline__ void load_stage(__amdgpu_buffer_rsrc_t rsrc, char* lds_stage, int ld_bytes,
                                           int k_byte, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rb = 4 * j + wave;
    const int row = rb * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    const int voff = row * ld_bytes + k_byte + chunk * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_stage + rb * 8 * KB), 16, voff, 0, 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ void mma_chunk(const uint4 (&a)[8], const uint4 (&b)[8], f32x4 (&acc)[8][8]) {
#pragma unroll
  for (int fm = 0; fm < 8; ++fm) {
#pragma unroll
    for (int fn = 0; fn < 8; ++fn) {
      if constexpr (sizeof(T) == 2) {
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[fm]),
                                                              __builtin_bit_cast(bf16x8, b[fn]),
                                                              acc[fm][fn], 0, 0, 0);
      } else {
        // four K=4 steps; lane group g contributes K index 4g+e of the 16-wide chunk in step e,
        // identically for both operands
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[fm].x), __uint_as_float(b[fn].x), acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[fm].y), __uint_as_float(b[fn].y), acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[fm].z), __uint_as_float(b[fn].z), acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[fm].w), __uint_as_float(b[fn].w), acc[fm][fn], 0, 0, 0);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void error_sse_kernel(const T* __restrict__ x, int64_t ld_x, const T* __restrict__ delta,
                      int64_t n_tokens, int64_t d_in, int64_t d_out, int tiles_m, int tiles_n,
                      int n_cols, double* __restrict__ tile_sse) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

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
  const int ldb_bytes = (int)(d_in * (int64_t)sizeof(T));
  const int row_bytes = (int)(d_in * (int64_t)sizeof(T));
  const T* a_base = x + m0 * ld_x;
  const T* b_base = delta + ((int64_t)cand * d_out + n0) * d_in;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a_base, 0, (rows_a - 1) * lda_bytes + row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)b_base, 0, (rows_b - 1) * ldb_bytes + row_bytes, 0x00020000);


  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15;  // row within a 16-row fragment
  const int fg = lane >> 4;  // 16-byte K chunk within a 64-byte sub-step
  const int k_steps = row_bytes / KB;

  load_stage<sizeof(T)>(ra, lds, lda_bytes, 0, wave, lane);
  load_stage<sizeof(T)>(rb, lds + BM * KB, ldb_bytes, 0, wave, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int kt = 0; kt < k_steps; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < k_steps) {
      char* nxt = lds + (st ^ 1) * kStageBytes;
      load_stage<sizeof(T)>(ra, nxt, lda_bytes, (kt + 1) * KB, wave, lane);
      load_stage<sizeof(T)>(rb, nxt + BM * KB, ldb_bytes, (kt + 1) * KB, wave, lane);
    }
    const char* As = lds + st * kStageBytes;
    const char* Bs = As + BM * KB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a[8], b[8];
      const int chunk = s * 4 + fg;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int ra_row = wm * 128 + f * 16 + fr;
        const int rb_row = wn * 128 + f * 16 + fr;
        a[f] = *reinterpret_cast<const uint4*>(As + ra_row * KB + ((chunk ^ swz(ra_row)) << 4));
        b[f] = *reinterpret_cast<const uint4*>(Bs + rb_row * KB + ((chunk ^ swz(rb_row)) << 4));
      }
      mma_chunk<T>(a, b, acc);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads of the next stage have landed
    __syncthreads();
  }

  // ---- epilogue: sum of squares of the 128 x 128 wave tile, float64
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double v = (double)acc[i][j][e];
        ss = fma(v, v, ss);
      }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
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
