// Device helpers shared by the kernels that move operands global -> LDS with buffer DMA (the error
// GEMM, the block-level GEMM, the W4A16 many-token kernel): the s_waitcnt immediate, the DMA load,
// LDS addresses and raw buffer descriptors; and the tile order and LDS swizzle of the two 256 x 256
// GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9 encoding;
// expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// One 16-byte-per-lane buffer load that writes LDS directly (M0 = the wave's LDS destination, lane
// i's 16 bytes at M0 + 16 i). It is issued from inline assembly so that the compiler does not treat
// it as a possible writer of every later LDS read and wait for it there: the kernels that use it
// order their stages themselves (s_waitcnt vmcnt + barrier). The instruction has no register
// results. M0 is set in the same statement; nothing else in those kernels uses M0 (no LDS-DMA
// builtins, GWS or message sends), so the compiler holds no value there across it.
__device__ __forceinline__ void dma_load16(i32x4 rsrc, uint32_t lds_addr, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, num_records bytes; reads at byte
// offsets >= num_records return zero. Word 3 selects 32-bit data format, no swizzle.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)num_records);
  r.w = 0x00020000;
  return r;
}

// 16-byte slot of K chunk c in LDS row r of the 256 x 256 GEMMs is c ^ swz(r): their fragment
// reads (lane l: row l % 32, chunk 2 s + l / 32) then show no LDS bank-conflict cycles on gfx950.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Tile order of the persistent 256 x 256 GEMMs: the hardware deals workgroups round-robin to the
// 8 XCDs, so the 256 tiles processed together form a 16 x 16 super-block of (token tile, column)
// pairs, each XCD taking an 8 x 4 sub-block. In the last super-block row, h < 16 tiles high, each
// XCD takes all h rows of 2 adjacent columns, so that every column's panel is still read by one
// XCD's L2; super-blocks cut by the last column go column-major. Tile of linear index G: token
// tile tm, column col.
constexpr int kSuper = 16;
constexpr int kXcds = 8;
__device__ __forceinline__ void tile_of(int G, int tiles_m, int n_cols, int& tm, int& col) {
  const int n_sbm = (tiles_m + kSuper - 1) / kSuper, n_sbn = (n_cols + kSuper - 1) / kSuper;
  const int r = min(G / (kSuper * n_cols), n_sbm - 1);
  const int G1 = G - kSuper * r * n_cols;
  const int h = min(kSuper, tiles_m - kSuper * r);
  const int c = min(G1 / (h * kSuper), n_sbn - 1);
  const int G2 = G1 - c * h * kSuper;
  const int w = min(kSuper, n_cols - kSuper * c);
  if (h == kSuper && w == kSuper) {
    const int x = G2 % kXcds, q = G2 / kXcds;
    tm = kSuper * r + (x / 4) * 8 + q % 8;
    col = kSuper * c + (x % 4) * 4 + q / 8;
  } else if (w == kSuper) {
    const int x = G2 % kXcds, q = G2 / kXcds;  // q < 2 h
    tm = kSuper * r + q % h;
    col = kSuper * c + 2 * x + q / h;
  } else {
    tm = kSuper * r + G2 % h;
    col = kSuper * c + G2 / h;
  }
}

}  // namespace awq
