// LDS layouts of the grouped GEMM's operand tiles: where the buffer->LDS DMA
// puts each 16-byte chunk of a tile, and the per-lane offsets of the MFMA
// fragment reads.  Plain integer functions, usable from host code as well (a
// CPU test checks them against the MFMA operand layout and the 64-bank LDS).
#pragma once

#include <stdint.h>

namespace moe {

constexpr int BK = 32;        // K step of the 4-slot ring (bf16 elements)
constexpr int KCH = BK / 8;   // 16-byte chunks per K-contiguous row of that ring

// K-contiguous tiles hold rows of BKX bf16: BKX = 32 (64-byte rows, the K step
// of the 4-slot ring) or BKX = 64 (128-byte rows, the K block of the 5-region
// ring: each DMA row is one whole 128-byte cache line).
//   BKX = 32: four rows per 256-byte line of the 64 LDS banks.  The 16 lanes
//   of one ds_read_b128 phase read the same logical chunk of 16 consecutive
//   rows; XOR with (r / 4) % 4 puts them on 16 distinct 16-byte bank groups
//   (measured on gfx950: the XOR with (r / 2) % 4 that suits 32 banks loses
//   about 28% of the LDS read rate to conflicts).
//   BKX = 64: two rows per bank line; XOR with (r / 2) % 8 gives the 16 rows
//   of a phase the 16 pairs (r % 2, chunk position).
template <int BKX = BK>
__host__ __device__ __forceinline__ int kc_swz(int r) {
  static_assert(BKX == 32 || BKX == 64, "K-contiguous row length");
  return BKX == 32 ? (r >> 2) & 3 : (r >> 1) & 7;
}
// first element of logical 16-byte chunk `chunk` of row r
template <int BKX = BK>
__host__ __device__ __forceinline__ int kc_idx(int r, int chunk) {
  return r * BKX + ((chunk ^ kc_swz<BKX>(r)) << 3);
}
// MC tile [BKX][W] (rows = k): LDS position of logical 16-byte chunk c of row k (and back).
__host__ __device__ __forceinline__ int mc_chunk(int k, int c) { return c ^ ((k & 3) << 2); }

// KC operand: DMA instruction u of wave w covers 16-byte LDS chunks
// p = (w*N + u)*64 + lane, i.e. tile row p/(BKX/8), LDS chunk p%(BKX/8), which
// holds the logical k chunk (p%(BKX/8)) ^ swz(row).
template <int N, int BKX = BK>
__host__ __device__ __forceinline__ void kc_rows(int wave, int lane, int u, int& row, int& chunk) {
  constexpr int ch = BKX / 8;
  const int p = (wave * N + u) * 64 + lane;
  row = p / ch;
  chunk = (p % ch) ^ kc_swz<BKX>(row);
}

// MC operand of width W: chunk p -> k row p / (W/8), LDS chunk p % (W/8),
// holding logical chunk mc_chunk(row, p % (W/8)).
template <int N, int W>
__host__ __device__ __forceinline__ void mc_rows(int wave, int lane, int u, int& row, int& chunk) {
  const int p = (wave * N + u) * 64 + lane;
  row = p / (W / 8);
  chunk = mc_chunk(row, p % (W / 8));
}

// Byte offset of a lane's KC fragment for k16 sub-step s inside a 32-row
// block: lane l reads row l % 32, logical chunk 2 s + l / 32; the block's
// first row (a multiple of 16) does not change the swizzle.
template <int BKX = BK>
__host__ __device__ __forceinline__ uint32_t kc_lane_offset(int lane, int s) {
  const int r = lane & 31;
  return (uint32_t)(r * BKX * 2 + (((2 * s + (lane >> 5)) ^ kc_swz<BKX>(r)) << 4));
}

// Byte offset of a lane's first transposing read (ds_read_b64_tr_b16) of the
// MC fragment of 32-column block M (absolute within the tile, width W), k
// sub-step 0.  With g = l / 16, i = l % 16 the lane reads k = 8 (g / 2) + i / 4
// and column 32 M + 16 (g % 2) + 4 (i % 4), i.e. logical chunk 4 M + x,
// x = 2 (g % 2) + (i % 4) / 2, which sits at chunk 4 (M ^ (k % 4)) + x.  The
// four k rows one half-wave reads (k % 4 = 0..3) thus fall in four different
// 64-byte quarters of the 256-byte bank line: the 32 lanes cover all 64
// banks once.  The second read is 4 rows further (+ 8 W bytes), sub-step s
// adds 16 s rows.
template <int W>
__host__ __device__ __forceinline__ uint32_t mc_lane_offset(int lane, int M) {
  const int g = lane >> 4, i = lane & 15;
  const int x = 2 * (g & 1) + ((i & 3) >> 1);
  const int r = (i >> 2) & 3;
  const int rowpart = (8 * (g >> 1) + (i >> 2)) * W + 4 * (i & 1);
  const int c = 4 * ((M & ~3) | ((M & 3) ^ r)) + x;
  return (uint32_t)(2 * (rowpart + 8 * c));
}

// Epilogue staging: fp32 element (row r < 16, col c < 128) of a wave's 8 KB
// area; 32-column halves swap every four rows, so the row pairs one MFMA
// output register writes hit different banks.
__host__ __device__ __forceinline__ int stage_idx(int r, int c) {
  return r * 128 + (c ^ (((r >> 2) & 1) << 5));
}

}  // namespace moe
