// Layout of the prepared (tiled) expert weights and of the LDS operand rows,
// shared by the weight-preparation kernel and the grouped GEMMs.
//
// A weight [E, N, K] (N output rows, K = reduction) is stored as
//   [E][NT = ceil(N / 256)][KB = K / 128][256 tile rows][128 bytes],
// i.e. every 128-wide K block of a 256-row tile is one contiguous 32 KB piece,
// and every group of 8 tile rows is one contiguous 1 KB piece: one LDS-DMA
// wave instruction (64 lanes x 16 bytes) copies it straight into LDS.  Inside a
// 128-byte row the 16-byte chunks are permuted by swz(tile_row) so that the MFMA
// fragment reads from LDS are free of bank conflicts.  Rows past N are zero.
//
// Paired tiles (the gate_up weight, N = 2I): tile j holds the 128 gate rows
// [128 j, 128 j + 128) and the 128 matching up rows [I + 128 j, ...), interleaved
// 16 at a time (tile rows 32 p + [0, 16) gate, 32 p + [16, 32) up), so one tile
// yields a whole 128-wide block of SwiGLU outputs and g and u of the same output
// land in the same lane.
//
// MX weights (e2m1 packed two per byte along K, even k in the low nibble, a
// UE8M0 byte per 32 K) use the same tiling with 64-byte rows (128 K elements):
//   codes  [E][NT][K/128][256 tile rows][64 bytes], chunks permuted by swz4(row),
//   scales [E][NT][K/128][256 tile rows][4 bytes]  (the 4 scale bytes of the row's
//                                                   128-wide K block, in order).
// MX activation / h scales are [K/128][rows][4 bytes] for the same reason: one
// dword per row per K block.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kTileN = 256;  // weight rows per tile
constexpr int kBlockK = 128; // bytes of K per block row (FP8: 128 elements)

// Physical 16-byte chunk position of logical chunk c in tile row r.  Rows
// r..r+7 (and with 64 banks r..r+15) put the same logical chunk in distinct banks.
__host__ __device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Chunk permutation of a 64-byte (MX weight) row: rows r..r+7 with the same
// parity, and rows r..r+15 with the same r mod 4, get distinct chunks, which
// keeps 16-byte fragment reads free of bank conflicts with 32 or 64 banks.
__host__ __device__ __forceinline__ int swz4(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// Source row (within the expert) of tile row tr of tile nt.  Returns -1 for a
// padding row (plain tiles past N).
template <bool PAIRED>
__host__ __device__ __forceinline__ int tile_src_row(int nt, int tr, int N) {
  if (PAIRED) {
    const int I = N / 2;
    const int p = tr >> 5, within = tr & 31;
    const int h = nt * 128 + 16 * p + (within & 15);
    return within < 16 ? h : I + h;
  }
  const int r = nt * kTileN + tr;
  return r < N ? r : -1;
}

}  // namespace moe
