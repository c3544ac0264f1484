// Layout of the prepared (tiled) expert weights and of the LDS operand rows,
// shared by the weight-preparation kernel and the grouped GEMMs.
//
// A weight [E, N, K] (N output rows, K = reduction) is stored as
//   [E][NT = ceil(N / 256)][KB = K / 128][16 row groups][2048 bytes],
// i.e. every 128-wide K block of a 256-row tile is one contiguous 32 KB piece,
// and every group of 16 tile rows is one contiguous 2 KB piece in the order
// the MFMA A operand wants it: [half h][lane l][16 bytes], where lane l holds
// tile row 16 * group + l % 16 and logical 16-byte chunk c = 4 h + l / 16 of its
// 128-byte row (K bytes [16 c, 16 c + 16)).  So a wave's fragment of a 16-row
// group is two contiguous 1 KB reads (lane l at l * 16 and 1024 + l * 16): one
// coalesced global load each, one LDS-DMA wave instruction each, and LDS reads
// with no bank conflicts and no address swizzle.  Rows past N are zero.
//
// Paired tiles (the gate_up weight, N = 2I): tile j holds the 128 gate rows
// [128 j, 128 j + 128) and the 128 matching up rows [I + 128 j, ...), interleaved
// 16 at a time (tile rows 32 p + [0, 16) gate, 32 p + [16, 32) up), so one tile
// yields a whole 128-wide block of SwiGLU outputs and g and u of the same output
// land in the same lane.
//
// MX weights (e2m1 packed two per byte along K, even k in the low nibble, a
// UE8M0 byte per 32 K) use the same tiling with 64-byte rows (128 K elements):
//   codes  [E][NT][K/128][16 row groups][1024 bytes], a group stored as
//          [lane l][16 bytes] = tile row 16 * group + l % 16, chunk l / 16 (K
//          elements [32 c, 32 c + 32)), the FP4 MFMA operand order,
//   scales [E][NT][K/128][256 tile rows][4 bytes]  (the 4 scale bytes of the row's
//                                                   128-wide K block, in order).
// MX activation / h scales are [K/128][rows][4 bytes] for the same reason: one
// dword per row per K block.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kTileN = 256;  // weight rows per tile
constexpr int kBlockK = 128; // bytes of K per block row (FP8: 128 elements)

// Physical 16-byte chunk position of logical chunk c in row r of an LDS
// activation stage (128-byte rows gathered by LDS-DMA) is c ^ swz(r).  An
// MFMA operand read has 16 lanes on 16 consecutive rows reading the same
// logical chunk; with this XOR their 16-byte reads are conflict-free on gfx950
// (measured with the LDS bank-conflict counter, which also showed that adding
// row bit 3 to the XOR makes every such read two-way conflicted).
__host__ __device__ __forceinline__ int swz(int row) { return row & 7; }

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
