// Launchers of the gfx950 kernels, called by the C-ABI layer (moe_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Parameters of one grouped GEMM launch (see moe_grouped_gemm in include/moe.h).
struct GemmParams {
  const uint8_t* a_codes;
  const void* a_scales;
  const int32_t* a_row_index;
  int32_t a_row_div;
  int32_t a_rows;  // rows of each K-block plane of A ([K/128][a_rows][128] codes, [K/128][a_rows] scales)
  const int32_t* offsets;
  int32_t E;
  const uint8_t* b_codes;  // tiled weight codes (tile_layout.h)
  const void* b_scales;     // weight scales, [E][N/128][K/128]
  int32_t N;  // rows of B per expert
  int32_t K;
  int32_t max_rows;
  // epilogues
  float* c_f32;
  uint8_t* h_codes;
  void* h_scales;
  int32_t has_limit;
  float limit;
  uint16_t* slot_out;
  const float* top_k_weights;
  const int32_t* slot_of_row;
  // tile dispensing: NULL = static order, else 8 zeroed counters 128 bytes apart
  int32_t* sched;
  // non-NULL: the activation scales by sorted row, [K/128][max_rows] floats
  // (FP8) or [K/128][max_rows][4] bytes (MX), read instead of a_scales at the
  // gathered rows (tiled FP8 and MX kernels)
  const void* a_scales_sorted;
  // tiled FP8 and MX kernels: nonzero = the short remainder tiles of large
  // experts run last (phase 1 of the tile table), set by the launcher when a
  // launch has few rounds of tiles; zero = they stay beside their expert's
  // other m-tiles, whose weight tiles they then read from L2
  int32_t two_phase;
};

enum Epilogue { kEpiStoreF32 = 0, kEpiSwiGLUQuant = 1, kEpiWeightedScatter = 2 };

// Router in front of the route sort (see moe_route_topk in include/moe.h): the
// softmax top-k of each token's logits is written to ids / weights, and ids is
// then what the sort reads.  A launcher given a NULL RouterArgs* (or logits ==
// NULL) sorts the caller's ids as they are.
struct RouterArgs {
  const float* logits;  // [T, n_experts]
  int32_t n_experts;    // 1 .. 512
  int32_t renormalize;
  int32_t* ids;         // [T, k] out
  float* weights;       // [T, k] out
};

// Precomputed activation scales of the static scheme: row t's block scales
// (fp32 per 1x128 block, or UE8M0 bytes per 1x32 block) start `stride`
// elements after row t - 1's; stride 0 gives every row the same scales.  A
// launcher given a NULL StaticScales* quantizes dynamically.
struct StaticScales {
  const void* p;
  int32_t stride;
};

size_t route_sort_lds_bytes(int32_t E);
// Device workspace the sort of S slots needs (0 for the one-workgroup path).
size_t route_sort_ws_bytes(int32_t S, int32_t E);
// The route sort of ids [T, k] (S = T * k slots), preceded by the router when
// `router` is non-NULL (ids must then be router->ids).  slot_pos may be NULL.
hipError_t launch_route_sort(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets, int32_t* slot_pos,
                             int32_t* invalid_count, void* ws, hipStream_t stream);
// The same, also setting zero[0 .. n_zero) to 0.
hipError_t launch_route_sort_zero(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                                  int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets, int32_t* slot_pos,
                                  int32_t* invalid_count, void* ws, int32_t* zero, int32_t n_zero,
                                  hipStream_t stream);
// Whether S slots take the multi-workgroup sort (three launches, then the
// quantization as a launch of its own).
bool route_sort_multiblock(int32_t S);
// The (router and) route sort and the activation quantization of x [rows, H],
// in one launch for small batches, else one after the other; the first kernel
// also sets zero[0 .. n_zero) to 0 (the GEMMs' tile counters).  With the
// multi-workgroup sort and sorted_scales non-NULL, the scales are then also
// copied by sorted row into sorted_scales (launch_gather_scales).
hipError_t launch_route_sort_and_quant(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                                      int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets,
                                      int32_t* invalid_count, void* sort_ws, const uint16_t* x, int32_t rows,
                                      int32_t H, int fmt, uint8_t* codes, void* scales, int32_t* zero,
                                      int32_t n_zero, hipStream_t stream, void* sorted_scales = nullptr,
                                      const StaticScales* static_scales = nullptr);
// The router alone (no sort).
hipError_t launch_router_only(const RouterArgs& router, int32_t T, int32_t k, hipStream_t stream);
// static_scales non-NULL: the caller's block scales instead of the amax rule.
hipError_t launch_quant_act(const uint16_t* x, int32_t rows, int32_t H, int fmt, uint8_t* codes, void* scales,
                            hipStream_t stream, const StaticScales* static_scales = nullptr);
// The activation scales of T token rows ([H/128][T] fp32, or [H/128][T][4]
// UE8M0 bytes) copied by sorted row: dst [H/128][T * k], row r taking token
// sorted_slot[r] / k.
hipError_t launch_gather_scales(const void* scales, const int32_t* sorted_slot, int32_t k, int32_t T, int32_t H,
                                void* dst, hipStream_t stream);
// epi: Epilogue; paired: gate/up row pairing of B (used with kEpiSwiGLUQuant and
// optionally kEpiStoreF32 on the gate_up weight).
hipError_t launch_gemm_fp8_b128(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream);
// The same FP8 grouped GEMM for a few rows per expert: weights stream through
// registers, 16 rows per tile.
hipError_t launch_gemm_fp8_skinny(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream);
hipError_t launch_gemm_mx(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream);
// The unquantized bf16 grouped GEMM on the same tiles (A bf16 rows [a_rows][K],
// B bf16 tiled as in tile_layout.h with 2K-byte rows; the SwiGLU epilogue writes
// h as bf16 [max_rows, N/2] into h_codes).
hipError_t launch_gemm_bf16(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream);
hipError_t launch_combine(const uint16_t* slot_out, const int32_t* ids, int32_t T, int32_t k, int32_t H, int32_t E,
                          int32_t expert_begin, uint16_t* out, hipStream_t stream);
// Tile one weight [E, N, K] (nt, or nn = [E, K, N] when `nn`) into the layout
// of tile_layout.h; `paired` selects the gate/up pairing (N = 2I).
hipError_t launch_tile_weight_fp8(const uint8_t* src, bool nn, bool paired, int32_t E, int32_t N, int32_t K,
                                  uint8_t* dst, hipStream_t stream);
// Tile one MX weight (packed codes [E, N, K/2], UE8M0 scales [E, N, K/32]) into
// the MX layout of tile_layout.h (codes and scales each get their own array).
hipError_t launch_tile_weight_mx(const uint8_t* codes, const uint8_t* scales, bool paired, int32_t E, int32_t N,
                                 int32_t K, uint8_t* dst_codes, uint8_t* dst_scales, hipStream_t stream);
// bf16 weights [E, N, K] (nt) or [E, K, N] (nn) into the layout of
// tile_layout.h, each row taken as 2K bytes (K % 64 == 0).
hipError_t launch_tile_weight_bf16(const uint16_t* src, bool nn, bool paired, int32_t E, int32_t N, int32_t K,
                                   uint16_t* dst, hipStream_t stream);
hipError_t launch_transpose_u8(const uint8_t* in, uint8_t* out, int32_t batch, int32_t rows, int32_t cols,
                               hipStream_t stream);
// The matrix-core issue-rate probe (probe.hip): one workgroup of
// probe_threads() threads per CU; sink holds grid * probe_threads() floats,
// clk 2 * grid counters (shader-clock and 100 MHz ticks per workgroup).
int probe_threads();
int64_t probe_flops_per_mfma(int kind);
int probe_mfmas_per_round(int kind);
hipError_t launch_mfma_probe(int kind, int iters, int grid, float* sink, unsigned long long* clk,
                             hipStream_t stream);
hipError_t launch_clock_stamp(unsigned long long* out, int n, hipStream_t stream);
hipError_t launch_transpose_f32(const float* in, float* out, int32_t batch, int32_t rows, int32_t cols,
                                hipStream_t stream);

}  // namespace moe
