// Grouped GEMM of the unquantized bf16 experts, for gfx950.
//
// What it computes: the grouped matmuls of the pages' bf16 grouped_mm experts,
// the path the FP8 dispatch falls back to ("DeepGEMM experts selected on a
// model spanning multiple CUDA devices", the record's source: use
// experts_implementation='grouped_mm'), with the same sorted rows, row gather
// and epilogues as the quantized kernels: C[r, n] = sum_k A[a_row(r), k] *
// B[e, n, k] over bf16 operands with fp32 accumulation; then fp32 stores, the
// SwiGLU (h rounded once to bf16, the down projection's operand) or the
// routing-weighted bf16 scatter into the slot buffer.
//
// Layout: B is the expert weight [E, N, K] in operand order (prepare.hip): per
// 16-row group and 64-element K stage a 2 KB block of two 1 KB sub-steps, each
// the 64 lanes' 16-byte fragments in lane order, so a wave's weight load is 1 KB
// contiguous.  A rows are bf16 [rows, K] row-major, gathered through
// a_row_index / divisor.
//
// Tile: 256 weight rows x 128 sorted rows, 4 waves.  Wave w owns 64 weight rows
// (four 16-row groups) and all 128 rows of A (eight 16-row groups), so each lane
// ends with 4 consecutive weight rows of one A row per (group, A group) pair,
// from v_mfma_f32_16x16x32_bf16 with the weights as operand A; each A fragment
// read from LDS feeds four MFMAs.  In a paired (gate_up) tile, groups 2q and
// 2q + 1 of wave w are gate rows h0 + 32 w + 16 q .. + 16 and the matching up
// rows I + h0 + 32 w + 16 q .., so g and u of an output meet in one lane.  Per K stage of 64 elements the 128 gathered A rows (16 KB) are loaded
// once by the workgroup into registers and stored to a double-buffered LDS
// stage (16-byte chunks XOR-swizzled by row & 7, so the 16 rows a fragment read
// touches spread over the banks); weights go straight from global memory to
// registers, one stage ahead, each byte read by exactly one wave.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr int kWavesB = 4;
constexpr int kThreadsB = kWavesB * kWave;
constexpr int BMB = 128;            // sorted rows per tile
constexpr int BNB = 256;            // weight rows per tile
constexpr int kStageK = 64;         // K elements per stage (128 bytes of a row)
constexpr int kStageBytes = BMB * kStageK * 2;
constexpr int kMaxEB = 512;

constexpr int kRing = 3;            // A stages in LDS, weight stages in registers

struct SmemB {
  u32x4 stage[kRing][BMB * 8];  // [buffer][row * 8 + swizzled 16-byte chunk]
  int off[kMaxEB + 1];
  int tp[kMaxEB + 1];
  int scan[kThreadsB];
};
static_assert(sizeof(u32x4) * BMB * 8 == kStageBytes, "stage size");

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int EPI, bool PAIRED>
__global__ __launch_bounds__(kThreadsB, 2) void gemm_bf16_kernel(GemmParams p) {
  __shared__ SmemB sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int E = p.E, N = p.N, K = p.K;
  const int NT = PAIRED ? (N / 2) / (BNB / 2) : (N + BNB - 1) / BNB;
  const int KS = K / kStageK;
  const size_t row_bytes = (size_t)K * 2;

  const int total = build_tile_table<kThreadsB>(p.offsets, E, BMB, NT, sm.off, sm.tp, sm.scan);
  const uint8_t* A = p.a_codes;
  const uint8_t* B = p.b_codes;

  // A by LDS-DMA: DMA instruction q (< 4) of wave w copies rows 32 w + 8 q ..
  // + 8 of the stage, lane l taking row 32 w + 8 q + l / 8 into chunk position
  // l % 8; it reads logical chunk (l % 8) ^ (l / 8), so position c of row r
  // holds chunk c ^ (r & 7), the swizzle the fragment reads undo
  const int dma_rr = lane >> 3, dma_chunk = (lane & 7) ^ dma_rr;

  for (int t = xcd_virtual_block(); t < total; t += gridDim.x) {
    const TileCoord tc = locate_tile(t, E, BMB, NT, sm.off, sm.tp);
    // this lane's gathered A rows (rows past the expert's end repeat its last
    // row; their results are never stored)
    // (byte offsets from A, 32-bit: the host keeps A under 4 GiB)
    uint32_t a_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r_ld = min(tc.m0 + 32 * wave + 8 * q + dma_rr, tc.m_end - 1);
      const int arow = p.a_row_index ? p.a_row_index[r_ld] / p.a_row_div : r_ld;
      a_off[q] = (uint32_t)arow * (uint32_t)row_bytes + (uint32_t)dma_chunk * 16;
    }
    // this wave's 16-row weight groups 0..3 (a group past N, in the last tile of
    // an N that is not a multiple of 256, repeats the last group; its results
    // are never stored); the lane's fragment is 16 bytes at lane * 16
    // (group bases are wave-uniform, in scalar registers; the lane adds lane * 16)
    const uint8_t* wp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int grp;
      if (PAIRED)
        grp = ((q & 1) * (N / 2) + tc.n_tile * (BNB / 2) + 32 * wave + 16 * (q >> 1)) / 16;
      else
        grp = min((tc.n_tile * BNB + 64 * wave + 16 * q) / 16, N / 16 - 1);
      grp = __builtin_amdgcn_readfirstlane(grp);
      wp[q] = B + (((size_t)tc.e * (N / 16) + grp) * KS) * 2048;
    }
    const uint32_t wl = (uint32_t)lane * 16;

    v4f acc[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[q][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // stage s: 4 A DMAs into LDS buffer s % 3 and 8 weight loads into register
    // slot s % 3 (weights [substep ks][group q] at ks * 1024 of the stage block),
    // 12 vector-memory instructions per wave, issued two stages ahead
    u32x4 wr[kRing][8];
    auto issue = [&](int st, int b, u32x4(&w)[8]) {
      const uint32_t lds = lds_addr(&sm.stage[b][0]) + (uint32_t)(32 * wave) * 128;
#pragma unroll
      for (int q = 0; q < 4; ++q) lds_dma16_s(A, a_off[q] + (uint32_t)st * 128, lds + q * 1024);
      const size_t ow = (size_t)st * 2048;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = *(const u32x4*)(wp[q] + ow + wl);
        w[4 + q] = *(const u32x4*)(wp[q] + ow + 1024 + wl);
      }
    };
    __syncthreads();  // the previous tile's LDS reads are done
    issue(0, 0, wr[0]);
    issue(1, 1, wr[1]);

    // Every step issues (past the last stage it repeats stage KS - 1 into a
    // buffer and a register slot nobody reads again), so the same 12
    // instructions are in flight at every wait and the compiler's own waits for
    // the weight registers stay exact; only the MFMAs are skipped past KS.
    for (int s0 = 0; s0 < KS; s0 += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int st = s0 + j;
        // stage st has landed once only stage st + 1's instructions are still in
        // flight (the compiler's waits for the weight registers never wait less:
        // it does not count the DMAs)
        wait_vmcnt<12>();
        __syncthreads();  // every wave's part landed; every wave is done with stage st - 1
        issue(min(st + 2, KS - 1), (j + 2) % kRing, wr[(j + 2) % kRing]);
        if (st < KS) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int row = 16 * jj + l16;
              const int chunk = (ks * 4 + g) ^ (row & 7);
              const bf16x8 b = as_bf16x8(sm.stage[j][row * 8 + chunk]);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[q][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wr[j][4 * ks + q]), b, acc[q][jj], 0, 0,
                                                                    0);
            }
          }
        }
      }
    }
    wait_vmcnt<0>();  // the trailing repeats land before the next tile reuses the buffers

    // epilogue: lane holds weight rows 4 g .. 4 g + 3 of each group, A row 16 j + l16
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = tc.m0 + 16 * j + l16;
      if (r >= tc.m_end) continue;
      if constexpr (EPI == kEpiStoreF32) {
        if constexpr (PAIRED) {
          const int I = N / 2;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int h = tc.n_tile * (BNB / 2) + 32 * wave + 16 * q + 4 * g;
            *(v4f*)(p.c_f32 + (size_t)r * N + h) = acc[2 * q][j];
            *(v4f*)(p.c_f32 + (size_t)r * N + I + h) = acc[2 * q + 1][j];
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = tc.n_tile * BNB + 64 * wave + 16 * q + 4 * g;
            if (n < N) *(v4f*)(p.c_f32 + (size_t)r * N + n) = acc[q][j];
          }
        }
      } else if constexpr (EPI == kEpiSwiGLUQuant) {
        static_assert(PAIRED, "SwiGLU needs the paired gate/up tile");
        const int I = N / 2;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int h = tc.n_tile * (BNB / 2) + 32 * wave + 16 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = p.has_limit ? swiglu<true>(acc[2 * q][j][i], acc[2 * q + 1][j][i], p.limit)
                               : swiglu<false>(acc[2 * q][j][i], acc[2 * q + 1][j][i], p.limit);
          uint2 o;
          o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *(uint2*)((uint16_t*)p.h_codes + (size_t)r * I + h) = o;
        }
      } else {  // kEpiWeightedScatter
        const int slot = p.slot_of_row[r];
        const float wt = p.top_k_weights[slot];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = tc.n_tile * BNB + 64 * wave + 16 * q + 4 * g;
          if (n < N) {
            const v4f y = acc[q][j] * wt;
            uint2 o;
            o.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
            o.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
            *(uint2*)(p.slot_out + (size_t)slot * N + n) = o;
          }
        }
      }
    }
  }
}

template <int EPI, bool PAIRED>
hipError_t launch_bf16_epi(const GemmParams& p, int num_cus, hipStream_t stream) {
  const int NT = PAIRED ? (p.N / 2) / (BNB / 2) : (p.N + BNB - 1) / BNB;
  const long bound = ((long)(p.max_rows + BMB - 1) / BMB + p.E) * NT;
  long grid = 2L * num_cus;
  if (bound < grid) grid = bound;
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, PAIRED>), dim3((unsigned)grid), dim3(kThreadsB), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_bf16_epi<kEpiSwiGLUQuant, true>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_bf16_epi<kEpiWeightedScatter, false>(p, num_cus, stream);
  if (paired) return launch_bf16_epi<kEpiStoreF32, true>(p, num_cus, stream);
  return launch_bf16_epi<kEpiStoreF32, false>(p, num_cus, stream);
}

}  // namespace moe
