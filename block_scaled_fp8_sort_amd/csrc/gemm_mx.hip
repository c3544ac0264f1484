// Grouped GEMM over expert-sorted rows for the MX format: e4m3 activations
// with a UE8M0 scale per 1x32 block times e2m1 weights (packed two per byte
// along K) with a UE8M0 scale per 1x32 block along K, for gfx950.
//
// What it computes: the same grouped matmul and epilogues as the FP8 kernel
// (the pages' grouped experts forward, "grouped_mm experts dispatch does not
// support activation_scheme='static'", sections "What it means" and "Source";
// FP4 weights arrive packed in int8, "DeepGEMM Mega MoE requires FP4-packed
// expert weights (dtype=int8)", section "Source").
//
// Design (gfx950): power-of-two block scales ride the MFMA itself:
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = e2m1 weights (format 4), B = e4m3
// activations (format 0), and per-lane E8M0 scale bytes, so the accumulators
// take the MFMA result directly (no VALU promotion).  Operand lane layout, as
// measured on the chip: an FP4 lane of group g (lane / 16) holds K elements
// [32 g, 32 g + 32) as 32 nibbles; an FP8 lane of group g holds K elements
// [16 g, 16 g + 16) in bytes 0-15 and [64 + 16 g, 64 + 16 g + 16) in bytes 16-31;
// the scale byte of lane group g applies to K elements [32 g, 32 g + 32).
// Tiles: 256 weight rows x BM tokens x 128 K (BM = 256, or 64 / 128 / 256 for an
// expert's last, partial m-tile, 192 for a gate_up expert's only one), eight
// waves (2 x 4), three or four LDS stages
// fed by LDS-DMA from the tiled weights (64-byte rows) and the K-block-major
// activations; persistent XCD-aware tile walk and staged, whole-row epilogue
// stores as in the FP8 kernel.
#include "gemm_common.h"
#include "internal.h"
#include "tile_layout.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = kTileN;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxE = 512;
constexpr int kWRow = 64;   // bytes of a 128-wide K block of one FP4 weight row
constexpr int kARow = 128;  // bytes of a 128-wide K block of one FP8 activation row

template <int BM>
struct StageBuf {
  uint8_t w[BN * kWRow];     // FP4 weight rows (16-row groups in operand order)
  uint8_t a[BM * kARow];     // FP8 activation rows (swz chunk order)
  uint8_t ws[BN * 4];        // weight scale bytes [row][4]
  uint8_t as[BM * 4];        // activation scale bytes [row][4]
  uint8_t spare[256];        // target of the waves with no scale to fetch
};

constexpr int kMaxBM = 256;

struct Misc {
  int off[kMaxE + 1];
  int tp[kMaxE + 1];
  uint16_t cnt[kMaxE + 2];
  int next[2];  // dispensed tile values, alternating per tile
  int2 scan[kThreads];
};

// LDS shared by the pipeline stages of every tile height: three stages of the
// 256-row layout (with the tile table, 159.8 of the 160 KiB), which also
// hold three of the 192-row one and four of the 128-row and of the 64-row
// one.  A third 256-row stage (two
// before) took Mega-MoE's gate_up GEMM from 3.32 to 3.28 ms.
constexpr int kStageArea = 3 * (int)sizeof(StageBuf<256>);
template <int BM>
constexpr int stages_for() {
  return kStageArea / (int)sizeof(StageBuf<BM>) < 4 ? kStageArea / (int)sizeof(StageBuf<BM>) : 4;
}
static_assert(stages_for<256>() == 3 && stages_for<64>() == 4, "stage area");

template <int BM>
struct TileSrc {
  static constexpr int A_LOADS = BM / 64;  // 1 KB activation DMAs per wave per stage
  const uint8_t* w_tile;    // tiled FP4 codes of (expert, n-tile), K block 0
  const uint8_t* ws_tile;   // tiled weight scales of (expert, n-tile), K block 0
  const uint8_t* a_codes;
  size_t a_plane;           // bytes per K-block plane of activation codes
  uint32_t a_off[A_LOADS];  // per-lane gathered row chunk offset
  const uint8_t* as_base;   // activation scale planes ([K/128][a_rows][4])
  size_t as_plane;
  uint32_t as_off;          // per-lane gathered row offset (waves < BM/64)
};

// DMA instruction idx (0 .. LOADS - 1) of the stage for block kb: 0-1 the
// weights (16 KB per K block, wave w copies 2 KB = 32 rows, contiguous), then
// BM / 64 activation gathers, last exactly one scale DMA per wave, so every wave
// has the same DMA count per stage.  idx is a compile-time constant after
// unrolling.
template <int BM>
__device__ __forceinline__ void issue_part(StageBuf<BM>* st, const TileSrc<BM>& src, int kb, int wave, int lane,
                                           int idx) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st));
  const uint32_t w = __builtin_amdgcn_readfirstlane(wave);
  constexpr uint32_t oW = 0, oA = BN * kWRow, oWS = oA + BM * kARow, oAS = oWS + BN * 4;
  if (idx < 2) {
    const uint8_t* wsrc = src.w_tile + (size_t)kb * (BN * kWRow) + w * 2048;
    lds_dma16_s(wsrc + idx * 1024, lane * 16, base + oW + w * 2048 + idx * 1024);
  } else if (idx < 2 + TileSrc<BM>::A_LOADS) {
    const int q = idx - 2;
    const uint8_t* plane = src.a_codes + (size_t)kb * src.a_plane;
    lds_dma16_s(plane, src.a_off[q], base + oA + (w * (BM / 8) + 8 * q) * kARow);
  } else if (w < BM / 64) {  // activation scales: 64 rows x 4 bytes per wave
    lds_dma4(src.as_base + (size_t)kb * src.as_plane + src.as_off, base + oAS + w * 256);
  } else if (w == BM / 64) {  // weight scales: 256 rows x 4 bytes, contiguous
    lds_dma16_s(src.ws_tile + (size_t)kb * (BN * 4), lane * 16, base + oWS);
  } else {
    lds_dma4(src.as_base + (size_t)kb * src.as_plane + src.as_off, base + oAS + BM * 4);
  }
}

template <int BM>
__device__ __forceinline__ void issue_stage(StageBuf<BM>* st, const TileSrc<BM>& src, int kb, int wave, int lane) {
  constexpr int LOADS = 2 + BM / 64 + 1;
#pragma unroll
  for (int idx = 0; idx < LOADS; ++idx) issue_part<BM>(st, src, kb, wave, lane, idx);
}

// 16 bytes = 32 FP4 values, K elements [32 g, 32 g + 32) of row l % 16 of the
// 16-row weight group grp, stored in operand order (lane l at l * 16)
__device__ __forceinline__ v8i frag_w(const uint8_t* w, int grp, int lane) {
  const int4 x = *(const int4*)(w + grp * 1024 + lane * 16);
  return v8i{x.x, x.y, x.z, x.w, 0, 0, 0, 0};
}
// 32 bytes = K elements [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of activation row tr
__device__ __forceinline__ v8i frag_a(const uint8_t* a, int tr, int g) {
  const int s = swz(tr);
  const int4 x0 = *(const int4*)(a + tr * kARow + ((g ^ s) << 4));
  const int4 x1 = *(const int4*)(a + tr * kARow + (((4 + g) ^ s) << 4));
  return v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
}

// One K block (see the FP8 kernel: the DMA always goes out, spread over the
// sub-tiles, repeating block KB - 1 past the end, so the wait count is
// constant).
template <int BM, int STAGES>
__device__ __forceinline__ void k_step(const StageBuf<BM>* cur, StageBuf<BM>* nxt, const TileSrc<BM>& src, int kb,
                                       int KB, int wave, int lane, v4f (&acc)[8][BM / 64]) {
  constexpr int WM = BM / 4;
  constexpr int TS = WM / 16;
  constexpr int LOADS = 2 + BM / 64 + 1;  // DMA instructions per wave per stage
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  wait_vmcnt<LOADS * (STAGES - 2)>();
  raw_barrier();
  const int kb_dma = min(kb + STAGES - 1, KB - 1);
  v8i bf[TS];
  int sa[TS];
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) {
    const int tr = wt * WM + ti * 16 + l16;
    bf[ti] = frag_a(cur->a, tr, g);
    sa[ti] = cur->as[tr * 4 + g];
  }
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    // the DMAs of block kb + STAGES - 1 go out spread over the sub-tiles (all at
    // once they would queue in the texture addresser ahead of the MFMAs)
#pragma unroll
    for (int idx = 0; idx < LOADS; ++idx)
      if (idx * 8 / LOADS == ni) issue_part<BM>(nxt, src, kb_dma, wave, lane, idx);
    const int tr = wn * 128 + ni * 16 + l16;
    const v8i af = frag_w(cur->w, wn * 8 + ni, lane);
    const int sw = cur->ws[tr * 4 + g];
#pragma unroll
    for (int ti = 0; ti < TS; ++ti)
      acc[ni][ti] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[ti], acc[ni][ti], 4, 0, 0, sw, 0, sa[ti]);
  }
}

// One tile of BM sorted rows [m0, min(m0 + BM, m_end)) of expert e against
// n-tile n_tile, through a ring of STAGES LDS stages carved out of `area`.
template <int BM, int EPI, bool PAIRED>
__device__ __forceinline__ void run_tile(const GemmParams& p, uint8_t* area, int* srow, int e, int n_tile, int m0,
                                         int m_end) {
  constexpr int STAGES = stages_for<BM>();
  constexpr int WM = BM / 4;
  constexpr int TS = WM / 16;
  static_assert(TS >= 1 && BM <= 256, "64 <= BM <= 256");
  StageBuf<BM>* st = reinterpret_cast<StageBuf<BM>*>(area);

  // the thread id is made opaque per tile so that the per-lane address math of
  // each tile height stays inside its tile instead of being hoisted out of the
  // tile loop for all heights at once (which would spill registers)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int N = p.N, KB = p.K / 128;
  const int I = N / 2;
  const int NT = PAIRED ? I / 128 : (N + BN - 1) / BN;

  TileSrc<BM> src;
  const size_t tile = (size_t)e * NT + n_tile;
  src.w_tile = p.b_codes + tile * (size_t)KB * (BN * kWRow);
  src.ws_tile = (const uint8_t*)p.b_scales + tile * (size_t)KB * (BN * 4);
  src.a_codes = p.a_codes;
  src.a_plane = (size_t)p.a_rows * kARow;
#pragma unroll
  for (int q = 0; q < TileSrc<BM>::A_LOADS; ++q) {
    const int tr = wave * (BM / 8) + 8 * q + (lane >> 3);
    const int r = min(m0 + tr, m_end - 1);
    const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
    src.a_off[q] = (uint32_t)arow * kARow + (uint32_t)(((lane & 7) ^ swz(tr)) << 4);
  }
  {
    const int tr = (wave % (BM / 64 > 0 ? BM / 64 : 1)) * 64 + lane;  // rows of the waves that load scales
    const int r = min(m0 + min(tr, BM - 1), m_end - 1);
    if (p.a_scales_sorted) {  // by sorted row: the tile's scales are contiguous
      src.as_base = (const uint8_t*)p.a_scales_sorted;
      src.as_plane = (size_t)p.max_rows * 4;
      src.as_off = (uint32_t)r * 4;
    } else {
      const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
      src.as_base = (const uint8_t*)p.a_scales;
      src.as_plane = (size_t)p.a_rows * 4;
      src.as_off = (uint32_t)arow * 4;
    }
  }

  v4f acc[8][TS];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni)
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) acc[ni][ti] = v4f{0.f, 0.f, 0.f, 0.f};

  __syncthreads();
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue_stage<BM>(&st[s], src, min(s, KB - 1), wave, lane);
  for (int kb = 0; kb < KB; kb += STAGES) {
#pragma unroll
    for (int j = 0; j < STAGES; ++j)
      if (kb + j < KB) k_step<BM, STAGES>(&st[j], &st[(j + STAGES - 1) % STAGES], src, kb + j, KB, wave, lane, acc);
  }
  wait_vmcnt<0>();

  if constexpr (EPI == kEpiStoreF32) {
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      const int r = m0 + wt * WM + ti * 16 + l16;
      if (r < m_end) {
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
          int n;
          if constexpr (PAIRED) {
            const int h = n_tile * 128 + 16 * (wn * 4 + (ni >> 1)) + 4 * g;
            n = (ni & 1) ? I + h : h;
          } else {
            n = n_tile * BN + wn * 128 + ni * 16 + 4 * g;
          }
          if (n < N) *(v4f*)(p.c_f32 + (size_t)r * N + n) = acc[ni][ti];
        }
      }
    }
  } else if constexpr (EPI == kEpiSwiGLUQuant) {
    static_assert(PAIRED, "SwiGLU needs the paired gate/up layout");
    // this wave's 64 outputs of the tile's 128 are the 32-wide MX blocks 2 wn and
    // 2 wn + 1, each made of pairs q = 2b and 2b + 1: the block amax needs only
    // this wave (xor over the four lane groups)
    // codes and scale bytes are staged (after this barrier every wave is past
    // the K loop) and stored as whole rows
    static_assert(BM * (kHPitch + 4) <= kStageArea, "h staging");
    uint8_t* sstage = area + BM * kHPitch;  // [BM][4] scale bytes
    __syncthreads();
    // h, computed once into the gate's accumulators
    auto swiglu_all = [&](auto lim) {
      constexpr bool LIM = decltype(lim)::value;
#pragma unroll
      for (int ti = 0; ti < TS; ++ti)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[2 * q][ti][i] = swiglu<LIM>(acc[2 * q][ti][i], acc[2 * q + 1][ti][i], p.limit);
    };
    if (p.has_limit) swiglu_all(std::true_type{});
    else swiglu_all(std::false_type{});
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      const int tt = wt * WM + ti * 16 + l16;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float m = 0.0f;
#pragma unroll
        for (int q = 2 * b; q < 2 * b + 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(acc[2 * q][ti][i]));
        m = wave_max_xor(m, 16);
        m = wave_max_xor(m, 32);
        const int ex = mx_block_exponent(m);
#pragma unroll
        for (int q = 2 * b; q < 2 * b + 2; ++q) {
          const v4f h = acc[2 * q][ti];
          *(uint32_t*)(area + tt * kHPitch + 16 * (wn * 4 + q) + 4 * g) =
              e4m3x4(__builtin_ldexpf(h[0], -ex), __builtin_ldexpf(h[1], -ex), __builtin_ldexpf(h[2], -ex),
                     __builtin_ldexpf(h[3], -ex));
        }
        if (g == 0) sstage[tt * 4 + wn * 2 + b] = (uint8_t)(ex + 127);
      }
    }
    __syncthreads();
    copy_out_h_codes<BM>(p, area, n_tile, m0, m_end, tid);
    if (tid < BM && m0 + tid < m_end)
      *(uint32_t*)((uint8_t*)p.h_scales + ((size_t)n_tile * p.max_rows + m0 + tid) * 4) =
          *(const uint32_t*)(sstage + tid * 4);
  } else {  // kEpiWeightedScatter
    static_assert(BM * kOutPitch <= kStageArea, "output staging");
    scatter_rows_staged<BM>(p, area, srow, acc, n_tile * 256, m0, m_end, tid);
  }
}

// Persistent kernel; the last, partial m-tile of an expert runs at the
// smallest height of {64, 128, 256} that covers it (on the gate_up GEMM an
// expert's only m-tile at 192 rows when that covers it), and tiles come from the
// two-phase, longest-first table (as in the FP8 kernel).
template <int EPI, bool PAIRED>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t area[kStageArea];
  __shared__ __attribute__((aligned(16))) Misc misc;
  int* const srow = reinterpret_cast<int*>(misc.scan);  // scatter epilogue scratch (scan is free after the table)
  const int E = p.E, N = p.N;
  const int NT = PAIRED ? (N / 2) / 128 : (N + BN - 1) / BN;
  const int total = build_tile_table2<kThreads>(p.offsets, E, NT, misc.off, misc.tp, misc.cnt, misc.scan,
                                                  p.two_phase != 0);
  const int G = gridDim.x;
  auto run = [&](int t) {
    const TileCoord tc = locate_tile2(t, E, NT, misc.off, misc.tp, misc.cnt, p.two_phase != 0);
    const int left = tc.m_end - tc.m0;
    if constexpr (PAIRED) {
      // an expert whose only m-tile has 129-192 rows: 192-row tile (not the
      // last m-tile of an expert with full ones, which would run ahead of its
      // group's 256-row tiles and make them fetch its weight tile again)
      if (left > 128 && left <= 192 && tc.m0 == __builtin_amdgcn_readfirstlane(misc.off[tc.e])) {
        run_tile<192, EPI, PAIRED>(p, area, srow, tc.e, tc.n_tile, tc.m0, tc.m_end);
        return;
      }
    }
    if (left > 128)
      run_tile<256, EPI, PAIRED>(p, area, srow, tc.e, tc.n_tile, tc.m0, tc.m_end);
    else if (left > 64)
      run_tile<128, EPI, PAIRED>(p, area, srow, tc.e, tc.n_tile, tc.m0, tc.m_end);
    else
      run_tile<64, EPI, PAIRED>(p, area, srow, tc.e, tc.n_tile, tc.m0, tc.m_end);
  };
  // tiles come from the per-XCD dispensers when counters are given (the next
  // tile is grabbed at the start of the current one and handed to every wave
  // through LDS after it; a workgroup whose dispenser is exhausted takes from
  // another XCD's), else in the fixed round-robin order
  const bool dyn = p.sched != nullptr;
  const int tid = threadIdx.x;
  Dispenser d{};
  int td = 0;
  if (dyn) {
    d = make_dispenser(p.sched, total, G);
    if (tid == 0) misc.next[0] = take_tile(d, grab_tile(d));
    __syncthreads();
    td = __builtin_amdgcn_readfirstlane(misc.next[0]);  // the same in every lane
  }
  const int vb = xcd_virtual_block();
  for (int i = 1;; ++i) {
    const int t = dyn ? td : vb + (i - 1) * G;
    if (t < 0 || t >= total) {
      if (dyn && tid == 0) retire(d, G);
      break;
    }
    unsigned long long v_next = 0;
    if (dyn && tid == 0) v_next = grab_tile(d);
    run(t);
    if (dyn) {
      if (tid == 0) misc.next[i & 1] = take_tile(d, v_next);
      __syncthreads();
      td = __builtin_amdgcn_readfirstlane(misc.next[i & 1]);
    }
  }
}

template <int EPI, bool PAIRED>
hipError_t launch_one(const GemmParams& p, int num_cus, hipStream_t stream) {
  auto kern = gemm_mx_kernel<EPI, PAIRED>;
  const int NT = PAIRED ? (p.N / 2) / 128 : (p.N + BN - 1) / BN;
  const long bound = ((long)(p.max_rows + kMaxBM - 1) / kMaxBM + p.E) * NT;
  long grid = bound < num_cus ? bound : num_cus;
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  // the remainder tiles always run last: keeping them beside their expert's
  // other m-tiles made Mega-MoE's gate_up GEMM 2% slower
  GemmParams q = p;
  q.two_phase = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_one<kEpiSwiGLUQuant, true>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_one<kEpiWeightedScatter, false>(p, num_cus, stream);
  if (paired) return launch_one<kEpiStoreF32, true>(p, num_cus, stream);
  return launch_one<kEpiStoreF32, false>(p, num_cus, stream);
}

}  // namespace moe
