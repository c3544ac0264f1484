// Grouped GEMM for few rows per expert (decode batches), FP8 e4m3 x e4m3 with
// fp32 block scales (1x128 activations, 128x128 weights), for gfx950.
//
// What it computes: the same grouped matmul and epilogues as the tiled FP8
// kernel (the pages' grouped experts forward, "grouped_mm experts dispatch does
// not support activation_scheme='static'", sections "What it means" and
// "Source").
//
// Why a second kernel: with a handful of rows per expert the work is streaming
// the expert weights from HBM.  Here no weight goes through LDS: each of the 8
// waves of a workgroup owns 32 rows of the 256-row prepared weight tile and
// loads its MFMA fragments straight into VGPRs, in a ring of D register slots
// (one slot holds a K block's 4 KB of weight fragments and the activation
// fragment of a wave).  The ring runs on into the workgroup's next tile, so
// consecutive tiles do not drain the pipeline, and its loads are ordinary ones,
// so the compiler tracks them and waits exactly for the slot it consumes.  The
// weight loads carry the nontemporal hint: every weight byte is read once per
// launch, and hinted reads stream faster over the whole chip (a read-only
// probe on all 256 CUs: 7.2 against 6.0 TB/s; on the Qwen3-MoE decode layer
// the gate_up GEMM took 62 instead of 68.6 us, the down GEMM 33.5 instead of
// 37.9 us).  The launcher runs one slot (one K block ahead per wave) and one workgroup per
// CU: deeper rings (2 to 8 blocks, up to 256 KB of weights in flight per CU)
// were 2-5% slower on decode layers, and two or three workgroups per CU
// 10-16% slower; fewer concurrent streams stream faster on this part.
//
// Tile: 16 sorted rows x 256 weight rows.  MFMA A operand = 16 weight rows,
// B operand = the 16 gathered activation rows; each lane ends with 4
// consecutive outputs of one row.  A wave's two 16-row weight groups are the
// gate and up rows of the same 16 SwiGLU outputs in a paired tile, so the gate
// and up values of an output meet in one lane.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"
#include "tile_layout.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = kTileN;
constexpr int BK = kBlockK;
constexpr int BMS = 16;  // sorted rows per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxE = 512;

constexpr int kRowBatch = 16;  // tiles whose gathered row ids are fetched at once

struct Misc {
  int off[kMaxE + 1];
  int tp[kMaxE + 1];
  int scan[kThreads];
  float amax[kWaves][BMS];
  int arow[kRowBatch][BMS];    // activation row of each row of the next tiles
  int slot[kRowBatch][BMS];    // their flat slot (weighted scatter)
  float wt[kRowBatch][BMS];    // and routing weight (weighted scatter)
};

// Per-lane sources of one tile.
struct Src {
  bool valid;
  int e, n_tile, m0, m_end;
  const uint8_t* w;   // this tile's K block 0
  uint32_t swa;       // index of row group 0's weight scale at K block 0 (stride 1 per K block)
  uint32_t swb;       // the same for row group 1
  uint32_t sa;        // index of this lane's activation scale at K block 0 (stride a_rows)
  uint32_t a_off;     // this lane's activation row chunk offset in a K-block plane
};

// One K block of operands in registers.
struct Slot {
  int4 w[4];  // row group 0: chunks g, 4+g; row group 1: chunks g, 4+g
  int4 a[2];  // activation row: chunks g, 4+g
  float sa, swa, swb;
};

// Sources of tile t (an out-of-range t yields tile 0's, whose loads are
// harmless and never consumed); arow is this lane's activation row.
__device__ __forceinline__ Src make_src(const GemmParams& p, const Misc& misc, int t, int total, int NT, int KB,
                                        int NB, bool paired, int wave, int lane, int arow, int zero) {
  Src s;
  s.valid = t < total;
  if (!s.valid) t = 0;
  const TileCoord tc = locate_tile(t, p.E, BMS, NT, misc.off, misc.tp);
  s.e = tc.e;
  s.n_tile = tc.n_tile;
  s.m0 = tc.m0;
  s.m_end = tc.m_end;
  s.w = p.b_codes + ((size_t)tc.e * NT + tc.n_tile) * (size_t)KB * (BN * BK);
  int nba, nbb;
  if (paired) {
    nba = tc.n_tile;
    nbb = (p.N / 2) / 128 + tc.n_tile;
  } else {
    nba = nbb = min(tc.n_tile * 2 + (wave >= 4 ? 1 : 0), NB - 1);
  }
  // the zero keeps the (uniform) scale indices in VGPRs, so the scale loads are
  // vector loads: those are tracked in order, scalar ones are not, and waiting
  // on a scalar load would wait for every prefetched one
  s.swa = (uint32_t)(((size_t)tc.e * NB + nba) * KB) + (uint32_t)zero;
  s.swb = (uint32_t)(((size_t)tc.e * NB + nbb) * KB) + (uint32_t)zero;
  s.sa = (uint32_t)arow;
  s.a_off = (uint32_t)arow * BK + (uint32_t)((lane >> 4) << 4);
  return s;
}

// Fetch the per-row data of tiles t, t + G, ... (kRowBatch of them) into LDS:
// the activation row and, for the weighted scatter, the slot and its routing
// weight.  Loads whose results are waited for while the weight ring is in
// flight would drain it (the wait is by count, in order), so they are all made
// here, once per batch.
template <int EPI>
__device__ __forceinline__ void fetch_rows(const GemmParams& p, Misc& misc, int t, int G, int total, int NT) {
  __syncthreads();  // every wave is done reading the previous batch
  const int tid = threadIdx.x;
  if (tid < kRowBatch * BMS) {
    const int b = tid / BMS, i = tid % BMS;
    const int tb = t + b * G;
    int arow = 0, slot = 0;
    float wt = 0.0f;
    if (tb < total) {
      // a wave covers four tiles here, so the lookup stays per lane (the
      // shared locate_tile makes its result wave-uniform)
      int lo = 0, hi = p.E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (misc.tp[mid] <= tb) lo = mid; else hi = mid;
      }
      const int m_begin = misc.off[lo], m_end = misc.off[lo + 1];
      const int mt = (m_end - m_begin + BMS - 1) / BMS;
      int m_idx, n_idx;
      tile_position(tb - misc.tp[lo], mt, NT, m_idx, n_idx);
      const int r = min(m_begin + m_idx * BMS + i, m_end - 1);
      arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
      if constexpr (EPI == kEpiWeightedScatter) {
        slot = p.slot_of_row[r];
        wt = p.top_k_weights[slot];
      }
    }
    misc.arow[b][i] = arow;
    misc.slot[b][i] = slot;
    misc.wt[b][i] = wt;
  }
  __syncthreads();
}

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_slot_w(Slot& sl, const Src& s, int kb, const uint32_t (&w_off)[4]) {
  const uint8_t* wk = s.w + (size_t)kb * (BN * BK);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4i v = __builtin_nontemporal_load((const v4i*)(wk + w_off[q]));
    sl.w[q] = make_int4(v.x, v.y, v.z, v.w);
  }
}

__device__ __forceinline__ void load_slot_a(Slot& sl, const GemmParams& p, const Src& s, int kb) {
  const uint8_t* ak = p.a_codes + (size_t)kb * p.a_rows * BK + s.a_off;
  sl.a[0] = *(const int4*)ak;
  sl.a[1] = *(const int4*)(ak + 64);
  sl.sa = ((const float*)p.a_scales)[s.sa + (uint32_t)kb * (uint32_t)p.a_rows];
  sl.swa = ((const float*)p.b_scales)[s.swa + (uint32_t)kb];
  sl.swb = ((const float*)p.b_scales)[s.swb + (uint32_t)kb];
}

__device__ __forceinline__ void load_slot(Slot& sl, const GemmParams& p, const Src& s, int kb, const uint32_t (&w_off)[4]) {
  load_slot_w(sl, s, kb, w_off);
  load_slot_a(sl, p, s, kb);
}

template <int EPI, bool PAIRED>
__device__ __forceinline__ void epilogue(const GemmParams& p, Misc& misc, const Src& s, int slot, float wt,
                                         const v4f& acc0, const v4f& acc1, int wave, int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  const int N = p.N, I = N / 2;
  const int r = s.m0 + l16;
  if constexpr (EPI == kEpiStoreF32) {
    if (r < s.m_end) {
      if constexpr (PAIRED) {
        const int h = s.n_tile * 128 + 16 * wave + 4 * g;
        *(v4f*)(p.c_f32 + (size_t)r * N + h) = acc0;
        *(v4f*)(p.c_f32 + (size_t)r * N + I + h) = acc1;
      } else {
        const int n = s.n_tile * BN + 32 * wave + 4 * g;
        if (n < N) *(v4f*)(p.c_f32 + (size_t)r * N + n) = acc0;
        if (n + 16 < N) *(v4f*)(p.c_f32 + (size_t)r * N + n + 16) = acc1;
      }
    }
  } else if constexpr (EPI == kEpiSwiGLUQuant) {
    static_assert(PAIRED, "SwiGLU needs the paired gate/up layout");
    float h[4];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = p.has_limit ? swiglu<true>(acc0[i], acc1[i], p.limit) : swiglu<false>(acc0[i], acc1[i], p.limit);
      m = __builtin_fmaxf(m, __builtin_fabsf(h[i]));
    }
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    if (g == 0) misc.amax[wave][l16] = m;
    __syncthreads();
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) amax = __builtin_fmaxf(amax, misc.amax[w][l16]);
    __syncthreads();  // amax is reused by the next tile
    const float sc = fp8_block_scale(amax);
    const float inv = 1.0f / sc;
    if (r < s.m_end) {
      uint8_t* plane = p.h_codes + (size_t)s.n_tile * p.max_rows * 128;
      // h / sc as the activation rule's IEEE quotient (div_by_scale)
      *(uint32_t*)(plane + (size_t)r * 128 + 16 * wave + 4 * g) =
          e4m3x4(div_by_scale(h[0], sc, inv), div_by_scale(h[1], sc, inv), div_by_scale(h[2], sc, inv),
                 div_by_scale(h[3], sc, inv));
      if (wave == 0 && g == 0) ((float*)p.h_scales)[(size_t)s.n_tile * p.max_rows + r] = sc;
    }
  } else {  // kEpiWeightedScatter
    if (r < s.m_end) {
      const int n = s.n_tile * BN + 32 * wave + 4 * g;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v4f v = (q == 0 ? acc0 : acc1) * wt;
        if (n + 16 * q < N) {
          uint2 o;
          o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *(uint2*)(p.slot_out + (size_t)slot * N + n + 16 * q) = o;
        }
      }
    }
  }
}

template <int EPI, bool PAIRED, int D>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_skinny_kernel(GemmParams p) {
  __shared__ Misc misc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave offsets in SGPRs
  const int g = lane >> 4, l16 = lane & 15;
  const int E = p.E, N = p.N, KB = p.K / BK;
  const int NB = N / 128;
  const int NT = PAIRED ? (N / 2) / 128 : (N + BN - 1) / BN;
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));

  const int total = build_tile_table<kThreads>(p.offsets, E, BMS, NT, misc.off, misc.tp, misc.scan);
  const int G = gridDim.x;
  int t = xcd_virtual_block();
  if (t >= total) return;  // whole workgroup: no barrier follows

  // this lane's byte offsets inside a 32 KB K block of the tile: the wave's row
  // group 2 wave + q / 2, half q % 2 (logical chunk g or 4 + g); the tile stores
  // groups in operand order, so each load instruction reads 1 KB contiguous
  uint32_t w_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w_off[q] = (uint32_t)((2 * wave + (q >> 1)) * 2048 + (q & 1) * 1024 + lane * 16);

  fetch_rows<EPI>(p, misc, t, G, total, NT);
  Src cur = make_src(p, misc, t, total, NT, KB, NB, PAIRED, wave, lane, misc.arow[0][l16], zero);
  // the prologue issues the slots in the same order as the loop below: the
  // compiler waits by count and merges the two paths into the loop, so any
  // other order here would shorten the waits of every iteration
  Slot ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    load_slot(ring[j], p, cur, j, w_off);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int i = 0; t < total; t += G, ++i) {
    // this tile's scatter data, read before the batch can be refetched
    const int my_slot = misc.slot[i % kRowBatch][l16];
    const float my_wt = misc.wt[i % kRowBatch][l16];
    // the next tile's rows come from the LDS batch; when the next tile starts a
    // new batch it is refetched here (entry 0 = tile i + 1), which waits for the
    // loads in flight once per kRowBatch tiles
    if ((i + 1) % kRowBatch == 0) fetch_rows<EPI>(p, misc, t + G, G, total, NT);
    const Src nxt =
        make_src(p, misc, t + G, total, NT, KB, NB, PAIRED, wave, lane, misc.arow[(i + 1) % kRowBatch][l16], zero);
    v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < KB; kb0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        Slot& sl = ring[j];
        const v8i wa = v8i{sl.w[0].x, sl.w[0].y, sl.w[0].z, sl.w[0].w, sl.w[1].x, sl.w[1].y, sl.w[1].z, sl.w[1].w};
        const v8i wb = v8i{sl.w[2].x, sl.w[2].y, sl.w[2].z, sl.w[2].w, sl.w[3].x, sl.w[3].y, sl.w[3].z, sl.w[3].w};
        const v8i af = v8i{sl.a[0].x, sl.a[0].y, sl.a[0].z, sl.a[0].w, sl.a[1].x, sl.a[1].y, sl.a[1].z, sl.a[1].w};
        const v4f pa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        const v4f pb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb, af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc0 += pa * (sl.sa * sl.swa);
        acc1 += pb * (sl.sa * sl.swb);
        // refill the slot with the K block D steps ahead: later in this tile,
        // else the same position in the next tile (a valid, unused block past
        // the last tile); unconditional, so no register copies wait on loads
        const int kn = kb0 + j + D;
        const bool same = kn < KB;
        Src src;
        src.w = same ? cur.w : nxt.w;
        src.swa = same ? cur.swa : nxt.swa;
        src.swb = same ? cur.swb : nxt.swb;
        src.sa = same ? cur.sa : nxt.sa;
        src.a_off = same ? cur.a_off : nxt.a_off;
        // keep each slot's loads together and in ring order: the compiler
        // waits by count, so a load moved later would make the wait for it
        // drain the loads issued after it
        __builtin_amdgcn_sched_barrier(0);
        load_slot(sl, p, src, same ? kn : kn - KB, w_off);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    epilogue<EPI, PAIRED>(p, misc, cur, my_slot, my_wt, acc0, acc1, wave, lane);
    cur = nxt;
  }
}

template <int EPI, bool PAIRED, int D>
hipError_t launch_d(const GemmParams& p, int num_cus, hipStream_t stream) {
  const int NT = PAIRED ? (p.N / 2) / 128 : (p.N + BN - 1) / BN;
  const long bound = ((long)(p.max_rows + BMS - 1) / BMS + p.E) * NT;
  long grid = bound < num_cus ? bound : num_cus;
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((gemm_fp8_skinny_kernel<EPI, PAIRED, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// One K block in flight per wave (D = 1 divides every K / 128, so a tile ends
// on a ring boundary): measured faster than every deeper ring.
template <int EPI, bool PAIRED>
hipError_t launch_epi(const GemmParams& p, int num_cus, hipStream_t stream) {
  return launch_d<EPI, PAIRED, 1>(p, num_cus, stream);
}

}  // namespace

hipError_t launch_gemm_fp8_skinny(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_epi<kEpiSwiGLUQuant, true>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_epi<kEpiWeightedScatter, false>(p, num_cus, stream);
  if (paired) return launch_epi<kEpiStoreF32, true>(p, num_cus, stream);
  return launch_epi<kEpiStoreF32, false>(p, num_cus, stream);
}

}  // namespace moe
