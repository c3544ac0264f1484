// Grouped GEMM over expert-sorted rows, FP8 e4m3 x e4m3 with fp32 block scales
// (1x128 on the activations, 128x128 on the weights), for gfx950.
//
// What it computes: for expert e and sorted row r of its range,
// C[r, n] = sum_i A[a_row(r), i] * B[e, n, i] with dequantized operands (code
// times block scale), then one of the epilogues of moe_grouped_gemm.  This is
// the gate_up ("L1") and down ("L2") grouped matmul of the pages' grouped
// experts forward ("grouped_mm experts dispatch does not support
// activation_scheme='static'", sections "What it means" and "Source"), with the
// token-row gather (rows picked by perm // k) folded into the operand loads.
//
// Design (gfx950, wave64):
//  * MFMA A operand = weight rows (output features n), MFMA B operand = the
//    gathered activation rows (tokens).  In v_mfma_f32_16x16x128_f8f6f4's
//    output each lane holds 4 consecutive n of one token, so the activation
//    scale of a 128-wide K block is one value per lane and the weight scale is
//    one value per 16-row sub-tile.
//  * fp32 block scales cannot ride the MFMA's E8M0 scale operands, so each
//    128-wide K block is one MFMA with a zero accumulator (the block's partial
//    sum P of code products, exact products and fp32 sums) followed by
//    acc += P * (s_act * s_w) on the VALU (one FMA per output per K block).
//  * Workgroup tile 256 (n) x BM (tokens) x 128 (K), four waves as 2 x 2, each
//    128 n x BM/2 tokens.  Operands move global -> LDS by LDS-DMA
//    (global_load_lds_dwordx4): every lane supplies its own global address, so
//    the row gather costs nothing; the LDS row layout swizzles 16-byte chunks by
//    (row >> 1) & 7, which keeps the MFMA fragment reads free of bank conflicts.
//    Three stages are in flight.
//  * Persistent grid: each workgroup reads the expert offsets, builds the tile
//    table (experts x n-tiles x m-tiles, m fastest) in LDS, and walks tiles
//    with a stride of the grid size.  Workgroup ids are remapped so that
//    consecutive tiles land on the same XCD (dispatch is round-robin over the
//    8 XCDs), which keeps a weight tile shared by an expert's m-tiles in that
//    XCD's L2.  Partial m-tiles are masked; no host-visible counts are needed.
//  * Paired mode (gate_up weight): the 256 rows of an n-tile are 128 gate rows
//    and the 128 matching up rows, interleaved 16 at a time, so the SwiGLU
//    epilogue finds g and u of the same output in the same lane, and one tile
//    owns a whole 128-wide block of h for its quantization.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kMaxE = 512;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// One pipeline stage in LDS: 256 weight rows and BM activation rows of one
// 128-byte K block, and the activation scales of that block (one 256-byte DMA
// per wave; wave w's first BM/4 entries are rows [w*BM/4, (w+1)*BM/4)).  Each
// stage is its own __shared__ object so the compiler can tell a DMA into one
// stage from the fragment reads of another and does not wait on it.
template <int BM>
struct StageBuf {
  uint8_t w[BN * BK];
  uint8_t a[BM * BK];
  float s[4 * 64];
};

// Tile table and epilogue exchange.
template <int BM>
struct Misc {
  int off[kMaxE + 1];
  int tp[kMaxE + 1];
  int scan[kThreads];
  float amax[2][BM];
};

// Row of B (within the expert) held by tile row tr of n-tile nt.
template <bool PAIRED>
__device__ __forceinline__ int b_row(int nt, int tr, int N) {
  if constexpr (PAIRED) {
    const int I = N / 2;
    const int p = tr >> 5, within = tr & 31;
    const int h = nt * 128 + 16 * p + (within & 15);
    return within < 16 ? h : I + h;
  } else {
    return min(nt * BN + tr, N - 1);
  }
}

// 32 bytes of K (logical chunks 2g and 2g+1 of the 128-byte row) of LDS row tr.
__device__ __forceinline__ v8i lds_frag(const uint8_t* region, int tr, int g) {
  const int s = swz(tr);
  const int4 x0 = *(const int4*)(region + tr * BK + (((2 * g) ^ s) << 4));
  const int4 x1 = *(const int4*)(region + tr * BK + (((2 * g + 1) ^ s) << 4));
  return v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
}

// Barrier without a memory fence: the waits before it are explicit (vmcnt for
// the DMAs this wave issued, lgkmcnt for its LDS writes); the empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane DMA sources of one tile (fixed for the tile; K advances by 128
// bytes of codes and one float of scales per block).
template <int BM>
struct TileSrc {
  static constexpr int A_LOADS = BM / 32;
  const uint8_t* wbase;
  uint32_t w_off[8];
  const uint8_t* a_src[A_LOADS];
  const float* s_src;
};

template <int BM>
__device__ __forceinline__ void issue_stage(StageBuf<BM>* st, const TileSrc<BM>& src, int kb, int wave) {
  // wave-uniform LDS destinations, held in SGPRs
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st));
  const uint32_t wofs = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int q = 0; q < 8; ++q) lds_dma16(src.wbase + src.w_off[q] + (size_t)kb * BK, base + (64 * wofs + 8 * q) * BK);
#pragma unroll
  for (int q = 0; q < TileSrc<BM>::A_LOADS; ++q)
    lds_dma16(src.a_src[q] + (size_t)kb * BK, base + BN * BK + (wofs * (BM / 4) + 8 * q) * BK);
  lds_dma4(src.s_src + kb, base + (BN + BM) * BK + wofs * 256);
}

// One K block: wait for stage `cur`, start the DMA of block kb + 2 into `nxt`
// (the stage block kb - 1 used), then accumulate the block from `cur`.
template <int BM, bool PAIRED>
__device__ __forceinline__ void k_step(const StageBuf<BM>* cur, StageBuf<BM>* nxt,
                                       const TileSrc<BM>& src, int kb, int KB, int wave, int lane,
                                       v4f (&acc)[8][BM / 32]) {
  constexpr int WM = BM / 2;
  constexpr int TS = WM / 16;
  constexpr int LOADS = 8 + BM / 32 + 1;
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  // Stage kb is the oldest of the two stages in flight.  Past the last block the
  // DMA repeats block KB - 1 into a stage nobody reads, which keeps the number of
  // DMAs in flight, and so this wait, the same on every step.
  wait_vmcnt<LOADS>();
  raw_barrier();
  issue_stage<BM>(nxt, src, min(kb + 2, KB - 1), wave);
  const float swg = cur->s[PAIRED ? BM : BM + wn];
  const float swu = cur->s[BM + 1];
  typedef float vts __attribute__((ext_vector_type(TS)));
  const vts sav = *(const vts*)(cur->s + (wt * 16 + l16) * TS);
  v8i bf[TS];
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) bf[ti] = lds_frag(cur->a, wt * WM + ti * 16 + l16, g);
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    const v8i af = lds_frag(cur->w, wn * 128 + ni * 16 + l16, g);
    const float swn = (PAIRED && (ni & 1)) ? swu : swg;
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      const v4f part =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[ti], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      acc[ni][ti] += part * (sav[ti] * swn);
    }
  }
}

template <int BM, int EPI, bool PAIRED>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_b128_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) StageBuf<BM> st0;
  __shared__ __attribute__((aligned(16))) StageBuf<BM> st1;
  __shared__ __attribute__((aligned(16))) StageBuf<BM> st2;
  __shared__ __attribute__((aligned(16))) Misc<BM> misc;
  constexpr int WM = BM / 2;        // tokens per wave
  constexpr int TS = WM / 16;       // 16-token sub-tiles per wave
  constexpr int RPW = BM / 4;       // activation rows loaded per wave per stage
  constexpr int A_LOADS = RPW / 8;  // 1-KB DMAs of activation rows per wave per stage
  constexpr int W_LOADS = 8;        // 1-KB DMAs of weight rows per wave per stage
  static_assert(A_LOADS >= 1 && BM + 2 <= 256, "32 <= BM <= 248");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int E = p.E, N = p.N, K = p.K, KB = K / BK;
  const int I = N / 2;
  const int NB = N / 128;
  const int NT = PAIRED ? I / 128 : (N + BN - 1) / BN;
  const float* bsc = (const float*)p.b_scales;

  // ---- tile table: tiles of expert e = ceil(rows_e / BM) * NT, prefix in misc.tp
  for (int e = tid; e <= E; e += kThreads) misc.off[e] = p.offsets[e];
  __syncthreads();
  const int seg = (E + kThreads - 1) / kThreads;
  const int e_lo = min(E, tid * seg), e_hi = min(E, tid * seg + seg);
  int mine = 0;
  for (int e = e_lo; e < e_hi; ++e) mine += ((misc.off[e + 1] - misc.off[e] + BM - 1) / BM) * NT;
  misc.scan[tid] = mine;
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {
    const int v = tid >= d ? misc.scan[tid - d] : 0;
    __syncthreads();
    misc.scan[tid] += v;
    __syncthreads();
  }
  {
    int run = misc.scan[tid] - mine;
    for (int e = e_lo; e < e_hi; ++e) {
      misc.tp[e] = run;
      run += ((misc.off[e + 1] - misc.off[e] + BM - 1) / BM) * NT;
    }
    if (tid == kThreads - 1) misc.tp[E] = misc.scan[kThreads - 1];
  }
  __syncthreads();
  const int total = misc.tp[E];

  const int G = gridDim.x;
  const int vb = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

  for (int t = vb; t < total; t += G) {
    // ---- locate the tile: the last expert e with tp[e] <= t
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (misc.tp[mid] <= t) lo = mid; else hi = mid;
    }
    // every lane computed the same values: make them scalar (SGPR) so the
    // weight-scale reads below are scalar loads
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int m_begin = __builtin_amdgcn_readfirstlane(misc.off[e]);
    const int m_end = __builtin_amdgcn_readfirstlane(misc.off[e + 1]);
    const int mt = (m_end - m_begin + BM - 1) / BM;
    const int loc = t - __builtin_amdgcn_readfirstlane(misc.tp[e]);
    const int n_tile = loc / mt;
    const int m0 = m_begin + (loc % mt) * BM;

    // ---- per-lane DMA sources
    TileSrc<BM> src;
    src.wbase = p.b_codes + (size_t)e * N * K;
#pragma unroll
    for (int q = 0; q < W_LOADS; ++q) {
      const int tr = 64 * wave + 8 * q + (lane >> 3);
      src.w_off[q] = (uint32_t)b_row<PAIRED>(n_tile, tr, N) * (uint32_t)K + (uint32_t)(((lane & 7) ^ swz(tr)) << 4);
    }
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      const int tr = wave * RPW + 8 * q + (lane >> 3);
      const int r = min(m0 + tr, m_end - 1);
      const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
      src.a_src[q] = p.a_codes + (size_t)arow * K + (((lane & 7) ^ swz(tr)) << 4);
    }
    // Scale DMA, 4 bytes per lane, lane L of wave w filling scale slot
    // p = 64 w + L of the stage.  Slots [0, BM) hold the activation scales in
    // the order the MFMA lanes read them (slot (wt*16 + l16) * TS + ti is token
    // row wt*WM + ti*16 + l16), so each lane reads its TS scales with one LDS
    // load.  Slots BM and BM + 1 hold the two weight-block scales of the tile
    // (gate and up blocks when paired, the blocks of the two n-halves
    // otherwise).  The remaining lanes repeat slot 0.
    {
      const int slot = 64 * wave + lane;
      if (slot == BM || slot == BM + 1) {
        int nb;
        if constexpr (PAIRED) nb = slot == BM ? n_tile : I / 128 + n_tile;
        else nb = min(n_tile * 2 + (slot - BM), NB - 1);
        src.s_src = bsc + ((size_t)e * NB + nb) * KB;
      } else {
        const int q = slot < BM ? slot / TS : 0;
        const int ti = slot < BM ? slot % TS : 0;
        const int tr = (q / 16) * WM + ti * 16 + (q % 16);
        const int r = min(m0 + tr, m_end - 1);
        const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
        src.s_src = (const float*)p.a_scales + (size_t)arow * KB;
      }
    }

    v4f acc[8][TS];
#pragma unroll
    for (int ni = 0; ni < 8; ++ni)
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) acc[ni][ti] = v4f{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous tile's LDS readers are done
    issue_stage<BM>(&st0, src, 0, wave);
    issue_stage<BM>(&st1, src, min(1, KB - 1), wave);
    for (int kb = 0; kb < KB; kb += 3) {
      k_step<BM, PAIRED>(&st0, &st2, src, kb, KB, wave, lane, acc);
      if (kb + 1 < KB) k_step<BM, PAIRED>(&st1, &st0, src, kb + 1, KB, wave, lane, acc);
      if (kb + 2 < KB) k_step<BM, PAIRED>(&st2, &st1, src, kb + 2, KB, wave, lane, acc);
    }
    wait_vmcnt<0>();  // the trailing repeat DMAs land before the stages are reused

    // ---- epilogues
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
      // h of pair q, sub-tile ti, element i (recomputed in the second pass
      // instead of being held across the barrier).
      auto hval = [&](int q, int ti, int i) {
        float gv = acc[2 * q][ti][i];
        float uv = acc[2 * q + 1][ti][i];
        if (p.has_limit) {
          gv = __builtin_fminf(gv, p.limit);
          uv = __builtin_fminf(__builtin_fmaxf(uv, -p.limit), p.limit);
        }
        return gv / (1.0f + __expf(-gv)) * uv;
      };
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) {
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(hval(q, ti, i)));
        m = wave_max_xor(m, 16);
        m = wave_max_xor(m, 32);
        if (g == 0) misc.amax[wn][wt * WM + ti * 16 + l16] = m;
      }
      __syncthreads();
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) {
        const int tt = wt * WM + ti * 16 + l16;
        const float amax = __builtin_fmaxf(misc.amax[0][tt], misc.amax[1][tt]);
        const float s = fp8_block_scale(amax);
        const float inv = 1.0f / s;
        const int r = m0 + tt;
        if (r < m_end) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t code =
                e4m3x4(hval(q, ti, 0) * inv, hval(q, ti, 1) * inv, hval(q, ti, 2) * inv, hval(q, ti, 3) * inv);
            *(uint32_t*)(p.h_codes + (size_t)r * I + n_tile * 128 + 16 * (wn * 4 + q) + 4 * g) = code;
          }
          if (wn == 0 && g == 0) ((float*)p.h_scales)[(size_t)r * (I / 128) + n_tile] = s;
        }
      }
    } else {  // kEpiWeightedScatter
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) {
        const int r = m0 + wt * WM + ti * 16 + l16;
        if (r < m_end) {
          const int slot = p.slot_of_row[r];
          const float w = p.top_k_weights[slot];
#pragma unroll
          for (int ni = 0; ni < 8; ++ni) {
            const int n = n_tile * BN + wn * 128 + ni * 16 + 4 * g;
            if (n < N) {
              const v4f v = acc[ni][ti] * w;
              uint2 o;
              o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
              o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
              *(uint2*)(p.slot_out + (size_t)slot * N + n) = o;
            }
          }
        }
      }
    }
  }
}

template <int BM, int EPI, bool PAIRED>
hipError_t launch_one(const GemmParams& p, int num_cus, hipStream_t stream) {
  auto kern = gemm_fp8_b128_kernel<BM, EPI, PAIRED>;
  const int NT = PAIRED ? (p.N / 2) / 128 : (p.N + BN - 1) / BN;
  const long bound = ((long)(p.max_rows + BM - 1) / BM + p.E) * NT;
  long grid = bound < num_cus ? bound : num_cus;
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int BM>
hipError_t dispatch_epi(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_one<BM, kEpiSwiGLUQuant, true>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_one<BM, kEpiWeightedScatter, false>(p, num_cus, stream);
  if (paired) return launch_one<BM, kEpiStoreF32, true>(p, num_cus, stream);
  return launch_one<BM, kEpiStoreF32, false>(p, num_cus, stream);
}

}  // namespace

hipError_t launch_gemm_fp8_b128(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  const long avg_rows = p.E > 0 ? (long)p.max_rows / p.E : p.max_rows;
  if (avg_rows >= 96) return dispatch_epi<128>(p, epi, paired, num_cus, stream);
  if (avg_rows >= 48) return dispatch_epi<64>(p, epi, paired, num_cus, stream);
  return dispatch_epi<32>(p, epi, paired, num_cus, stream);
}

}  // namespace moe
