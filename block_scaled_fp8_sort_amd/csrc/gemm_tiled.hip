// Tiled grouped GEMM over expert-sorted rows for gfx950: FP8 e4m3 x e4m3 with
// fp32 block scales (1x128 on the activations, 128x128 on the weights), and on
// the same tiles bf16 x bf16.
//
// What it computes: for expert e and sorted row r of its range,
// C[r, n] = sum_i A[a_row(r), i] * B[e, n, i] with dequantized operands (code
// times block scale), then one of the epilogues of moe_grouped_gemm.  This is
// the gate_up ("L1") and down ("L2") grouped matmul of the pages' grouped
// experts forward ("grouped_mm experts dispatch does not support
// activation_scheme='static'", sections "What it means" and "Source"), with the
// token-row gather (rows picked by perm // k) folded into the operand loads.
// The same tiles also run the unquantized bf16 experts (the pages' grouped_mm
// fallback, "DeepGEMM experts selected on a model spanning multiple CUDA
// devices", the record's source): bf16 rows are tiled as rows of 2K bytes, and
// only the K step (two bf16 MFMAs per 128-byte block, no scales) and the SwiGLU
// store (h in bf16) differ.
//
// Design (gfx950, wave64):
//  * MFMA A operand = weight rows (output features n), MFMA B operand = the
//    gathered activation rows (tokens).  In v_mfma_f32_16x16x128_f8f6f4's
//    output each lane holds 4 consecutive n of one token, so the activation
//    scale of a 128-wide K block is one value per lane and the weight scale is
//    one value per 16-row sub-tile.
//  * fp32 block scales cannot ride the MFMA's E8M0 scale operands, so each
//    128-wide K block is one MFMA with a zero accumulator (the block's partial
//    sum of code products) followed by acc += P * (s_act * s_w) on the VALU.
//    The MFMAs of one n sub-tile and the FMAs of the previous one are
//    interleaved in program order, so the matrix core and the VALU overlap.
//  * Workgroup tile 256 (n) x BM (tokens) x 128 (K), eight waves as 2 (n) x 4
//    (tokens), two per SIMD, each 128 n x BM/4 tokens.  BM is 256 for full
//    m-tiles and 64, 128 or 256 for an expert's last, partial one (192 on the
//    gate_up GEMM for an expert whose only m-tile has 129-192 rows), chosen per
//    tile.  Two LDS stages at BM = 192 and 256, three at smaller BM: those
//    tiles stream their weights, and capping them at two stages made the
//    DeepSeek-V3 forward 6% slower.
//  * Operands move global -> LDS by LDS-DMA (global_load_lds_dwordx4, 16 bytes
//    per lane).  Weights are pre-tiled in MFMA operand order (tile_layout.h), so
//    each DMA instruction copies one contiguous 1 KB and each fragment read is
//    linear; activations are stored K-block-major
//    ([K/128][rows][128 bytes]), so a DMA instruction gathers 8 token rows'
//    128-byte chunks by per-lane address (the gather is free) without the
//    same-L2-channel aliasing that 4 KB-strided rows suffer.
//  * Persistent grid: each workgroup reads the expert offsets, builds the tile
//    table in LDS (per expert, groups of up to 4 m-tiles, m fastest inside a
//    group, then n; the short remainder tiles of large experts after all the
//    rest, so they fill the last round), and walks tiles with a stride of the
//    grid size.  Without the gate/up pairing those remainder tiles run as two
//    128-row halves of each n-tile: the last round then has twice the tiles to
//    spread over the CUs, and each half streams its weights through four or
//    five stages instead of three.
//    Workgroup ids are remapped so that consecutive tiles land on the same XCD
//    (dispatch is round-robin over the 8 XCDs): a weight tile is shared by the
//    group's m-tiles in that XCD's L2, and the group's activation rows stay
//    cached across its n-tiles.  Rows past the expert's end are masked; no
//    host-visible counts are needed.
//  * The epilogues stage their outputs (the SwiGLU's h codes, the down GEMM's
//    weighted bf16 rows) in the stage area, free once every wave is past the K
//    loop, and store them as whole rows, 16 bytes per lane.
#include <type_traits>

#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"
#include "tile_layout.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = kTileN;
constexpr int BK = kBlockK;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxE = 512;

// One pipeline stage in LDS: the WR weight rows (256, or one 128-row half of
// an n-tile) and BM activation rows of one 128-wide K block, and the scales of
// that block (one 256-byte DMA per wave: slots [0, BM) are the activation
// scales in the order the MFMA lanes read them, slots BM and BM + 1 the two
// weight-block scales).
template <int BM, int WR = BN>
struct StageBuf {
  uint8_t w[WR * BK];
  uint8_t a[BM * BK];
  float s[kWaves * 64];
};

constexpr int kMaxBM = 256;

// Tile table and epilogue exchange.
struct Misc {
  int off[kMaxE + 1];
  int tp[kMaxE + 1];
  uint16_t cnt[kMaxE + 2];
  int next[2];  // dispensed tile values, alternating per tile
  union {
    int2 scan[kThreads];     // tile table build (kernel start)
    float amax[2][kMaxBM];   // SwiGLU epilogue
  };
};

// LDS shared by the pipeline stages of every tile height: three stages of the
// 128-row layout, which also hold two of the 256-row and of the 192-row one,
// three of the 64-row one, and four or five of the half-width (128 weight
// rows) ones.
constexpr int kStageArea = 3 * (int)sizeof(StageBuf<128>);
template <int BM, int WR = BN>
constexpr int stages_for() {
  return kStageArea / (int)sizeof(StageBuf<BM, WR>) < 5 ? kStageArea / (int)sizeof(StageBuf<BM, WR>) : 5;
}
static_assert(stages_for<256>() >= 2 && stages_for<64>() >= 3 && stages_for<128, 128>() >= 4 &&
                  stages_for<64, 128>() >= 5,
              "stage area");

// The 32 bytes lane group g of an MFMA operand holds: K bytes [16 g, 16 g + 16)
// and [64 + 16 g, 64 + 16 g + 16) of its row (logical chunks g and 4 + g).
// Activation row tr of an LDS stage (chunks at their swizzled positions):
__device__ __forceinline__ v8i lds_frag_a(const uint8_t* region, int tr, int g) {
  const int s = swz(tr);
  const int4 x0 = *(const int4*)(region + tr * BK + ((g ^ s) << 4));
  const int4 x1 = *(const int4*)(region + tr * BK + (((4 + g) ^ s) << 4));
  return v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
}
// 16-row weight group grp of an LDS stage, stored in operand order: lane l's
// halves at l * 16 and 1024 + l * 16.
__device__ __forceinline__ v8i lds_frag_w(const uint8_t* region, int grp, int lane) {
  const uint8_t* b = region + grp * 2048 + lane * 16;
  const int4 x0 = *(const int4*)b;
  const int4 x1 = *(const int4*)(b + 1024);
  return v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
}

// Per-lane DMA sources of one tile.
template <int BM>
struct TileSrc {
  static constexpr int A_LOADS = BM / 64;  // 1 KB activation DMAs per wave per stage
  const uint8_t* w_tile;   // tiled weights of (expert, n-tile[, half]), K block 0 (uniform)
  const uint8_t* a_codes;  // activations (uniform)
  size_t a_plane;          // byte step of A per K block: one K-block plane (FP8), 128 (bf16 rows)
  uint32_t a_off[A_LOADS]; // per-lane byte offset of the gathered row chunk
  const float* s_base;     // per-lane scale address of K block 0
  uint32_t s_stride;       // per-lane scale advance per K block, in floats
};

// DMA instruction idx (0 .. LOADS - 1) of the stage for block kb: first WR / 64
// for the weights (wave w copies the WR / 8 rows [w WR/8, (w+1) WR/8) of the
// stage, contiguous in the tiled layout), then BM / 64 activation gathers (wave
// w gathers rows [w BM/8, (w+1) BM/8) of the tile), last the scales.  idx is a
// compile-time constant after unrolling.
template <int BM, int WR, bool BF>
__device__ __forceinline__ void issue_part(StageBuf<BM, WR>* st, const TileSrc<BM>& src, int kb, int wave,
                                           int lane, int idx) {
  constexpr int W_LOADS = WR / 64, WB = WR * BK / kWaves;  // per wave: 1 KB DMAs, bytes
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st));
  const uint32_t w = __builtin_amdgcn_readfirstlane(wave);
  if (idx < W_LOADS) {
    const uint8_t* wsrc = src.w_tile + (size_t)kb * (BN * BK) + w * WB;
    lds_dma16_s(wsrc + idx * 1024, lane * 16, base + w * WB + idx * 1024);
  } else if (idx < W_LOADS + TileSrc<BM>::A_LOADS) {
    const int q = idx - W_LOADS;
    const uint8_t* plane = src.a_codes + (size_t)kb * src.a_plane;
    lds_dma16_s(plane, src.a_off[q], base + WR * BK + (w * (BM / 8) + 8 * q) * BK);
  } else if constexpr (!BF) {
    lds_dma4(src.s_base + (size_t)kb * src.s_stride, base + (WR + BM) * BK + w * 256);
  }
}

// DMA instructions per wave per stage: weights, activations, and the scales
// (none for bf16 operands)
template <int BM, int WR, bool BF>
constexpr int stage_loads() {
  return WR / 64 + BM / 64 + (BF ? 0 : 1);
}

template <int BM, int WR, bool BF>
__device__ __forceinline__ void issue_stage(StageBuf<BM, WR>* st, const TileSrc<BM>& src, int kb, int wave,
                                            int lane) {
  constexpr int LOADS = stage_loads<BM, WR, BF>();
#pragma unroll
  for (int idx = 0; idx < LOADS; ++idx) issue_part<BM, WR, BF>(st, src, kb, wave, lane, idx);
}

// One K block: wait for stage `cur`, then accumulate the block from `cur` while
// the DMA of block kb + STAGES - 1 goes out into `nxt` (the stage block kb - 1
// used).
// Past the last block the DMA repeats block KB - 1 into a stage nobody reads,
// which keeps the number of DMAs in flight, and so this wait, the same on every
// step.
template <int BM, bool PAIRED, int STAGES, int WR>
__device__ __forceinline__ void k_step(const StageBuf<BM, WR>* cur, StageBuf<BM, WR>* nxt, const TileSrc<BM>& src,
                                       int kb, int KB, int wave, int lane, v4f (&acc)[WR / 32][BM / 64]) {
  constexpr int WM = BM / 4;
  constexpr int TS = WM / 16;
  constexpr int NW = WR / 32;                    // 16-row weight groups per wave
  constexpr int LOADS = stage_loads<BM, WR, false>();
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  wait_vmcnt<LOADS * (STAGES - 2)>();  // this wave's DMAs of stage kb have landed
  raw_barrier();  // ... and every other wave's; all waves are done with block kb - 1
  const int kb_dma = min(kb + STAGES - 1, KB - 1);
  // a half tile's 128 rows lie in one 128-row weight-scale block
  const float swg = cur->s[PAIRED || WR == 128 ? BM : BM + wn];
  const float swu = cur->s[BM + 1];
  // the lane's TS activation scales are consecutive slots: one vector read
  // (three single reads at TS = 3, whose slots are not 16-byte aligned)
  float sav[TS];
  if constexpr (TS == 3) {
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) sav[ti] = cur->s[(wt * 16 + l16) * TS + ti];
  } else {
    typedef float vts __attribute__((ext_vector_type(TS)));
    const vts v = *(const vts*)(cur->s + (wt * 16 + l16) * TS);
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) sav[ti] = v[ti];
  }
  v8i bf[TS];
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) bf[ti] = lds_frag_a(cur->a, wt * WM + ti * 16 + l16, g);
  float fg[TS], fu[TS];
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) {
    fg[ti] = sav[ti] * swg;
    fu[ti] = sav[ti] * swu;
  }
  // Software pipeline over the 8 n sub-tiles: the MFMAs of sub-tile ni write
  // one set of partial registers while the FMAs fold the other set (sub-tile
  // ni - 1) into the accumulators, and the weight fragment of sub-tile ni + 1 is
  // read from LDS meanwhile.  sched_barrier(0) keeps this program order.
  v4f part[2][TS];
  v8i af = lds_frag_w(cur->w, wn * NW, lane);
#pragma unroll
  for (int ni = 0; ni <= NW; ++ni) {
    // the DMAs of block kb + STAGES - 1 go out spread over the first six of the
    // eight sub-tiles: issued all at once they queue in the texture addresser
    // and hold every wave back from its MFMAs, between MFMAs they drain in the
    // background; spread over all eight, the last ones have too little of the
    // step left to land before the next step's wait (six: the gate_up GEMM 1-3%
    // faster than eight; five and seven about the same as six, four slower)
#pragma unroll
    for (int idx = 0; idx < LOADS; ++idx)
      if (idx * (NW * 3 / 4) / LOADS == ni) issue_part<BM, WR, false>(nxt, src, kb_dma, wave, lane, idx);
    v8i af_next = af;
    if (ni < NW - 1) af_next = lds_frag_w(cur->w, wn * NW + ni + 1, lane);
    const int pn = ni - 1;
    const bool up = PAIRED && (pn & 1);
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      if (ni < NW)
        part[ni & 1][ti] =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[ti], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      if (ni > 0) acc[pn][ti] += part[pn & 1][ti] * (up ? fu[ti] : fg[ti]);
      __builtin_amdgcn_sched_barrier(0);
    }
    af = af_next;
  }
}

// The same K step for bf16 operands.  A 128-byte K block holds 64 bf16, and
// the fragments the FP8 step reads (chunks g and 4 + g of a row, for both
// operands) are exactly the operands of two v_mfma_f32_16x16x32_bf16: chunk g
// covers K elements [8 g, 8 g + 8) of the block's first 32, chunk 4 + g the same
// of its last 32.  The products accumulate in the MFMA itself (no scales, no
// promotion); the two MFMAs of one accumulator are split by the tile's other
// token sub-tiles.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 frag_lo(const v8i& v) {
  return __builtin_bit_cast(bf16x8, v4i_t{v[0], v[1], v[2], v[3]});
}
__device__ __forceinline__ bf16x8 frag_hi(const v8i& v) {
  return __builtin_bit_cast(bf16x8, v4i_t{v[4], v[5], v[6], v[7]});
}

template <int BM, int STAGES, int WR>
__device__ __forceinline__ void k_step_bf16(const StageBuf<BM, WR>* cur, StageBuf<BM, WR>* nxt,
                                            const TileSrc<BM>& src, int kb, int KB, int wave, int lane,
                                            v4f (&acc)[WR / 32][BM / 64]) {
  constexpr int WM = BM / 4;
  constexpr int TS = WM / 16;
  constexpr int NW = WR / 32;
  constexpr int LOADS = stage_loads<BM, WR, true>();
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  wait_vmcnt<LOADS * (STAGES - 2)>();  // this wave's DMAs of stage kb have landed
  raw_barrier();  // ... and every other wave's; all waves are done with block kb - 1
  const int kb_dma = min(kb + STAGES - 1, KB - 1);
  v8i bf[TS];
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) bf[ti] = lds_frag_a(cur->a, wt * WM + ti * 16 + l16, g);
  v8i af = lds_frag_w(cur->w, wn * NW, lane);
#pragma unroll
  for (int ni = 0; ni < NW; ++ni) {
    // the next block's DMAs spread over the first six sub-tiles, as in k_step
#pragma unroll
    for (int idx = 0; idx < LOADS; ++idx)
      if (idx * (NW * 3 / 4) / LOADS == ni) issue_part<BM, WR, true>(nxt, src, kb_dma, wave, lane, idx);
    v8i af_next = af;
    if (ni < NW - 1) af_next = lds_frag_w(cur->w, wn * NW + ni + 1, lane);
#pragma unroll
    for (int ti = 0; ti < TS; ++ti)
      acc[ni][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_lo(af), frag_lo(bf[ti]), acc[ni][ti], 0, 0, 0);
#pragma unroll
    for (int ti = 0; ti < TS; ++ti)
      acc[ni][ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_hi(af), frag_hi(bf[ti]), acc[ni][ti], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    af = af_next;
  }
}

// One tile of BM sorted rows [m0, min(m0 + BM, m_end)) of expert e against
// n-tile n_tile (WR = 256), or against its 128 weight rows [128 half, 128 half +
// 128) (WR = 128, unpaired only): the K loop through a ring of STAGES LDS
// stages carved out of `area`, then the epilogue.  A half tile streams half the
// weights per stage, so more stages fit and more bytes are in flight per CU.
template <int BM, int EPI, bool PAIRED, bool BF, int WR = BN>
__device__ __forceinline__ void run_tile(const GemmParams& p, uint8_t* area, Misc& misc, int e, int n_tile, int m0,
                                         int m_end, int half = 0) {
  constexpr int STAGES = stages_for<BM, WR>();
  constexpr int WM = BM / 4;   // tokens per wave
  constexpr int TS = WM / 16;  // 16-token sub-tiles per wave
  constexpr int NW = WR / 32;  // 16-row weight groups per wave
  static_assert(TS >= 1 && BM + 2 <= kWaves * 64, "64 <= BM <= 256");
  static_assert(WR == BN || (WR == 128 && !PAIRED), "half tiles are unpaired");
  StageBuf<BM, WR>* st = reinterpret_cast<StageBuf<BM, WR>*>(area);

  // the thread id is made opaque per tile so that the per-lane address math of
  // each tile height stays inside its tile instead of being hoisted out of the
  // tile loop for all heights at once (which would spill registers)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wt = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int N = p.N;
  const int KB = BF ? p.K * 2 / BK : p.K / BK;  // 128-byte K blocks
  const int I = N / 2;
  const int NB = N / 128;
  const int NT = PAIRED ? I / 128 : (N + BN - 1) / BN;
  const float* bsc = (const float*)p.b_scales;

  // ---- per-lane DMA sources
  TileSrc<BM> src;
  src.w_tile = p.b_codes + ((size_t)e * NT + n_tile) * (size_t)KB * (BN * BK) + (WR == 128 ? half * (128 * BK) : 0);
  src.a_codes = p.a_codes;
  // FP8 codes are K-block-major ([K/128][rows][128]); bf16 rows are row-major
  // [rows][K] (the host keeps them under 4 GiB, so byte offsets fit 32 bits)
  src.a_plane = BF ? (size_t)BK : (size_t)p.a_rows * BK;
  const uint32_t a_pitch = BF ? (uint32_t)p.K * 2 : (uint32_t)BK;
#pragma unroll
  for (int q = 0; q < TileSrc<BM>::A_LOADS; ++q) {
    const int tr = wave * (BM / 8) + 8 * q + (lane >> 3);
    const int r = min(m0 + tr, m_end - 1);
    const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
    src.a_off[q] = (uint32_t)arow * a_pitch + (uint32_t)(((lane & 7) ^ swz(tr)) << 4);
  }
  if constexpr (!BF) {
    const int slot = 64 * wave + lane;
    if (slot == BM || slot == BM + 1) {
      int nb;
      if constexpr (PAIRED) nb = slot == BM ? n_tile : I / 128 + n_tile;
      else if constexpr (WR == 128) nb = min(n_tile * 2 + half, NB - 1);
      else nb = min(n_tile * 2 + (slot - BM), NB - 1);
      src.s_base = bsc + ((size_t)e * NB + nb) * KB;
      src.s_stride = 1;
    } else {
      const int q = slot < BM ? slot / TS : 0;
      const int ti = slot < BM ? slot % TS : 0;
      const int tr = (q / 16) * WM + ti * 16 + (q % 16);
      const int r = min(m0 + tr, m_end - 1);
      if (p.a_scales_sorted) {  // by sorted row: the tile's scales are contiguous
        src.s_base = (const float*)p.a_scales_sorted + r;
        src.s_stride = (uint32_t)p.max_rows;
      } else {
        const int arow = p.a_row_index ? p.a_row_index[r] / p.a_row_div : r;
        src.s_base = (const float*)p.a_scales + arow;
        src.s_stride = (uint32_t)p.a_rows;
      }
    }
  }

  v4f acc[NW][TS];
#pragma unroll
  for (int ni = 0; ni < NW; ++ni)
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) acc[ni][ti] = v4f{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // the previous tile's LDS readers are done
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue_stage<BM, WR, BF>(&st[s], src, min(s, KB - 1), wave, lane);
  for (int kb = 0; kb < KB; kb += STAGES) {
#pragma unroll
    for (int j = 0; j < STAGES; ++j)
      if (kb + j < KB) {
        if constexpr (BF)
          k_step_bf16<BM, STAGES, WR>(&st[j], &st[(j + STAGES - 1) % STAGES], src, kb + j, KB, wave, lane, acc);
        else
          k_step<BM, PAIRED, STAGES, WR>(&st[j], &st[(j + STAGES - 1) % STAGES], src, kb + j, KB, wave, lane, acc);
      }
  }
  wait_vmcnt<0>();  // the trailing repeat DMAs land before the stages are reused

  // ---- epilogues
  if constexpr (EPI == kEpiStoreF32) {
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      const int r = m0 + wt * WM + ti * 16 + l16;
      if (r < m_end) {
#pragma unroll
        for (int ni = 0; ni < NW; ++ni) {
          int n;
          if constexpr (PAIRED) {
            const int h = n_tile * 128 + 16 * (wn * 4 + (ni >> 1)) + 4 * g;
            n = (ni & 1) ? I + h : h;
          } else {
            n = n_tile * BN + (WR == 128 ? half * 128 : 0) + wn * NW * 16 + ni * 16 + 4 * g;
          }
          if (n < N) *(v4f*)(p.c_f32 + (size_t)r * N + n) = acc[ni][ti];
        }
      }
    }
  } else if constexpr (EPI == kEpiSwiGLUQuant && BF) {
    static_assert(PAIRED, "SwiGLU needs the paired gate/up layout");
    // h rounded once to bf16, row-major [rows][I] (the down GEMM's operand)
    auto store_h = [&](auto lim) {
      constexpr bool LIM = decltype(lim)::value;
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) {
        const int r = m0 + wt * WM + ti * 16 + l16;
        if (r >= m_end) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int h = n_tile * 128 + 16 * (wn * 4 + q) + 4 * g;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = swiglu<LIM>(acc[2 * q][ti][i], acc[2 * q + 1][ti][i], p.limit);
          uint2 o;
          o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *(uint2*)((uint16_t*)p.h_codes + (size_t)r * I + h) = o;
        }
      }
    };
    if (p.has_limit) store_h(std::true_type{});
    else store_h(std::false_type{});
  } else if constexpr (EPI == kEpiSwiGLUQuant) {
    static_assert(PAIRED, "SwiGLU needs the paired gate/up layout");
    // h of pair q, sub-tile ti, element i, computed once into the gate's
    // accumulator, and its amax over the tile's 128 outputs of each token
    auto swiglu_rows = [&](auto lim) {
      constexpr bool LIM = decltype(lim)::value;
#pragma unroll
      for (int ti = 0; ti < TS; ++ti) {
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h = swiglu<LIM>(acc[2 * q][ti][i], acc[2 * q + 1][ti][i], p.limit);
            acc[2 * q][ti][i] = h;
            m = __builtin_fmaxf(m, __builtin_fabsf(h));
          }
        m = wave_max_xor(m, 16);
        m = wave_max_xor(m, 32);
        if (g == 0) misc.amax[wn][wt * WM + ti * 16 + l16] = m;
      }
    };
    if (p.has_limit) swiglu_rows(std::true_type{});
    else swiglu_rows(std::false_type{});
    __syncthreads();
    // h codes go to the K-block-major layout [I/128][max_rows][128] that the
    // down GEMM reads; the tile's 128 outputs are exactly plane n_tile, staged
    // here (every wave is past the K loop) and stored as whole rows
    static_assert(BM * kHPitch <= kStageArea, "h staging");
#pragma unroll
    for (int ti = 0; ti < TS; ++ti) {
      const int tt = wt * WM + ti * 16 + l16;
      const float amax = __builtin_fmaxf(misc.amax[0][tt], misc.amax[1][tt]);
      const float s = fp8_block_scale(amax);
      const float inv = 1.0f / s;
      // h / s as the activation rule's IEEE quotient (div_by_scale)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f h = acc[2 * q][ti];
        *(uint32_t*)(area + tt * kHPitch + 16 * (wn * 4 + q) + 4 * g) =
            e4m3x4(div_by_scale(h[0], s, inv), div_by_scale(h[1], s, inv), div_by_scale(h[2], s, inv),
                   div_by_scale(h[3], s, inv));
      }
      const int r = m0 + tt;
      if (r < m_end && wn == 0 && g == 0) ((float*)p.h_scales)[(size_t)n_tile * p.max_rows + r] = s;
    }
    __syncthreads();
    copy_out_h_codes<BM>(p, area, n_tile, m0, m_end, tid);
  } else {  // kEpiWeightedScatter
    static_assert(BM * kOutPitch <= kStageArea, "output staging");
    scatter_rows_staged<BM, NW>(p, area, reinterpret_cast<int*>(&misc.amax[0][0]), acc,
                                n_tile * BN + (WR == 128 ? half * 128 : 0), m0, m_end, tid);
  }
}

// Persistent kernel.  An expert's rows are cut into 256-row m-tiles; the last,
// partial one runs at the smallest height of {64, 128, 256} that covers it (and
// on the gate_up GEMM an expert's only m-tile at 192 rows when that covers it),
// so little MFMA work goes to padding rows while the number of tiles stays that
// of 256-row tiles.  Tiles come from the two-phase table (longest first).  The
// body serves both operand types; each has a kernel of its own below.
template <int EPI, bool PAIRED, bool BF>
__device__ __forceinline__ void tiled_gemm(const GemmParams& p, uint8_t* area, Misc& misc) {
  const int E = p.E, N = p.N;
  const int NT = PAIRED ? (N / 2) / 128 : (N + BN - 1) / BN;
  // unpaired: the short remainder tiles (at most 128 rows, run last) go as two
  // 128-row halves each
  constexpr int SPLIT = PAIRED ? 1 : 2;
  const int total = build_tile_table2<kThreads, SPLIT>(p.offsets, E, NT, misc.off, misc.tp, misc.cnt, misc.scan,
                                                                 p.two_phase != 0);
  const int G = gridDim.x;
  auto run = [&](int t) {
    const TileCoord tc = locate_tile2<SPLIT>(t, E, NT, misc.off, misc.tp, misc.cnt, p.two_phase != 0);
    const int left = tc.m_end - tc.m0;
    if constexpr (!PAIRED) {
      if (tc.half >= 0) {  // uniform
        if (left > 64)
          run_tile<128, EPI, PAIRED, BF, 128>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end, tc.half);
        else
          run_tile<64, EPI, PAIRED, BF, 128>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end, tc.half);
        return;
      }
    }
    if constexpr (PAIRED) {
      // an expert whose only m-tile has 129-192 rows: 192-row tile.  Not for
      // the last m-tile of an expert with full ones: being shorter it runs
      // ahead of its group's 256-row tiles through the K loop, and they fetch
      // the weight tile it streamed again (Mega-MoE's gate_up L2 misses +34%)
      if (left > 128 && left <= 192 && tc.m0 == __builtin_amdgcn_readfirstlane(misc.off[tc.e])) {
        run_tile<192, EPI, PAIRED, BF>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end);
        return;
      }
    }
    if (left > 128)
      run_tile<256, EPI, PAIRED, BF>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end);
    else if (left > 64)
      run_tile<128, EPI, PAIRED, BF>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end);
    else
      run_tile<64, EPI, PAIRED, BF>(p, area, misc, tc.e, tc.n_tile, tc.m0, tc.m_end);
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
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_b128_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t area[kStageArea];
  __shared__ __attribute__((aligned(16))) Misc misc;
  tiled_gemm<EPI, PAIRED, false>(p, area, misc);
}

// bf16 x bf16 with fp32 accumulation: the unquantized experts (weights tiled
// the same way, two bytes per element, so a 128-byte K block is 64 of them).
template <int EPI, bool PAIRED>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_tiled_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t area[kStageArea];
  __shared__ __attribute__((aligned(16))) Misc misc;
  tiled_gemm<EPI, PAIRED, true>(p, area, misc);
}

template <int EPI, bool PAIRED, bool BF>
hipError_t launch_one(const GemmParams& p, int num_cus, hipStream_t stream) {
  auto kern = BF ? gemm_bf16_tiled_kernel<EPI, PAIRED> : gemm_fp8_b128_kernel<EPI, PAIRED>;
  const int NT = PAIRED ? (p.N / 2) / 128 : (p.N + BN - 1) / BN;
  const long bound = ((long)(p.max_rows + kMaxBM - 1) / kMaxBM + p.E) * NT;
  long grid = bound < num_cus ? bound : num_cus;
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  // the remainder tiles run last (in halves) on launches with few rounds; on
  // the unpaired GEMM with many rounds they stay beside their expert's other
  // m-tiles (DeepSeek-V3's down GEMM 3% faster); the gate_up GEMM gained
  // nothing measurable either way
  GemmParams q = p;
  q.two_phase = PAIRED || bound < kTwoPhaseMaxRounds * grid ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_b128(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_one<kEpiSwiGLUQuant, true, false>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_one<kEpiWeightedScatter, false, false>(p, num_cus, stream);
  if (paired) return launch_one<kEpiStoreF32, true, false>(p, num_cus, stream);
  return launch_one<kEpiStoreF32, false, false>(p, num_cus, stream);
}

hipError_t launch_gemm_bf16(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (epi == kEpiSwiGLUQuant) return launch_one<kEpiSwiGLUQuant, true, true>(p, num_cus, stream);
  if (epi == kEpiWeightedScatter) return launch_one<kEpiWeightedScatter, false, true>(p, num_cus, stream);
  if (paired) return launch_one<kEpiStoreF32, true, true>(p, num_cus, stream);
  return launch_one<kEpiStoreF32, false, true>(p, num_cus, stream);
}

}  // namespace moe
