// Pieces shared by the grouped GEMM kernels: the persistent tile table, the
// tile lookup and a fence-free barrier.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace moe {

// Barrier without a memory fence: the waits before it are explicit (vmcnt for
// the DMAs this wave issued); the empty asm statements keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive prefix sums over the block of one (x, y) pair per thread, and the
// block totals: a shuffle scan inside each wave, the wave totals through LDS
// (wsum, 2 * THREADS / 64 ints), one barrier.  wsum may be reused after the
// caller's next barrier.
template <int THREADS>
__device__ __forceinline__ void block_scan2(int x, int y, int* wsum, int& ex_x, int& ex_y, int& tot_x,
                                            int& tot_y) {
  constexpr int W = THREADS / 64;
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
  int ix = x, iy = y;
  for (int d = 1; d < 64; d <<= 1) {
    const int ox = __shfl_up(ix, d, 64);
    const int oy = __shfl_up(iy, d, 64);
    if (lane >= d) {
      ix += ox;
      iy += oy;
    }
  }
  if (lane == 63) {
    wsum[w] = ix;
    wsum[W + w] = iy;
  }
  __syncthreads();
  int bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const int sx = wsum[i], sy = wsum[W + i];
    bx += i < w ? sx : 0;
    by += i < w ? sy : 0;
    tx += sx;
    ty += sy;
  }
  ex_x = bx + ix - x;
  ex_y = by + iy - y;
  tot_x = tx;
  tot_y = ty;
}

// Tile table in LDS: off[e] = expert offsets, tp[e] = first tile of expert e,
// where expert e has ceil(rows_e / BM) m-tiles times NT n-tiles (in the order
// of tile_position); tp[E] = total.  All threads of the block must call it.
template <int THREADS>
__device__ __forceinline__ int build_tile_table(const int32_t* offsets, int E, int BM, int NT, int* off, int* tp,
                                                int* scan) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += THREADS) off[e] = offsets[e];
  __syncthreads();
  const int seg = (E + THREADS - 1) / THREADS;
  const int e_lo = min(E, tid * seg), e_hi = min(E, tid * seg + seg);
  int mine = 0;
  for (int e = e_lo; e < e_hi; ++e) mine += ((off[e + 1] - off[e] + BM - 1) / BM) * NT;
  int run, unused, total, unused_t;
  block_scan2<THREADS>(mine, 0, scan, run, unused, total, unused_t);
  for (int e = e_lo; e < e_hi; ++e) {
    tp[e] = run;
    run += ((off[e + 1] - off[e] + BM - 1) / BM) * NT;
  }
  if (tid == 0) tp[E] = total;
  __syncthreads();
  return tp[E];
}

struct TileCoord {
  int e, n_tile, m0, m_end;
  int half;  // two-phase table with split phase-1 tiles: which 128 weight rows of the n-tile, else -1
};

// Order of an expert's mt x NT tiles: groups of up to kTileGroupM m-tiles, m
// fastest inside a group, then n, then the next group.  Consecutive tiles run
// at the same time (on one XCD), so a group's activation rows stay cached
// while all n-tiles pass over them and each weight tile is fetched once per
// group.  With m fastest over a whole large expert instead, its activation rows
// (more than the last-level cache holds at large token counts) would come back
// from HBM once per n-tile.  A window of 32 consecutive tiles (one XCD's
// share, see the dispensers) then spans 4 m-tiles x 8 n-tiles, whose activation
// and weight tiles together are the least bytes when a weight tile is at most
// the size of an activation tile (equal for FP8, half for FP4 weights): on
// Mega-MoE's gate_up GEMM, 4 gave 13% fewer L2 misses and 0.8% less time than 8.
constexpr int kTileGroupM = 4;

// (m index, n index) of tile loc (0-based within its expert).
__device__ __forceinline__ void tile_position(int loc, int mt, int NT, int& m_idx, int& n_idx) {
  const int grp = loc / (kTileGroupM * NT);
  const int in = loc - grp * (kTileGroupM * NT);
  const int gm = min(kTileGroupM, mt - grp * kTileGroupM);
  n_idx = in / gm;
  m_idx = grp * kTileGroupM + (in - n_idx * gm);
}

// Tile t -> (expert, n-tile, first sorted row, end of the expert's rows).  Every
// lane computes the same values; they are made wave-uniform (scalar).
__device__ __forceinline__ TileCoord locate_tile(int t, int E, int BM, int NT, const int* off, const int* tp) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tp[mid] <= t) lo = mid; else hi = mid;
  }
  TileCoord c;
  c.half = -1;
  c.e = __builtin_amdgcn_readfirstlane(lo);
  const int m_begin = __builtin_amdgcn_readfirstlane(off[c.e]);
  c.m_end = __builtin_amdgcn_readfirstlane(off[c.e + 1]);
  const int mt = (c.m_end - m_begin + BM - 1) / BM;
  const int loc = t - __builtin_amdgcn_readfirstlane(tp[c.e]);
  int m_idx, n_idx;
  tile_position(loc, mt, NT, m_idx, n_idx);
  c.n_tile = n_idx;
  c.m0 = m_begin + m_idx * BM;
  return c;
}

// Two-phase tile table of the tiled GEMMs (256-row m-tiles, an expert's last,
// partial m-tile run at 64, 128, 192 or 256 rows).  Phase 1 holds the short
// remainder tiles (at most 128 rows) of experts that also have full m-tiles, NT
// per such expert; phase 0 holds every other tile, in expert order and
// tile_position order inside an expert, and comes first.  The long tiles go
// first, so with round-robin assignment the short remainders fill the last
// round instead of lengthening it; an expert whose only m-tile is short keeps
// its place in phase 0, where its weight-streaming tiles interleave with the
// MFMA-bound ones of the large experts.  With two_phase false every tile is
// in phase 0: a remainder tile then runs beside its expert's other m-tiles and
// reads their weight tile from L2 instead of streaming it again at the end
// (launches with many rounds of tiles, where the last round is a small part).
//   off[e]  expert offsets (E + 1)
//   tp[e]   first phase-0 tile of expert e; tp[E] = phase-0 total
//   cnt[e]  experts before e that have a phase-1 tile; expert e's phase-1 tiles
//           are [cnt[e] NT, cnt[e] NT + NT), or with SPLIT = 2 the two 128-row
//           halves of each n-tile, [2 cnt[e] NT, 2 cnt[e] NT + 2 NT)
// Returns the total tile count.  All threads of the block must call it.
// Unpaired FP8 launches with fewer rounds of tiles than this (tiles per
// workgroup, from the host's upper bound) run the remainder tiles last.
constexpr long kTwoPhaseMaxRounds = 4;

__device__ __forceinline__ int has_short_tile(int rows, bool two_phase) {
  return two_phase && rows > 256 && (rows % 256) > 0 && (rows % 256) <= 128;
}
__device__ __forceinline__ int full_m_tiles(int rows, bool two_phase) {
  return (rows + 255) / 256 - has_short_tile(rows, two_phase);
}

template <int THREADS, int SPLIT = 1>
__device__ __forceinline__ int build_tile_table2(const int32_t* offsets, int E, int NT, int* off, int* tp,
                                                 uint16_t* cnt, int2* scan, bool two_phase) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += THREADS) off[e] = offsets[e];
  __syncthreads();
  const int seg = (E + THREADS - 1) / THREADS;
  const int e_lo = min(E, tid * seg), e_hi = min(E, tid * seg + seg);
  int2 mine = make_int2(0, 0);
  for (int e = e_lo; e < e_hi; ++e) {
    const int rows = off[e + 1] - off[e];
    mine.x += full_m_tiles(rows, two_phase) * NT;
    mine.y += has_short_tile(rows, two_phase);
  }
  int run0, run1, tot0, tot1;
  block_scan2<THREADS>(mine.x, mine.y, reinterpret_cast<int*>(scan), run0, run1, tot0, tot1);
  for (int e = e_lo; e < e_hi; ++e) {
    const int rows = off[e + 1] - off[e];
    tp[e] = run0;
    cnt[e] = (uint16_t)run1;
    run0 += full_m_tiles(rows, two_phase) * NT;
    run1 += has_short_tile(rows, two_phase);
  }
  if (tid == 0) {
    tp[E] = tot0;
    cnt[E] = (uint16_t)tot1;
  }
  __syncthreads();
  return tp[E] + (int)cnt[E] * NT * SPLIT;
}

// Tile t of the two-phase table -> (expert, n-tile, first sorted row, end of
// the expert's rows, half), made wave-uniform.
template <int SPLIT = 1>
__device__ __forceinline__ TileCoord locate_tile2(int t, int E, int NT, const int* off, const int* tp,
                                                  const uint16_t* cnt, bool two_phase) {
  const int total0 = __builtin_amdgcn_readfirstlane(tp[E]);
  TileCoord c;
  c.half = -1;
  int lo = 0, hi = E;
  if (t < total0) {
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tp[mid] <= t) lo = mid; else hi = mid;
    }
    c.e = __builtin_amdgcn_readfirstlane(lo);
    const int m_begin = __builtin_amdgcn_readfirstlane(off[c.e]);
    c.m_end = __builtin_amdgcn_readfirstlane(off[c.e + 1]);
    const int loc = t - __builtin_amdgcn_readfirstlane(tp[c.e]);
    int m_idx, n_idx;
    tile_position(loc, full_m_tiles(c.m_end - m_begin, two_phase), NT, m_idx, n_idx);
    c.n_tile = n_idx;
    c.m0 = m_begin + m_idx * 256;
  } else {
    const int t1 = t - total0;
    const int j = t1 / (NT * SPLIT);  // the j-th expert that has a phase-1 tile
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int)cnt[mid] <= j) lo = mid; else hi = mid;
    }
    c.e = __builtin_amdgcn_readfirstlane(lo);
    const int m_begin = __builtin_amdgcn_readfirstlane(off[c.e]);
    c.m_end = __builtin_amdgcn_readfirstlane(off[c.e + 1]);
    const int loc = t1 - j * NT * SPLIT;
    c.n_tile = loc / SPLIT;
    if (SPLIT == 2) c.half = loc - c.n_tile * 2;
    c.m0 = m_begin + ((c.m_end - m_begin) / 256) * 256;
  }
  return c;
}

// Dynamic tile dispensing, one dispenser per XCD.  The tile sequence is cut
// into windows of kWindow consecutive tiles and window w belongs to dispenser
// w % 8, so each XCD gets a fair slice of the whole sequence (its short tail
// included) while the tiles that share a weight or activation tile still run
// together on one XCD, whose workgroups (dispatch puts block b on XCD b % 8)
// take them in order from the front of its dispenser.  Equal tile counts are
// not equal work (tiles of different heights, skewed experts), so a workgroup
// whose own dispenser is exhausted takes tiles from the back of the dispenser
// with the most left: the tail of that XCD's share, away from the tiles its own
// workgroups run (and share their L2 with) at the front.  A dispenser is one
// 64-bit counter, taken from the front in its low half and from the back in its
// high half; a take with old halves (f, b) is valid iff f + b < count, and then
// hands out index f (front) or count - 1 - b (back), so every index goes out
// exactly once.  Dispenser x's counter is at counters[x * 32] (own 128-byte
// line), the count of retired workgroups at counters[2]; the last workgroup to
// retire zeroes them, so the counters are zero again when the launch ends.
// With a grid that is not a multiple of 8, one dispenser hands out the plain
// sequence.
constexpr int kWindow = 32;
constexpr int kCounterStride = 32;  // ints between counters: 128 bytes

struct Dispenser {
  int32_t* base;  // the counters
  int x, y, nd;   // own dispenser, the one taken from, number of dispensers
  int back;       // taking from the back of dispenser y (after the own one ran out)
  int total;      // tiles in the sequence
};

// Tiles that dispenser x hands out.
__device__ __forceinline__ int dispenser_count(int x, int nd, int total) {
  if (nd == 1) return total;
  const int nwin = (total + kWindow - 1) / kWindow;
  const int owned = x < nwin ? (nwin - 1 - x) / 8 + 1 : 0;
  int count = owned * kWindow;
  if (nwin > 0 && (nwin - 1) % 8 == x) count -= nwin * kWindow - total;
  return count;
}

__device__ __forceinline__ Dispenser make_dispenser(int32_t* counters, int total, int G) {
  Dispenser d;
  d.nd = (G % 8 == 0) ? 8 : 1;
  d.x = d.y = (int)blockIdx.x % d.nd;
  d.back = 0;
  d.base = counters;
  d.total = total;
  return d;
}

// The tile of dispenser y's index i.
__device__ __forceinline__ int dispensed_tile(int y, int nd, int i) {
  if (nd == 1) return i;
  return ((i / kWindow) * 8 + y) * kWindow + (i % kWindow);
}

__device__ __forceinline__ unsigned long long* dispenser_word(const Dispenser& d, int y) {
  int zero;  // the address goes through a VGPR, so the atomics are vector memory atomics
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return reinterpret_cast<unsigned long long*>(d.base + y * kCounterStride + zero);
}

// One take from dispenser y, from the front or the back (single thread); the
// old counter word comes back, take_tile decodes it.
__device__ __forceinline__ unsigned long long grab_tile(const Dispenser& d) {
  return atomicAdd(dispenser_word(d, d.y), d.back ? 1ull << 32 : 1ull);
}

// The tile of a take whose old counter word was `old`, or, once that dispenser
// is exhausted, a tile from the back of the dispenser with the most left; -1
// when every dispenser is exhausted (single thread).
__device__ __forceinline__ int take_tile(Dispenser& d, unsigned long long old) {
  {
    const int f = (int)(uint32_t)old, b = (int)(uint32_t)(old >> 32);
    const int count = dispenser_count(d.y, d.nd, d.total);
    if (f >= 0 && b >= 0 && f + b < count) return dispensed_tile(d.y, d.nd, d.back ? count - 1 - b : f);
  }
  // a take that fails leaves its dispenser out of every later look, so at most
  // nd looks find work; the bound also ends the search on counters that were
  // not zero at the launch (negative halves count as empty)
  for (int look = 0; look < 2 * 8; ++look) {
    int best = -1, most = 0;
    unsigned long long seen[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      seen[j] = j < d.nd ? __hip_atomic_load(dispenser_word(d, j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = (int)(uint32_t)seen[j], b = (int)(uint32_t)(seen[j] >> 32);
      const int left = j < d.nd && f >= 0 && b >= 0 ? dispenser_count(j, d.nd, d.total) - f - b : 0;
      if (left > most) {
        most = left;
        best = j;
      }
    }
    if (best < 0) return -1;
    d.y = best;
    d.back = 1;
    const unsigned long long w = grab_tile(d);
    const int f = (int)(uint32_t)w, b = (int)(uint32_t)(w >> 32);
    const int count = dispenser_count(best, d.nd, d.total);
    if (f >= 0 && b >= 0 && f + b < count) return dispensed_tile(best, d.nd, count - 1 - b);
  }
  return -1;
}

// After a workgroup's last take (single thread): the last to retire zeroes the
// counters for the next launch.
__device__ __forceinline__ void retire(const Dispenser& d, int G) {
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  if (atomicAdd(d.base + 2 + zero, 1) == G - 1) {
    for (int j = 0; j < d.nd; ++j) atomicExch(dispenser_word(d, j), 0ull);
    atomicExch(d.base + 2 + zero, 0);
  }
}

// Workgroup id remap for the persistent tile loop: dispatch places block b on
// XCD b % 8, so consecutive virtual ids go to one XCD and the tiles that share
// an expert's weight tile share that XCD's L2.
__device__ __forceinline__ int xcd_virtual_block() {
  const int G = gridDim.x;
  return (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
}

// Epilogue of the down GEMM (weighted scatter) shared by the tiled kernels,
// whose 8 waves each hold 128 columns x BM/4 rows of the 256 x BM tile (lane:
// 4 consecutive columns of one row per 16-column sub-tile ni, sub-tile ti of
// 16 rows).  Row r of the tile is scaled by its slot's routing weight, rounded
// to bf16 and written to slot_out[slot][256 n_tile ...].  The rows are staged in
// the stage area (free once every wave is past the K loop) at a padded pitch
// and leave as whole 512-byte row segments, 16 bytes per lane: stored straight
// from the accumulators, each lane's 8-byte pieces would reach memory as
// partial lines.  srow: BM ints of LDS scratch.
constexpr int kOutPitch = 528;  // bytes per staged row: 512 + 16 (fewer bank conflicts)

// Second half of the staged scatter: ROWS staged rows (bf16, pitch
// kOutPitch) leave as COLS * 2-byte row segments to slot_out[srow[r]][col0 ...];
// rows with srow < 0 are skipped.  Staging must be complete (barrier) on entry.
template <int ROWS, int COLS = 256>
__device__ __forceinline__ void copy_out_staged_rows(const GemmParams& p, const uint8_t* area, const int* srow,
                                                     int col0, int tid) {
  constexpr int LPR = COLS / 8;        // lanes per row, 8 columns each
  constexpr int RPP = 8 * 64 / LPR;    // rows per pass of the 8 waves
  const int wave = tid >> 6, lane = tid & 63;
  const int N = p.N;
  // wave w, pass j: tile row RPP j + (64 / LPR) w + lane / LPR
  const int n0 = col0 + (lane % LPR) * 8;
#pragma unroll 4
  for (int j = 0; j < ROWS / RPP; ++j) {
    const int tr = RPP * j + (64 / LPR) * wave + lane / LPR;
    const int slot = srow[tr];
    if (slot >= 0 && n0 < N) {
      const int4 v = *(const int4*)(area + tr * kOutPitch + (lane % LPR) * 16);
      *(int4*)(p.slot_out + (size_t)slot * N + n0) = v;
    }
  }
}

// The weighted scatter of a tile's outputs: NW 16-column groups per wave (8: a
// 256-column n-tile, the two waves of a token quarter 128 columns each; 4: one
// 128-column half, starting at column col0 of the output).
template <int BM, int NW = 8, typename V>
__device__ __forceinline__ void scatter_rows_staged(const GemmParams& p, uint8_t* area, int* srow,
                                                    const V (&acc)[NW][BM / 64], int col0, int m0, int m_end,
                                                    int tid) {
  constexpr int WM = BM / 4, TS = WM / 16;
  const int wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wt = wave >> 1, g = lane >> 4, l16 = lane & 15;
  __syncthreads();  // every wave is done reading the stages
  if (tid < BM) srow[tid] = m0 + tid < m_end ? p.slot_of_row[m0 + tid] : -1;
#pragma unroll
  for (int ti = 0; ti < TS; ++ti) {
    const int tr = wt * WM + ti * 16 + l16;
    const int r = m0 + tr;
    const float w = r < m_end ? p.top_k_weights[p.slot_of_row[r]] : 0.0f;
#pragma unroll
    for (int ni = 0; ni < NW; ++ni) {
      const V v = acc[ni][ti] * w;
      uint2 o;
      o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *(uint2*)(area + tr * kOutPitch + (wn * NW * 16 + ni * 16 + 4 * g) * 2) = o;
    }
  }
  __syncthreads();
  copy_out_staged_rows<BM, NW * 32>(p, area, srow, col0, tid);
}

// SwiGLU epilogues: a tile's h codes are BM sorted rows x 128 bytes of one
// K-block plane of the down GEMM's operand ([I/128][rows][128]), so they form
// one contiguous block in memory.  They are staged in the stage area (free
// once every wave is past the K loop) at a padded pitch and leave 16 bytes per
// lane, in whole 128-byte rows; rows at or past m_end are not written (they
// belong to the next expert).  Staging must be complete (barrier) on entry.
constexpr int kHPitch = 144;  // bytes per staged code row: 128 + 16 (no bank conflicts)

template <int BM>
__device__ __forceinline__ void copy_out_h_codes(const GemmParams& p, const uint8_t* area, int n_tile, int m0,
                                                 int m_end, int tid) {
  uint8_t* plane = p.h_codes + (size_t)n_tile * p.max_rows * 128;
#pragma unroll
  for (int i = tid; i < BM * 8; i += 512) {
    const int tr = i >> 3, c = i & 7;
    if (m0 + tr < m_end)
      *(int4*)(plane + (size_t)(m0 + tr) * 128 + c * 16) = *(const int4*)(area + tr * kHPitch + c * 16);
  }
}

}  // namespace moe
