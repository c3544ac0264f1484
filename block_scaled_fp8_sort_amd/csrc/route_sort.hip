// Route sort: stable counting sort of the flat (token, slot) pairs by expert.
//
// The pages' grouped forward sorts the flattened expert ids and gathers token
// rows by perm // k ("grouped_mm experts dispatch does not support
// activation_scheme='static'", section "Source").  Here the key of slot s is its
// local expert id, or the sentinel E for a skipped slot (-1, or an id outside
// this GPU's range), and equal keys keep ascending s, so the permutation is
// unique and sentinels come last.
//
// One workgroup of 16 wavefronts.  Wave w owns a contiguous chunk of slots.
//  1. Each wave histograms its chunk into its own LDS row hist[w][0..E].
//  2. Column-wise exclusive prefix: start[w][e] = offsets[e] + sum_{w'<w} hist[w'][e],
//     with offsets[e] the exclusive prefix of the key totals.
//  3. Each wave walks its chunk 64 slots at a time, in order.  Lanes holding the
//     same key find each other with one ballot per key bit; a lane's position is
//     start[w][key] + (number of lower lanes with its key), and the lowest such
//     lane then advances start[w][key].  Order inside a key is therefore slot
//     order, as a stable sort requires.
// Small inputs (decode) run all three steps in one workgroup.  Large inputs
// split the slots over up to kMaxChunks chunks of at least 256 slots, one wave
// each, in three launches:
//  A. each wave histograms its chunk and writes it key-major, hist[key][chunk];
//  B. one wave per key turns its row into the exclusive prefix over the chunks
//     and writes the row total;
//  C. each wave scans the E + 1 totals into offsets[key], so that its start is
//     offsets[key] + hist[key][chunk] (all smaller keys, then the same key in
//     earlier chunks), and runs step 3 above on its chunk.
// The result is the same unique permutation in both cases.
//
// Router (optional, in front of the sort): each token's top-k is taken by one
// DPP row of 16 lanes, lane i holding the token's logits i, i + 16, ...
// Softmax is increasing in the logit, so the k most probable experts are the k
// largest logits; k rounds of an in-row (value, id) max-reduction, lower id on
// equal values, pick them in descending order.  Weights are exp(l - max) over
// the sum of the same terms, taken over all E (plain softmax) or over the k
// chosen (renormalised), in fp32.  Small batches run the router in the sort's
// own workgroup before it sorts; large ones run it as a launch of its own.
#include "device_common.h"
#include "internal.h"
#include "quant_act.h"

namespace moe {

namespace {

constexpr int kSortWaves = 16;
constexpr int kSortThreads = kSortWaves * kWave;

constexpr int kMaxChunks = 2048;      // chunks (one wave each) of the multi-block path, at most
constexpr int kMinChunk = 256;        // slots per chunk, at least
constexpr int kMultiBlockFrom = 16384;  // S at which the multi-block path takes over
constexpr int kChunkWaves = 4;        // waves per workgroup in the three steps

__device__ __forceinline__ int sort_key(int32_t id, int32_t E, int32_t expert_begin) {
  const int64_t local = (int64_t)id - expert_begin;
  return (local >= 0 && local < E) ? (int)local : E;
}

constexpr int kRouterThreads = 256;
// The sort's workgroup runs the router itself up to this many tokens and
// experts: up to 16 tokens its router rows fill at most one wave per SIMD and
// save a launch; beyond, the waves share the CU's SIMDs, and a launch of its own
// over several CUs is faster (64 tokens of 128 experts: router + sort 10.4 us
// against 12.4 us in the sort's workgroup).
constexpr int kRouterFusedMaxT = 16;
constexpr int kRouterFusedMaxE = 128;
constexpr int kRouterLanes = 16;           // lanes per token: one DPP row

// All-reduce step s (0..3) of a DPP row: exchange with lane i ^ 1, i ^ 2, then
// the mirrored lane in the half row (i ^ 7) and in the row (i ^ 15).  After the
// four steps every lane of the row holds the combination of all 16; the
// partners are symmetric, so every lane computes the same bits.
__device__ __forceinline__ int dpp_step(int v, int s) {
  switch (s) {
    case 0: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    default: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  }
}
__device__ __forceinline__ float dpp_step_f(float v, int s) { return __int_as_float(dpp_step(__float_as_int(v), s)); }

// Top-k of tokens, one DPP row of 16 lanes per token: lane i of the row holds
// logits e = i + 16 v, v < NV (NV >= ceil(E / 16)).  Rows of a wave take tokens
// wave_id * 4 + row, stepping by n_waves * 4.  All lanes of a row take the same
// path, so the row never reads an idle lane.
template <int NV>
__device__ __forceinline__ void router_tokens(const RouterArgs r, int32_t T, int32_t k, int wave_id, int n_waves) {
  const int E = r.n_experts;
  const int lane = threadIdx.x % kWave;
  const int lig = lane & (kRouterLanes - 1);
  constexpr int kPerWave = kWave / kRouterLanes;
  constexpr int kNone = 0x7FFFFFFF;
  const float ninf = -__builtin_inff();
  for (int64_t t = (int64_t)wave_id * kPerWave + lane / kRouterLanes; t < T; t += (int64_t)n_waves * kPerWave) {
    const float* row = r.logits + t * E;
    float vals[NV];
    uint32_t avail = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = lig + v * kRouterLanes;
      vals[v] = ninf;
      if (e < E) {
        vals[v] = row[e];
        avail |= 1u << v;
      }
    }
    float m = ninf;
#pragma unroll
    for (int v = 0; v < NV; ++v) m = __builtin_fmaxf(m, vals[v]);  // absent values are -inf
#pragma unroll
    for (int st = 0; st < 4; ++st) m = __builtin_fmaxf(m, dpp_step_f(m, st));
    float z = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if ((avail >> v) & 1) z += expf(vals[v] - m);
#pragma unroll
    for (int st = 0; st < 4; ++st) z += dpp_step_f(z, st);

    // k rounds; pick j = 16 c + i is kept by lane i of the row in slot c
    int pick_id[4] = {0, 0, 0, 0};
    float pick_val[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float sel = 0.0f;  // sum of exp(pick - m) over the picks, in pick order
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c * kRouterLanes >= k) break;
      const int jn = min(k - c * kRouterLanes, kRouterLanes);
      for (int jj = 0; jj < jn; ++jj) {
        // the lane's best remaining logit (v, hence e, ascending: lowest e
        // among equals); a lane with none left offers (-inf, kNone), which
        // loses to any real logit (logits are finite)
        float bv = ninf;
        int be = kNone;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const bool take = ((avail >> v) & 1) && (be == kNone || vals[v] > bv);
          bv = take ? vals[v] : bv;
          be = take ? lig + v * kRouterLanes : be;
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float ov = dpp_step_f(bv, st);
          const int oe = dpp_step(be, st);
          const bool take = ov > bv || (ov == bv && oe < be);
          bv = take ? ov : bv;
          be = take ? oe : be;
        }
        if ((be & (kRouterLanes - 1)) == lig) avail &= ~(1u << (be / kRouterLanes));
        sel += expf(bv - m);
        if (lig == jj) {
          pick_id[c] = be;
          pick_val[c] = bv;
        }
      }
    }
    const float denom = r.renormalize ? sel : z;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = c * kRouterLanes + lig;
      if (j < k) {
        r.ids[t * k + j] = pick_id[c];
        r.weights[t * k + j] = expf(pick_val[c] - m) / denom;
      }
    }
  }
}
template <int NV>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(const RouterArgs r, int32_t T, int32_t k) {
  const int wave = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kWave);
  router_tokens<NV>(r, T, k, wave, (int)(gridDim.x * blockDim.x / kWave));
}

// One 64-slot step of a wave's stable scatter: lane i holds slot s (valid if
// active) with its key; start[key] is where the wave's next slot of that key
// goes (advanced in place, in LDS).
__device__ __forceinline__ void scatter_step(int s, bool active, int key, int key_bits, int32_t* start,
                                             int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos) {
  const int lane = threadIdx.x % kWave;
  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t peers = __ballot(active);
  for (int b = 0; b < key_bits; ++b) {
    const uint64_t m = __ballot(active && ((key >> b) & 1));
    peers &= ((key >> b) & 1) ? m : ~m;
  }
  if (active) {
    const int st = start[key];
    const int pos = st + __popcll(peers & lower_lanes);
    sorted_slot[pos] = s;
    if (slot_pos) slot_pos[s] = pos;
    // the lowest lane of each key group advances the start after all lanes read it
    const bool leader = (peers & lower_lanes) == 0;
    __builtin_amdgcn_wave_barrier();
    if (leader) start[key] = st + __popcll(peers);
  }
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int key_bits_for(int32_t E) {
  int key_bits = 1;
  while ((1 << key_bits) <= E) ++key_bits;
  return key_bits;
}

// Stable scatter of slots [c_begin, c_end) by one wave.
__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ ids, int c_begin, int c_end, int32_t E,
                                              int32_t expert_begin, int32_t* start, int32_t* __restrict__ sorted_slot,
                                              int32_t* __restrict__ slot_pos) {
  const int lane = threadIdx.x % kWave;
  const int key_bits = key_bits_for(E);
  for (int s0 = c_begin; s0 < c_end; s0 += kWave) {
    const int s = s0 + lane;
    const bool active = s < c_end;
    const int key = active ? sort_key(ids[s], E, expert_begin) : 0;
    scatter_step(s, active, key, key_bits, start, sorted_slot, slot_pos);
  }
}

// Step A: hist[key][chunk] for keys 0..E, and the invalid ids of the chunk in
// row E + 1.
__global__ __launch_bounds__(kChunkWaves * kWave) void sort_hist_kernel(const int32_t* __restrict__ ids, int32_t S,
                                                                       int32_t E, int32_t expert_begin, int32_t chunk,
                                                                       int32_t n_chunks, int32_t* __restrict__ hist,
                                                                       int32_t* __restrict__ zero, int32_t n_zero) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  extern __shared__ int32_t lh[];  // [kChunkWaves][E + 2]
  const int K2 = E + 2;
  const int wl = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x * kChunkWaves + wl;
  for (int i = threadIdx.x; i < kChunkWaves * K2; i += blockDim.x) lh[i] = 0;
  __syncthreads();
  if (c < n_chunks) {
    const int c_begin = min(S, c * chunk), c_end = min(S, c_begin + chunk);
    int bad = 0;
    for (int s = c_begin + lane; s < c_end; s += kWave) {
      const int32_t id = ids[s];
      const int key = sort_key(id, E, expert_begin);
      bad += (key == E && id != -1) ? 1 : 0;
      atomicAdd(&lh[wl * K2 + key], 1);
    }
    if (bad) atomicAdd(&lh[wl * K2 + E + 1], bad);
  }
  __syncthreads();
  if (c < n_chunks)
    for (int e = lane; e < K2; e += kWave) hist[(size_t)e * n_chunks + c] = lh[wl * K2 + e];
}

// Exclusive prefix sum over the wave of one value per lane, and the wave total.
__device__ __forceinline__ int wave_exclusive_scan(int v, int lane, int& total) {
  int incl = v;
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  total = __shfl(incl, kWave - 1, kWave);
  return incl - v;
}

// Step B: one wave per row e of hist (keys 0..E and the invalid row E + 1):
// the row becomes its exclusive prefix sum over the chunks, in place, and its
// total goes to totals[e].
__global__ __launch_bounds__(kChunkWaves * kWave) void sort_rowscan_kernel(int32_t E, int32_t n_chunks,
                                                                          int32_t* __restrict__ hist,
                                                                          int32_t* __restrict__ totals) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * kChunkWaves + threadIdx.x / kWave;
  if (e > E + 1) return;  // whole waves only; no workgroup barrier here
  int32_t* row = hist + (size_t)e * n_chunks;
  int run = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += kWave) {
    const int c = c0 + lane;
    const int v = c < n_chunks ? row[c] : 0;
    int sum;
    const int ex = wave_exclusive_scan(v, lane, sum);
    if (c < n_chunks) row[c] = run + ex;
    run += sum;
  }
  if (lane == 0) totals[e] = run;
}

// Step C: each wave scans the key totals itself (E + 1 values: a few per lane,
// then a shuffle scan), adds its chunk's row prefix to get its start per key,
// and scatters its chunk.  Chunk 0's wave also writes the offsets and the
// invalid count.
__global__ __launch_bounds__(kChunkWaves * kWave) void sort_scatter_kernel(
    const int32_t* __restrict__ ids, int32_t S, int32_t E, int32_t expert_begin, int32_t chunk, int32_t n_chunks,
    const int32_t* __restrict__ start, const int32_t* __restrict__ totals, int32_t* __restrict__ offsets,
    int32_t* __restrict__ invalid_count, int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos) {
  extern __shared__ int32_t ls[];  // [kChunkWaves][E + 1]
  const int K1 = E + 1;
  const int wl = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x * kChunkWaves + wl;
  if (c >= n_chunks) return;  // whole waves only; no workgroup barrier follows
  int32_t* my = ls + wl * K1;
  const int per = (K1 + kWave - 1) / kWave;
  const int e0 = lane * per;
  int lsum = 0;
  for (int i = 0; i < per; ++i)
    if (e0 + i < K1) {
      const int t = totals[e0 + i];
      my[e0 + i] = t;
      lsum += t;
    }
  int unused;
  int run = wave_exclusive_scan(lsum, lane, unused);
  for (int i = 0; i < per; ++i)
    if (e0 + i < K1) {
      const int t = my[e0 + i];
      my[e0 + i] = run;
      if (c == 0) offsets[e0 + i] = run;
      run += t;
    }
  if (c == 0 && lane == 0 && invalid_count) invalid_count[0] = totals[K1];
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < K1; e += kWave) my[e] += start[(size_t)e * n_chunks + c];
  __builtin_amdgcn_wave_barrier();
  const int c_begin = min(S, c * chunk), c_end = min(S, c_begin + chunk);
  scatter_chunk(ids, c_begin, c_end, E, expert_begin, my, sorted_slot, slot_pos);
}

// Chunk size of the multi-block path: at least kMinChunk, a multiple of the
// wave size, and at most kMaxChunks chunks.
int32_t sort_chunk(int32_t S) {
  int64_t c = ((int64_t)S + kMaxChunks - 1) / kMaxChunks;
  c = (c + kWave - 1) / kWave * kWave;
  return (int32_t)(c < kMinChunk ? kMinChunk : c);
}

// The whole sort in one workgroup of kSortThreads threads (steps 1-3 above).
__device__ __forceinline__ void sort_one_workgroup(const int32_t* __restrict__ ids, int32_t S, int32_t E,
                                                   int32_t expert_begin, int32_t* __restrict__ sorted_slot,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ slot_pos,
                                                   int32_t* __restrict__ invalid_count) {
  extern __shared__ int32_t hist[];  // [kSortWaves][E + 1], then the key totals [E + 1]
  __shared__ int32_t s_invalid;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int K1 = E + 1;
  int32_t* total = hist + kSortWaves * K1;

  for (int i = tid; i < kSortWaves * K1; i += kSortThreads) hist[i] = 0;
  if (tid == 0) s_invalid = 0;
  __syncthreads();

  const int chunk = (S + kSortWaves - 1) / kSortWaves;
  const int c_begin = min(S, wave * chunk);
  const int c_end = min(S, c_begin + chunk);

  // the wave's keys, all loads in flight at once (at most kSteps per lane, as
  // S < kMultiBlockFrom), kept in registers for both passes
  constexpr int kSteps = (kMultiBlockFrom / kSortWaves + kWave - 1) / kWave;
  int keys[kSteps];
  int my_invalid = 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int s = c_begin + lane + i * kWave;
    const int32_t id = s < c_end ? ids[s] : -1;
    keys[i] = sort_key(id, E, expert_begin);
    my_invalid += (keys[i] == E && id != -1) ? 1 : 0;
  }

  // 1. per-wave histogram
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
    if (c_begin + lane + i * kWave < c_end) atomicAdd(&hist[wave * K1 + keys[i]], 1);
  if (my_invalid) atomicAdd(&s_invalid, my_invalid);
  __syncthreads();

  // 2. key totals, exclusive scan over keys, then per-wave starts
  for (int e = tid; e < K1; e += kSortThreads) {
    int t = 0;
    for (int w = 0; w < kSortWaves; ++w) t += hist[w * K1 + e];
    total[e] = t;
  }
  __syncthreads();
  // exclusive scan of total[0..K1) by wave 0 alone (K1 <= 513: at most 9
  // entries per lane, then a shuffle scan of the lane sums), with no workgroup
  // barrier inside
  if (wave == 0) {
    const int per = (K1 + kWave - 1) / kWave;
    const int e0 = lane * per;
    int lsum = 0;
    for (int i = 0; i < per; ++i)
      if (e0 + i < K1) lsum += total[e0 + i];
    int incl = lsum;
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    int run = incl - lsum;
    for (int i = 0; i < per; ++i)
      if (e0 + i < K1) {
        const int v = total[e0 + i];
        total[e0 + i] = run;
        run += v;
      }
  }
  __syncthreads();
  for (int e = tid; e < K1; e += kSortThreads) {
    int run = total[e];
    offsets[e] = run;
    for (int w = 0; w < kSortWaves; ++w) {
      const int h = hist[w * K1 + e];
      hist[w * K1 + e] = run;
      run += h;
    }
  }
  if (tid == 0 && invalid_count) invalid_count[0] = s_invalid;
  __syncthreads();

  // 3. stable scatter, 64 slots per step, in slot order within each wave
  const int key_bits = key_bits_for(E);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int s0 = c_begin + i * kWave;
    if (s0 < c_end)  // wave-uniform
      scatter_step(s0 + lane, s0 + lane < c_end, keys[i], key_bits, hist + wave * K1, sorted_slot, slot_pos);
  }
}

// The router's writes of ids reach the sort's reads through the workgroup
// barrier (workgroup-scope release/acquire covers global memory too).
__device__ __forceinline__ void router_in_workgroup(const RouterArgs& router, int32_t T, int32_t k) {
  if (router.logits) {
    router_tokens<kRouterFusedMaxE / kRouterLanes>(router, T, k, threadIdx.x / kWave, kSortWaves);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(const RouterArgs router,
                                                                   const int32_t* ids, int32_t T, int32_t k,
                                                                   int32_t E, int32_t expert_begin,
                                                                   int32_t* __restrict__ sorted_slot,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ slot_pos,
                                                                   int32_t* __restrict__ invalid_count,
                                                                   int32_t* __restrict__ zero, int32_t n_zero) {
  for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  router_in_workgroup(router, T, k);
  sort_one_workgroup(ids, T * k, E, expert_begin, sorted_slot, offsets, slot_pos, invalid_count);
}

// Small batches: the sort and the activation quantization are independent and
// each too small to fill the chip, so one launch runs both: workgroup 0 sorts,
// the next q_blocks quantize (a grid-stride loop whose stride is a multiple of
// the lanes of one quantization block).  Workgroups that read the start of the
// next GEMM's weights into the last-level cache while the sorting workgroup
// runs saved 1 us of the Qwen3-MoE decode forward while that GEMM's weight
// loads were plain; with the nontemporal hint on them the read-ahead cost
// 0.4-0.7 us instead, so there is none.
template <int BLOCK, bool STATIC>
__global__ __launch_bounds__(kSortThreads) void route_quant_kernel(
    const RouterArgs router, const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t expert_begin,
    int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ offsets, int32_t* __restrict__ invalid_count, const uint4* __restrict__ x,
    int64_t n_chunks, int32_t rows, int32_t H, uint8_t* __restrict__ codes, void* __restrict__ scales,
    int32_t* __restrict__ zero, int32_t n_zero, StaticScales st, int32_t q_blocks) {
  if (blockIdx.x == 1 || gridDim.x == 1)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  if (blockIdx.x == 0) {
    router_in_workgroup(router, T, k);
    sort_one_workgroup(ids, T * k, E, expert_begin, sorted_slot, offsets, nullptr, invalid_count);
    return;
  }
  const int64_t stride = (int64_t)q_blocks * blockDim.x;
  for (int64_t c = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; c < n_chunks; c += stride)
    quant_chunk<BLOCK, STATIC>(x, c, rows, H, codes, scales, st);
}

}  // namespace

size_t route_sort_lds_bytes(int32_t E) { return sizeof(int32_t) * (size_t)(kSortWaves + 1) * (E + 1); }

bool route_sort_multiblock(int32_t S) { return S >= kMultiBlockFrom; }

size_t route_sort_ws_bytes(int32_t S, int32_t E) {
  if (S < kMultiBlockFrom) return 0;
  const int32_t chunk = sort_chunk(S);
  const size_t n_chunks = ((size_t)S + chunk - 1) / chunk;
  return sizeof(int32_t) * (size_t)(E + 2) * (n_chunks + 1);  // hist rows, then the row totals
}

namespace {

const RouterArgs kNoRouter{nullptr, 0, 0, nullptr, nullptr};

// Whether the sort's one workgroup runs the router itself.
bool router_fused(const RouterArgs* router, int32_t T, int32_t k) {
  return (int64_t)T * k < kMultiBlockFrom && T <= kRouterFusedMaxT && router->n_experts <= kRouterFusedMaxE;
}

hipError_t launch_router(const RouterArgs& r, int32_t T, int32_t k, hipStream_t stream) {
  const int64_t per_block = kRouterThreads / kRouterLanes;  // one token per DPP row
  int64_t blocks = (T + per_block - 1) / per_block;
  if (blocks > 8192) blocks = 8192;
  const int v = (r.n_experts + kRouterLanes - 1) / kRouterLanes;
  const dim3 g((unsigned)blocks), b(kRouterThreads);
  if (v <= 1)
    hipLaunchKernelGGL(router_topk_kernel<1>, g, b, 0, stream, r, T, k);
  else if (v <= 2)
    hipLaunchKernelGGL(router_topk_kernel<2>, g, b, 0, stream, r, T, k);
  else if (v <= 4)
    hipLaunchKernelGGL(router_topk_kernel<4>, g, b, 0, stream, r, T, k);
  else if (v <= 8)
    hipLaunchKernelGGL(router_topk_kernel<8>, g, b, 0, stream, r, T, k);
  else if (v <= 16)
    hipLaunchKernelGGL(router_topk_kernel<16>, g, b, 0, stream, r, T, k);
  else
    hipLaunchKernelGGL(router_topk_kernel<32>, g, b, 0, stream, r, T, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_only(const RouterArgs& router, int32_t T, int32_t k, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  return launch_router(router, T, k, stream);
}

hipError_t launch_route_sort(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets, int32_t* slot_pos,
                             int32_t* invalid_count, void* ws, hipStream_t stream) {
  return launch_route_sort_zero(router, ids, T, k, E, expert_begin, sorted_slot, offsets, slot_pos, invalid_count,
                                ws, nullptr, 0, stream);
}

hipError_t launch_route_sort_zero(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                                  int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets, int32_t* slot_pos,
                                  int32_t* invalid_count, void* ws, int32_t* zero, int32_t n_zero,
                                  hipStream_t stream) {
  if (router && !router->logits) router = nullptr;
  const int32_t S = T * k;
  if (S < kMultiBlockFrom) {
    const bool fuse = router && router_fused(router, T, k);
    if (router && !fuse) {
      hipError_t e = launch_router(*router, T, k, stream);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(kSortThreads), route_sort_lds_bytes(E), stream,
                       fuse ? *router : kNoRouter, ids, T, k, E, expert_begin, sorted_slot, offsets, slot_pos,
                       invalid_count, zero, n_zero);
    return hipGetLastError();
  }
  if (router) {
    hipError_t e = launch_router(*router, T, k, stream);
    if (e != hipSuccess) return e;
  }
  const int32_t chunk = sort_chunk(S);
  const int32_t n_chunks = (S + chunk - 1) / chunk;
  const int blocks = (n_chunks + kChunkWaves - 1) / kChunkWaves;
  int32_t* hist = (int32_t*)ws;                         // [E + 2][n_chunks]
  int32_t* totals = hist + (size_t)(E + 2) * n_chunks;  // [E + 2]
  hipLaunchKernelGGL(sort_hist_kernel, dim3(blocks), dim3(kChunkWaves * kWave),
                     sizeof(int32_t) * kChunkWaves * (E + 2), stream, ids, S, E, expert_begin, chunk, n_chunks, hist,
                     zero, n_zero);
  hipLaunchKernelGGL(sort_rowscan_kernel, dim3((E + 2 + kChunkWaves - 1) / kChunkWaves), dim3(kChunkWaves * kWave), 0,
                     stream, E, n_chunks, hist, totals);
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(blocks), dim3(kChunkWaves * kWave),
                     sizeof(int32_t) * kChunkWaves * (E + 1), stream, ids, S, E, expert_begin, chunk, n_chunks, hist,
                     totals, offsets, invalid_count, sorted_slot, slot_pos);
  return hipGetLastError();
}

hipError_t launch_route_sort_and_quant(const RouterArgs* router, const int32_t* ids, int32_t T, int32_t k, int32_t E,
                                      int32_t expert_begin, int32_t* sorted_slot, int32_t* offsets,
                                      int32_t* invalid_count, void* sort_ws, const uint16_t* x, int32_t rows,
                                      int32_t H, int fmt, uint8_t* codes, void* scales, int32_t* zero,
                                      int32_t n_zero, hipStream_t stream, void* sorted_scales,
                                      const StaticScales* static_scales) {
  if (router && !router->logits) router = nullptr;
  const int32_t S = T * k;
  const int64_t n_chunks = (int64_t)rows * H / 8;
  if (S >= kMultiBlockFrom || n_chunks == 0) {
    hipError_t e = launch_route_sort_zero(router, ids, T, k, E, expert_begin, sorted_slot, offsets, nullptr,
                                          invalid_count, sort_ws, zero, n_zero, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_quant_act(x, rows, H, fmt, codes, scales, stream, static_scales)) != hipSuccess) return e;
    if (S >= kMultiBlockFrom && sorted_scales && rows == T)
      e = launch_gather_scales(scales, sorted_slot, k, T, H, sorted_scales, stream);
    return e;
  }
  const bool fuse = router && router_fused(router, T, k);
  if (router && !fuse) {
    hipError_t e = launch_router(*router, T, k, stream);
    if (e != hipSuccess) return e;
  }
  const RouterArgs r = fuse ? *router : kNoRouter;
  const int64_t want = (n_chunks + kSortThreads - 1) / kSortThreads;
  const int q_blocks = (int)(want < 256 * 16 ? want : 256 * 16);
  const int blocks = 1 + q_blocks;
  const StaticScales st = static_scales ? *static_scales : StaticScales{nullptr, 0};
  auto kern = fmt == 0 ? (static_scales ? route_quant_kernel<128, true> : route_quant_kernel<128, false>)
                       : (static_scales ? route_quant_kernel<32, true> : route_quant_kernel<32, false>);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kSortThreads), route_sort_lds_bytes(E), stream, r, ids, T, k, E,
                     expert_begin, sorted_slot, offsets, invalid_count, (const uint4*)x, n_chunks, rows, H, codes,
                     scales, zero, n_zero, st, q_blocks);
  return hipGetLastError();
}

}  // namespace moe
