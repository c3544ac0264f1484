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
// The work is latency-bound (S <= a few hundred thousand int32), so one
// workgroup is enough and no global synchronization is needed.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kSortWaves = 16;
constexpr int kSortThreads = kSortWaves * kWave;

__device__ __forceinline__ int sort_key(int32_t id, int32_t E, int32_t expert_begin) {
  const int64_t local = (int64_t)id - expert_begin;
  return (local >= 0 && local < E) ? (int)local : E;
}

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(const int32_t* __restrict__ ids, int32_t S,
                                                                   int32_t E, int32_t expert_begin,
                                                                   int32_t* __restrict__ sorted_slot,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ slot_pos,
                                                                   int32_t* __restrict__ invalid_count) {
  extern __shared__ int32_t hist[];  // [kSortWaves][E + 1], then the key totals [E + 1]
  __shared__ int32_t s_invalid;
  __shared__ int32_t s_scan[kSortThreads];
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

  // 1. per-wave histogram
  int my_invalid = 0;
  for (int s = c_begin + lane; s < c_end; s += kWave) {
    const int32_t id = ids[s];
    const int key = sort_key(id, E, expert_begin);
    my_invalid += (key == E && id != -1) ? 1 : 0;
    atomicAdd(&hist[wave * K1 + key], 1);
  }
  if (my_invalid) atomicAdd(&s_invalid, my_invalid);
  __syncthreads();

  // 2. key totals, exclusive scan over keys, then per-wave starts
  for (int e = tid; e < K1; e += kSortThreads) {
    int t = 0;
    for (int w = 0; w < kSortWaves; ++w) t += hist[w * K1 + e];
    total[e] = t;
  }
  __syncthreads();
  // exclusive scan of total[0..K1) in blocks of kSortThreads
  int carry = 0;
  for (int base = 0; base < K1; base += kSortThreads) {
    const int e = base + tid;
    const int v = e < K1 ? total[e] : 0;
    s_scan[tid] = v;
    __syncthreads();
    for (int d = 1; d < kSortThreads; d <<= 1) {
      const int add = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int incl = s_scan[tid];
    const int block_sum = s_scan[kSortThreads - 1];
    __syncthreads();
    if (e < K1) total[e] = carry + incl - v;  // exclusive prefix
    carry += block_sum;
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
  int key_bits = 1;
  while ((1 << key_bits) <= E) ++key_bits;
  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = c_begin; s0 < c_end; s0 += kWave) {
    const int s = s0 + lane;
    const bool active = s < c_end;
    const int key = active ? sort_key(ids[s], E, expert_begin) : 0;
    uint64_t peers = __ballot(active);
    for (int b = 0; b < key_bits; ++b) {
      const uint64_t m = __ballot(active && ((key >> b) & 1));
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    if (active) {
      const int start = hist[wave * K1 + key];
      const int pos = start + __popcll(peers & lower_lanes);
      sorted_slot[pos] = s;
      if (slot_pos) slot_pos[s] = pos;
      // the lowest lane of each key group advances the start after all lanes read it
      const bool leader = (peers & lower_lanes) == 0;
      __builtin_amdgcn_wave_barrier();
      if (leader) hist[wave * K1 + key] = start + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

size_t route_sort_lds_bytes(int32_t E) { return sizeof(int32_t) * (size_t)(kSortWaves + 1) * (E + 1); }

hipError_t launch_route_sort(const int32_t* ids, int32_t S, int32_t E, int32_t expert_begin, int32_t* sorted_slot,
                             int32_t* offsets, int32_t* slot_pos, int32_t* invalid_count, hipStream_t stream) {
  hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(kSortThreads), route_sort_lds_bytes(E), stream, ids, S, E,
                     expert_begin, sorted_slot, offsets, slot_pos, invalid_count);
  return hipGetLastError();
}

}  // namespace moe
