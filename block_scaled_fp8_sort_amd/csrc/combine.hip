// Deterministic combine of the k weighted slot outputs of each token.
//
// The pages' forward ends with weighted_out.view(T, k, H).sum(dim=1) after the
// sentinel rows were zeroed, and casts to the input dtype; a reshape+sum is used
// instead of index_add_ because atomic adds with duplicate indices are not
// deterministic ("grouped_mm experts dispatch does not support
// activation_scheme='static'", section "Source").  Here the slot rows of a token
// (already multiplied by their routing weight in the down GEMM's epilogue) are
// added in ascending j in fp32 and rounded once to bf16.  Skipped slots add
// nothing: their rows were never written, and whatever they hold (NaN included)
// is dropped by a select before the sum.  HBM-bound at large sizes (16-byte
// loads and stores, 8 bf16 per lane), latency-bound at decode sizes.  The slot
// rows, read once, are loaded with the nontemporal hint (DeepSeek-V3's combine
// 169 instead of 200 us, Mega-MoE's 348 instead of 406 us); with the hint on
// the output stores as well the combine ran 4-9% slower than with it on the
// loads alone.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Sum of one token's valid slot rows at 8 columns (one 16-byte chunk).  Every
// slot's load is issued before any is used (one memory round trip, which is
// what decode-sized calls are bound by); a skipped slot loads its own row,
// which exists but holds anything, and is dropped by a select, never scaled.
template <int KU>
__device__ __forceinline__ void combine_chunk(const uint4* __restrict__ slot_out, const int32_t* __restrict__ ids,
                                              int64_t t, int64_t col, int32_t k, int32_t H8, int32_t E,
                                              int32_t expert_begin, uint4* __restrict__ out, int64_t c) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += KU) {
    uint4 v[KU];
    bool ok[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int j = min(j0 + u, k - 1);
      const int64_t local = (int64_t)ids[t * k + j] - expert_begin;
      ok[u] = j0 + u < k && local >= 0 && local < E;
      const v4u x = __builtin_nontemporal_load((const v4u*)&slot_out[(t * k + j) * H8 + col]);
      v[u] = make_uint4(x.x, x.y, x.z, x.w);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += ok[u] ? bf16_bits_to_f32(w[i] & 0xFFFF) : 0.0f;
        acc[2 * i + 1] += ok[u] ? bf16_bits_to_f32(w[i] >> 16) : 0.0f;
      }
    }
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[c] = o;
}

__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ slot_out,
                                                      const int32_t* __restrict__ ids, int32_t T, int32_t k,
                                                      int32_t H8, int32_t E, int32_t expert_begin,
                                                      uint4* __restrict__ out) {
  const int64_t n = (int64_t)T * H8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += stride) {
    const int64_t t = c / H8;
    const int64_t col = c - t * H8;
    // adding +0 for a dropped slot leaves the running sum unchanged: a sum
    // that starts at +0 is never -0, the one value +0 would change
    // loads in flight per round: the smallest of 2, 4, 8, 16 that covers k
    // (a round past k repeats the last slot's load, which the select drops)
    if (k <= 2) combine_chunk<2>(slot_out, ids, t, col, k, H8, E, expert_begin, out, c);
    else if (k <= 4) combine_chunk<4>(slot_out, ids, t, col, k, H8, E, expert_begin, out, c);
    else if (k <= 8) combine_chunk<8>(slot_out, ids, t, col, k, H8, E, expert_begin, out, c);
    else combine_chunk<16>(slot_out, ids, t, col, k, H8, E, expert_begin, out, c);
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* slot_out, const int32_t* ids, int32_t T, int32_t k, int32_t H, int32_t E,
                          int32_t expert_begin, uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t want = (n + threads - 1) / threads;
  // one chunk per thread (a grid-stride loop only past 2^22 workgroups, which
  // keeps the launch under 2^32 work-items): against 8192 workgroups, the
  // DeepSeek-V3 combine took 197.6 instead of 202.5 us, Mega-MoE's 408 instead
  // of 420 us
  const int blocks = (int)(want < (1 << 22) ? want : (1 << 22));
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(threads), 0, stream, (const uint4*)slot_out, ids, T, k,
                     H / 8, E, expert_begin, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
