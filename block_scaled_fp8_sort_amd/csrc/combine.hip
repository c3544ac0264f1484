// Deterministic combine of the k weighted slot outputs of each token.
//
// The pages' forward ends with weighted_out.view(T, k, H).sum(dim=1) after the
// sentinel rows were zeroed, and casts to the input dtype; a reshape+sum is used
// instead of index_add_ because atomic adds with duplicate indices are not
// deterministic ("grouped_mm experts dispatch does not support
// activation_scheme='static'", section "Source").  Here the slot rows of a token
// (already multiplied by their routing weight in the down GEMM's epilogue) are
// added in ascending j in fp32 and rounded once to bf16.  Skipped slots are never
// read: their rows were never written, so whatever they hold (NaN included)
// cannot reach the sum.  HBM-bound: 16-byte loads and stores, 8 bf16 per lane.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ slot_out,
                                                      const int32_t* __restrict__ ids, int32_t T, int32_t k,
                                                      int32_t H8, int32_t E, int32_t expert_begin,
                                                      uint4* __restrict__ out) {
  const int64_t n = (int64_t)T * H8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += stride) {
    const int64_t t = c / H8;
    const int64_t col = c - t * H8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int64_t local = (int64_t)ids[t * k + j] - expert_begin;
      if (local < 0 || local >= E) continue;
      const uint4 v = slot_out[(t * k + j) * H8 + col];
      acc[0] += bf16_bits_to_f32(v.x & 0xFFFF);
      acc[1] += bf16_bits_to_f32(v.x >> 16);
      acc[2] += bf16_bits_to_f32(v.y & 0xFFFF);
      acc[3] += bf16_bits_to_f32(v.y >> 16);
      acc[4] += bf16_bits_to_f32(v.z & 0xFFFF);
      acc[5] += bf16_bits_to_f32(v.z >> 16);
      acc[6] += bf16_bits_to_f32(v.w & 0xFFFF);
      acc[7] += bf16_bits_to_f32(v.w >> 16);
    }
    uint4 o;
    o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
    out[c] = o;
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* slot_out, const int32_t* ids, int32_t T, int32_t k, int32_t H, int32_t E,
                          int32_t expert_begin, uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t want = (n + threads - 1) / threads;
  const int blocks = (int)(want < 256 * 32 ? want : 256 * 32);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(threads), 0, stream, (const uint4*)slot_out, ids, T, k,
                     H / 8, E, expert_begin, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
