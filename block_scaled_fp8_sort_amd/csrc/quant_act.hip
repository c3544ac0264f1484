// Per-block activation quantization of bf16 rows.
//
// The pages' grouped experts dispatch quantizes activations dynamically per
// block, and the eager one also takes the static scheme's precomputed scales
// ("grouped_mm experts dispatch does not support activation_scheme='static'",
// sections "What it means" and "Example fix"); both are served here, the
// static one by reading the caller's block scales instead of the amax.  Block
// rule:
//  FP8_B128 (blocks of 128): s = max(amax, 1e-4) / 448 (fp32), code = e4m3(x / s)
//  with x / s the IEEE fp32 quotient, so codes match a host implementation bit
//  for bit (computed from one reciprocal per block, see quant_chunk).
//  MX (blocks of 32): s = 2^e, e = ceil(log2(max(amax, 1e-4) / 448)) from the
//  fp32 bits, stored as the byte e + 127; code = e4m3(x * 2^-e), exact scaling.
//
// Output layout (the grouped GEMM's operand layout): K-block-major, codes
// [H/128][rows][128 bytes] and scales [H/128][rows] (FP8_B128) or
// [H/128][rows][4 bytes] (MX: the four UE8M0 bytes of a row's 128-wide block).  One 128-wide block of a row is 128 contiguous bytes, and the blocks of
// different rows for the same K range sit side by side.
//
// The kernel is HBM-bound (2 bytes in, 1 byte + a scale out per element): each
// lane reads 16 contiguous bytes (8 bf16), the lanes of one block reduce the
// amax with xor butterflies, and each lane stores its 8 codes as one 8-byte
// store (16 lanes cover one 128-byte block row).  Quantizing the T token rows
// once and gathering codes by index later is the same as gathering first (the
// rule is row-local).
#include "device_common.h"
#include "internal.h"
#include "quant_act.h"

namespace moe {

namespace {

template <int BLOCK, bool STATIC>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint4* __restrict__ x, int64_t n_chunks, int32_t rows,
                                                        int32_t H, uint8_t* __restrict__ codes,
                                                        void* __restrict__ scales, StaticScales st) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // n_chunks and the stride are multiples of the lanes of one block, so every
  // lane group stays together
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks; c += stride)
    quant_chunk<BLOCK, STATIC>(x, c, rows, H, codes, scales, st);
}

// The activation scales by sorted row: dst[kb][r] = scales[kb][sorted_slot[r] / k]
// for every K block kb and sorted row r < S (fp32 scales, or the four UE8M0
// bytes of a row's 128-wide block as one word).  Writes are contiguous over r;
// the reads gather from the token scales, which stay in the L2.
__global__ __launch_bounds__(256) void gather_scales_kernel(const uint32_t* __restrict__ scales,
                                                            const int32_t* __restrict__ sorted_slot, int32_t k,
                                                            int32_t T, int32_t S, int64_t n,
                                                            uint32_t* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t kb = i / S;
    const int32_t r = (int32_t)(i - kb * S);
    dst[i] = scales[kb * T + sorted_slot[r] / k];
  }
}

}  // namespace

hipError_t launch_gather_scales(const void* scales, const int32_t* sorted_slot, int32_t k, int32_t T, int32_t H,
                                void* dst, hipStream_t stream) {
  const int32_t S = T * k;
  const int64_t n = (int64_t)(H / 128) * S;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(gather_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint32_t*)scales,
                     sorted_slot, k, T, S, n, (uint32_t*)dst);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int32_t rows, int32_t H, int fmt, uint8_t* codes, void* scales,
                            hipStream_t stream, const StaticScales* st) {
  const int64_t n_chunks = (int64_t)rows * H / 8;
  if (n_chunks == 0) return hipSuccess;
  const int threads = 256;
  const int64_t want = (n_chunks + threads - 1) / threads;
  const int blocks = (int)(want < 256 * 64 ? want : 256 * 64);
  const dim3 g(blocks), b(threads);
  const StaticScales none{nullptr, 0};
  if (fmt == 0) {
    if (st)
      hipLaunchKernelGGL((quant_act_kernel<128, true>), g, b, 0, stream, (const uint4*)x, n_chunks, rows, H, codes,
                         scales, *st);
    else
      hipLaunchKernelGGL((quant_act_kernel<128, false>), g, b, 0, stream, (const uint4*)x, n_chunks, rows, H, codes,
                         scales, none);
  } else {
    if (st)
      hipLaunchKernelGGL((quant_act_kernel<32, true>), g, b, 0, stream, (const uint4*)x, n_chunks, rows, H, codes,
                         scales, *st);
    else
      hipLaunchKernelGGL((quant_act_kernel<32, false>), g, b, 0, stream, (const uint4*)x, n_chunks, rows, H, codes,
                         scales, none);
  }
  return hipGetLastError();
}

}  // namespace moe
