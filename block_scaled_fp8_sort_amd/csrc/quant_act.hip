// Dynamic per-block activation quantization of bf16 rows.
//
// The grouped experts dispatch quantizes activations dynamically per block and
// cannot take precomputed scales ("grouped_mm experts dispatch does not support
// activation_scheme='static'", section "What it means").  Block rule:
//  FP8_B128 (blocks of 128): s = max(amax, 1e-4) / 448 (fp32), code = e4m3(x / s)
//  with an IEEE fp32 division, so codes match a host implementation bit for bit.
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

namespace moe {

namespace {

template <int BLOCK>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint4* __restrict__ x, int64_t n_chunks, int32_t rows,
                                                        int32_t H, uint8_t* __restrict__ codes,
                                                        void* __restrict__ scales) {
  constexpr int kLanesPerBlock = BLOCK / 8;  // 16 (FP8_B128) or 4 (MX)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // n_chunks is a multiple of kLanesPerBlock and every lane group stays together
  const int H8 = H / 8;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
    const uint4 v = x[c];
    const int64_t row = c / H8;
    const int col8 = (int)(c - row * H8);
    const int64_t blk128 = col8 / 16;  // K-block plane
    uint2* dst = (uint2*)(codes + (blk128 * rows + row) * 128 + (col8 % 16) * 8);
    float f[8];
    f[0] = bf16_bits_to_f32(v.x & 0xFFFF);
    f[1] = bf16_bits_to_f32(v.x >> 16);
    f[2] = bf16_bits_to_f32(v.y & 0xFFFF);
    f[3] = bf16_bits_to_f32(v.y >> 16);
    f[4] = bf16_bits_to_f32(v.z & 0xFFFF);
    f[5] = bf16_bits_to_f32(v.z >> 16);
    f[6] = bf16_bits_to_f32(v.w & 0xFFFF);
    f[7] = bf16_bits_to_f32(v.w >> 16);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
#pragma unroll
    for (int m = 1; m < kLanesPerBlock; m <<= 1) amax = wave_max_xor(amax, m);
    uint2 out;
    if constexpr (BLOCK == 128) {
      const float s = fp8_block_scale(amax);
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = f[i] / s;  // IEEE division
      out.x = e4m3x4(q[0], q[1], q[2], q[3]);
      out.y = e4m3x4(q[4], q[5], q[6], q[7]);
      if ((col8 % kLanesPerBlock) == 0) ((float*)scales)[blk128 * rows + row] = s;
    } else {
      const int e = mx_block_exponent(amax);
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = __builtin_ldexpf(f[i], -e);
      out.x = e4m3x4(q[0], q[1], q[2], q[3]);
      out.y = e4m3x4(q[4], q[5], q[6], q[7]);
      if ((col8 % kLanesPerBlock) == 0)
        ((uint8_t*)scales)[(blk128 * rows + row) * 4 + (col8 % 16) / 4] = (uint8_t)(e + 127);
    }
    *dst = out;
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int32_t rows, int32_t H, int fmt, uint8_t* codes, void* scales,
                            hipStream_t stream) {
  const int64_t n_chunks = (int64_t)rows * H / 8;
  if (n_chunks == 0) return hipSuccess;
  const int threads = 256;
  const int64_t want = (n_chunks + threads - 1) / threads;
  const int blocks = (int)(want < 256 * 64 ? want : 256 * 64);
  if (fmt == 0)
    hipLaunchKernelGGL(quant_act_kernel<128>, dim3(blocks), dim3(threads), 0, stream, (const uint4*)x, n_chunks,
                       rows, H, codes, scales);
  else
    hipLaunchKernelGGL(quant_act_kernel<32>, dim3(blocks), dim3(threads), 0, stream, (const uint4*)x, n_chunks, rows,
                       H, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
