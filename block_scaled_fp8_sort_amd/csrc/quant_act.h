// One 16-byte chunk (8 bf16) of the dynamic per-block activation quantization,
// shared by the quantization kernel and the fused route-sort + quantization
// launch used for small batches.  The rule and the output layout are described
// in quant_act.hip.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace moe {

// Chunk c of the row-major bf16 input [rows, H] (8 elements).  The BLOCK / 8
// lanes of one quantization block must run this together (they reduce the
// block's amax with xor butterflies).  With STATIC the block scale is read from
// the caller's array instead (no amax), and the encoding is the same.
template <int BLOCK, bool STATIC = false>
__device__ __forceinline__ void quant_chunk(const uint4* __restrict__ x, int64_t c, int32_t rows, int32_t H,
                                            uint8_t* __restrict__ codes, void* __restrict__ scales,
                                            StaticScales st = StaticScales{nullptr, 0}) {
  constexpr int kLanesPerBlock = BLOCK / 8;  // 16 (FP8_B128) or 4 (MX)
  const int H8 = H / 8;
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
  if constexpr (!STATIC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
#pragma unroll
    for (int m = 1; m < kLanesPerBlock; m <<= 1) amax = wave_max_xor(amax, m);
  }
  uint2 out;
  if constexpr (BLOCK == 128) {
    const float s = STATIC ? ((const float*)st.p)[row * st.stride + blk128] : fp8_block_scale(amax);
    // x / s without a division per element: one IEEE reciprocal, then the
    // product and one fma correction (div_by_scale), which rounds to the same
    // e4m3 code as the IEEE quotient for every bf16 x of the block and every
    // scale of this rule (checked exhaustively on the host).
    const float r = 1.0f / s;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_by_scale(f[i], s, r);
    out.x = e4m3x4(q[0], q[1], q[2], q[3]);
    out.y = e4m3x4(q[4], q[5], q[6], q[7]);
    if ((col8 % kLanesPerBlock) == 0) ((float*)scales)[blk128 * rows + row] = s;
  } else {
    const int e = STATIC ? (int)((const uint8_t*)st.p)[row * st.stride + col8 / 4] - 127 : mx_block_exponent(amax);
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

}  // namespace moe
