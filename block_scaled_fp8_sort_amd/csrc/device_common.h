// Device helpers shared by the gfx950 kernels: bf16 and e4m3 conversions, the
// block-scale rules, wave-level reductions and the LDS-DMA load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite on this path).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Four fp32 values -> four OCP e4m3fn codes packed little-endian (a in the low
// byte).  The hardware conversion rounds to nearest even; clamping to +-448
// first (one v_med3 per value) makes every out-of-range magnitude saturate to
// 448 (the rule's "round, then saturate" gives the same code for every input
// above 448).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// SwiGLU of one (gate, up) pair, silu(g) * u with silu(g) = g / (1 + e^-g);
// with the "swiglu_limit" clamp (LIMIT) the gate is first capped above at L and
// up clamped to [-L, L] (one v_med3 each).  The division is the hardware
// reciprocal (about 1 ulp; h is compared by tolerance, not bit for bit).  Very
// negative g gives e^-g = inf and h = -0 * u.  The limit is a compile-time
// choice so the unclamped form carries no selects.
template <bool LIMIT>
__device__ __forceinline__ float swiglu(float g, float u, float limit) {
  if constexpr (LIMIT) {
    g = __builtin_amdgcn_fmed3f(g, -__builtin_inff(), limit);
    u = __builtin_amdgcn_fmed3f(u, -limit, limit);
  }
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Block scale of the FP8_B128 format: max(amax, 1e-4) / 448 with IEEE fp32 division.
__device__ __forceinline__ float fp8_block_scale(float amax) { return __builtin_fmaxf(amax, 1e-4f) / 448.0f; }

// x / s as the FP8_B128 rule writes it (an IEEE fp32 quotient), from r = 1 / s
// (one IEEE reciprocal per block): the product q0 = x r, its exact residual
// x - s q0 (one fma) and one correction step (Markstein's division by
// reciprocal), which is the correctly rounded quotient wherever nothing
// underflows; the copysign keeps -0.  Where |x / s| is below 2^-10 the result
// may differ from the quotient, but both encode to the same signed e4m3 zero.
// Checked on the host against the IEEE quotient: exhaustively for bf16 x and
// every scale the rule gives, and on seeded fp32 x (the SwiGLU output h).
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = __fmul_rn(x, r);
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-s, q0, x), r, q0), x);
}

// MX format: e = ceil(log2(max(amax, 1e-4) / 448)) read from the fp32 bits of
// the (always normal) ratio: the exponent, plus one when a mantissa bit is set.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const uint32_t u = __float_as_uint(__builtin_fmaxf(amax, 1e-4f) / 448.0f);
  return (int)((u >> 23) & 0xFF) - 127 + ((u & 0x7FFFFF) != 0 ? 1 : 0);
}

// Max over the lanes l, l ^ m for the given xor masks (width-64 butterflies).
__device__ __forceinline__ float wave_max_xor(float v, int mask) { return __builtin_fmaxf(v, __shfl_xor(v, mask, kWave)); }

// LDS byte address of a __shared__ object (the low 32 bits of its generic
// address are its offset in the workgroup's LDS).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Direct global -> LDS copy (LDS-DMA): lane i of the wave writes bytes
// [i*16, i*16 + 16) (dma16) or [i*4, i*4 + 4) (dma4) after the wave-uniform LDS
// byte address `lds`, read from its own global address `g`.
// Written as inline asm on purpose: the compiler then does not know these
// loads write LDS, so it adds no conservative vmcnt(0) before unrelated LDS
// reads; the kernels order them with explicit wait_vmcnt + barrier instead.
// M0 carries the LDS base; it is saved and restored around the load, and the
// s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}
// The same 16-byte DMA with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the saddr form): no per-lane 64-bit address math.
__device__ __forceinline__ void lds_dma16_s(const void* sbase_any, uint32_t voff, uint32_t lds) {
  // the base is wave-uniform; under register pressure the compiler may compute
  // it in VGPRs, so move it to SGPRs explicitly (a no-op when it already is)
  const uint64_t a = (uint64_t)(uintptr_t)sbase_any;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const void* sbase = (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace moe
