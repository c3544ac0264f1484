// Matrix-core issue-rate probe and clock stamps for gfx950 (measurement
// utilities, not steps of the forward).
//
// The grouped GEMMs are priced against the MFMA rate of their own operand
// types.  The published peaks give FP8 and FP4 rates for matching operands,
// but the MX experts multiply e2m1 weights by e4m3 activations, and the FP8
// experts add an fp32 promotion per 128-wide K block; this kernel measures
// the rate each form the GEMMs use actually issues at, with random operands
// held in registers (no memory traffic), eight waves on every CU, and reads
// the shader clock it ran at.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeWaves = 8;

// 32-bit mixing function (the xorshift-multiply finalizer of a counter hash):
// operand bits that toggle like real data
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// KIND: 0 e4m3 x e4m3 accumulating in the MFMA, 1 e2m1 x e4m3 and 2 e2m1 x e2m1
// with per-lane UE8M0 scales (the MX GEMM's form), 3 bf16 16x16x32, 4 e4m3 x
// e4m3 with a fresh accumulator and the fp32 promotion acc += P * s (the FP8
// GEMM's form, pipelined as the GEMM does it).  Every wave runs iters (even)
// rounds of probe_mfmas_per_round(KIND) independent MFMAs, the operands
// rotating each round.
template <int KIND>
__global__ __launch_bounds__(kProbeWaves * 64, 1) void mfma_rate_kernel(int iters, float* sink,
                                                                         unsigned long long* clk) {
  const int tid = threadIdx.x;
  const uint32_t seed = (uint32_t)(blockIdx.x * blockDim.x + tid) * 128u;
  // e4m3 bytes with the exponent's top bit cleared (no NaN code), bf16 values
  // likewise finite; e2m1 has no special codes
  const uint32_t mask = KIND == 3 ? 0xBFFFBFFFu : (KIND == 0 || KIND == 4) ? 0xBFBFBFBFu : 0xFFFFFFFFu;
  const uint32_t mask_b = KIND == 1 ? 0xBFBFBFBFu : mask;
  // four operand sets rotated through, as a K step's four token sub-tiles and
  // changing weight fragments are; the promotion form runs 4 x 2 outputs per
  // round (its partials take the registers of the other eight)
  constexpr int NOPS = 4;
  constexpr int TN = KIND == 4 ? 2 : 4;
  v8i A[NOPS], B[NOPS];
#pragma unroll
  for (int j = 0; j < NOPS; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      A[j][i] = (int)(mix32(seed + j * 16 + i) & mask);
      B[j][i] = (int)(mix32(seed + 64 + j * 16 + i) & mask_b);
    }
  int sc;  // UE8M0 1.0 in a VGPR, as the MX GEMM passes its per-lane scales
  asm volatile("v_mov_b32 %0, 127" : "=v"(sc));
  const float s = 1e-3f * (float)(tid + 1);
  v4f acc[4][TN], pa[4][TN], pb[4][TN];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[n][t] = pa[n][t] = pb[n][t] = v4f{0.f, 0.f, 0.f, 0.f};
  // one round: an MFMA per output; the promotion form writes this round's
  // partials into `wr` while folding the previous round's, in `rd`, into the
  // accumulators (the FP8 GEMM's pipeline: no FMA waits on the MFMA before it)
  auto round = [&](int o, v4f(&wr)[4][TN], v4f(&rd)[4][TN]) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const v8i a = A[(n + o) % NOPS], b = B[(t + o) % NOPS];
        if constexpr (KIND == 0) {
          acc[n][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[n][t], 0, 0, 0, 0, 0, 0);
        } else if constexpr (KIND == 1) {
          acc[n][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0}, b,
                                                                       acc[n][t], 4, 0, 0, sc, 0, sc);
        } else if constexpr (KIND == 2) {
          acc[n][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0}, v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0}, acc[n][t], 4, 4, 0, sc,
              0, sc);
        } else if constexpr (KIND == 3) {
          acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v4i{a[0], a[1], a[2], a[3]}),
                                                              __builtin_bit_cast(bf16x8, v4i{b[0], b[1], b[2], b[3]}),
                                                              acc[n][t], 0, 0, 0);
        } else {
          wr[n][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          acc[n][t] += rd[n][t] * s;
        }
      }
  };
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {  // iters is even
    round(it & 3, pa, pb);
    round((it + 1) & 3, pb, pa);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const v4f v = acc[n][t] + pa[n][t] + pb[n][t];
      sum += v[0] + v[1] + v[2] + v[3];
    }
  sink[blockIdx.x * blockDim.x + tid] = sum;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// One stamp per workgroup: the compute unit it runs on (XCD id x 256 + the
// shader engine, array and CU ids of the hardware-id register, bits 8-15), that
// unit's shader-clock counter and the 100 MHz real-time counter.  Two stamps on
// one stream bracket the work enqueued between them; the shader-clock counters
// of different units are not aligned, so spans are measured per unit.
__global__ __launch_bounds__(64) void clock_stamp_kernel(unsigned long long* out) {
  if (threadIdx.x != 0) return;
  unsigned xcc, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID, 8, 8)" : "=s"(hw));
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  out[3 * blockIdx.x] = (unsigned long long)(xcc * 256u + hw);
  out[3 * blockIdx.x + 1] = t;
  out[3 * blockIdx.x + 2] = r;
}

}  // namespace

hipError_t launch_clock_stamp(unsigned long long* out, int n, hipStream_t stream) {
  hipLaunchKernelGGL(clock_stamp_kernel, dim3((unsigned)n), dim3(64), 0, stream, out);
  return hipGetLastError();
}

int probe_threads() { return kProbeWaves * 64; }

int64_t probe_flops_per_mfma(int kind) { return kind == 3 ? 16 * 16 * 32 * 2 : 16 * 16 * 128 * 2; }

int probe_mfmas_per_round(int kind) { return kind == 4 ? 8 : 16; }

hipError_t launch_mfma_probe(int kind, int iters, int grid, float* sink, unsigned long long* clk,
                             hipStream_t stream) {
  const dim3 g((unsigned)grid), b(kProbeWaves * 64);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, g, b, 0, stream, iters, sink, clk); break;
    case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, g, b, 0, stream, iters, sink, clk); break;
    case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, g, b, 0, stream, iters, sink, clk); break;
    case 3: hipLaunchKernelGGL(mfma_rate_kernel<3>, g, b, 0, stream, iters, sink, clk); break;
    default: hipLaunchKernelGGL(mfma_rate_kernel<4>, g, b, 0, stream, iters, sink, clk); break;
  }
  return hipGetLastError();
}

}  // namespace moe
