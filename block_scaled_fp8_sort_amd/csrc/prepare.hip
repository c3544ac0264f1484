// One-shot weight preparation kernels: batched transposes that turn the nn
// weight layout ([E, K, N] per weight) into the nt layout the GEMMs read
// ([E, N, K]).  The pages' forward transforms both weight pairs once, before the
// first forward, and picks the nn or nt grouped matmul by a layout flag ("DeepGEMM
// Mega MoE requires a `process_group` for the EP group", docstring; "DeepGEMM
// experts selected on a model spanning multiple CUDA devices", the record's
// source).  Not on the timed path: a plain 64x64 LDS-tiled transpose.
#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int32_t rows,
                                                        int32_t cols) {
  __shared__ T tile[64][65];
  const int64_t b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* src = in + b * (int64_t)rows * cols;
  T* dst = out + b * (int64_t)rows * cols;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    if (r0 + rr < rows && c0 + cc < cols) tile[rr][cc] = src[(int64_t)(r0 + rr) * cols + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (r0 + rr < rows && c0 + cc < cols) dst[(int64_t)(c0 + cc) * rows + r0 + rr] = tile[rr][cc];
  }
}

template <typename T>
hipError_t launch_t(const T* in, T* out, int32_t batch, int32_t rows, int32_t cols, hipStream_t stream) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, stream, in, out, rows, cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose_u8(const uint8_t* in, uint8_t* out, int32_t batch, int32_t rows, int32_t cols,
                               hipStream_t stream) {
  return launch_t<uint8_t>(in, out, batch, rows, cols, stream);
}
hipError_t launch_transpose_f32(const float* in, float* out, int32_t batch, int32_t rows, int32_t cols,
                                hipStream_t stream) {
  return launch_t<float>(in, out, batch, rows, cols, stream);
}

}  // namespace moe
