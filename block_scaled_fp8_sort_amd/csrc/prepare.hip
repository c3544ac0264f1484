// One-shot weight preparation kernels: the tiling of the FP8 weights into the
// layout the grouped GEMMs stream (tile_layout.h), from the nt ([E, N, K]) or
// the nn ([E, K, N]) layout, and batched transposes for the nn scales.  The pages' forward transforms both weight pairs once, before the
// first forward, and picks the nn or nt grouped matmul by a layout flag ("DeepGEMM
// Mega MoE requires a `process_group` for the EP group", docstring; "DeepGEMM
// experts selected on a model spanning multiple CUDA devices", the record's
// source).  Not on the timed path.
#include "device_common.h"
#include "internal.h"
#include "tile_layout.h"

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

// One thread per 16-byte piece of the tiled destination [E][NT][KB][32 KB]:
// find the tile row tr and logical chunk c the piece holds (the MFMA operand
// order of tile_layout.h), copy the source row's 16 K-bytes there, or zeros for
// a padding row.  ESZ is the element size: 1 for FP8 codes, 2 for bf16, whose
// rows are tiled as rows of 2K bytes (a 128-byte K block is 64 elements).
template <bool PAIRED, int ESZ>
__global__ __launch_bounds__(256) void tile_weight_kernel(const uint8_t* __restrict__ src, int nn, int32_t N,
                                                          int32_t K, int32_t NT, int64_t n_chunks,
                                                          uint8_t* __restrict__ dst) {
  const int KB = K * ESZ / kBlockK;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < n_chunks; d += stride) {
    const int piece = (int)(d & 2047);  // 16-byte piece inside the 32 KB block
    int64_t rest = d >> 11;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int nt = (int)(rest % NT);
    const int64_t e = rest / NT;
    const int grp = piece >> 7, h = (piece >> 6) & 1, l = piece & 63;
    const int tr = grp * 16 + (l & 15);
    const int c = 4 * h + (l >> 4);
    const int row = tile_src_row<PAIRED>(nt, tr, N);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row >= 0) {
      const int64_t k0 = (int64_t)kb * kBlockK + c * 16;  // byte offset in the row
      if (!nn) {
        v = *(const uint4*)(src + (e * N + row) * (int64_t)K * ESZ + k0);
      } else if constexpr (ESZ == 1) {  // [E][K][N]: gather 16 bytes down a column
        uint8_t b[16];
        for (int j = 0; j < 16; ++j) b[j] = src[(e * K + k0 + j) * (int64_t)N + row];
        v = *(const uint4*)b;
      } else {  // bf16 [E][K][N]: 8 elements down a column
        const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
        uint32_t w[4];
        for (int j = 0; j < 4; ++j)
          w[j] = (uint32_t)s16[(e * K + k0 / 2 + 2 * j) * (int64_t)N + row] |
                 ((uint32_t)s16[(e * K + k0 / 2 + 2 * j + 1) * (int64_t)N + row] << 16);
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    *(uint4*)(dst + d * 16) = v;
  }
}

// MX codes: one thread per 16-byte piece of [E][NT][KB][16 KB] (the FP4 MFMA
// operand order of tile_layout.h); the source row is packed [E][N][K/2].
template <bool PAIRED>
__global__ __launch_bounds__(256) void tile_weight_mx_kernel(const uint8_t* __restrict__ src, int32_t N, int32_t K,
                                                             int32_t NT, int64_t n_chunks, uint8_t* __restrict__ dst) {
  const int KB = K / 128;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < n_chunks; d += stride) {
    const int piece = (int)(d & 1023);  // 16-byte piece inside the 16 KB block
    int64_t rest = d >> 10;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int nt = (int)(rest % NT);
    const int64_t e = rest / NT;
    const int grp = piece >> 6, l = piece & 63;
    const int tr = grp * 16 + (l & 15);
    const int c = l >> 4;
    const int row = tile_src_row<PAIRED>(nt, tr, N);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row >= 0) v = *(const uint4*)(src + (e * N + row) * (int64_t)(K / 2) + (int64_t)kb * 64 + c * 16);
    *(uint4*)(dst + d * 16) = v;
  }
}

// MX scales: one thread per 4-byte entry of [E][NT][KB][256][4]; the source is
// [E][N][K/32] bytes.
template <bool PAIRED>
__global__ __launch_bounds__(256) void tile_scale_mx_kernel(const uint8_t* __restrict__ src, int32_t N, int32_t K,
                                                            int32_t NT, int64_t n_entries, uint32_t* __restrict__ dst) {
  const int KB = K / 128;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < n_entries; d += stride) {
    int64_t rest = d;
    const int tr = (int)(rest % kTileN);
    rest /= kTileN;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int nt = (int)(rest % NT);
    const int64_t e = rest / NT;
    const int row = tile_src_row<PAIRED>(nt, tr, N);
    uint32_t v = 0x7F7F7F7Fu;  // padding rows: scale 1, codes 0
    if (row >= 0) {
      const uint8_t* s = src + (e * N + row) * (int64_t)(K / 32) + kb * 4;
      v = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
    }
    dst[d] = v;
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

namespace {

template <int ESZ>
hipError_t launch_tile_weight(const uint8_t* src, bool nn, bool paired, int32_t E, int32_t N, int32_t K, uint8_t* dst,
                              hipStream_t stream) {
  const int32_t NT = paired ? (N / 2) / 128 : (N + kTileN - 1) / kTileN;
  const int64_t n_chunks = (int64_t)E * NT * (K * ESZ / kBlockK) * kTileN * 8;
  if (n_chunks == 0) return hipSuccess;
  const int64_t want = (n_chunks + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  if (paired)
    hipLaunchKernelGGL((tile_weight_kernel<true, ESZ>), dim3(blocks), dim3(256), 0, stream, src, nn ? 1 : 0, N, K,
                       NT, n_chunks, dst);
  else
    hipLaunchKernelGGL((tile_weight_kernel<false, ESZ>), dim3(blocks), dim3(256), 0, stream, src, nn ? 1 : 0, N, K,
                       NT, n_chunks, dst);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_weight_fp8(const uint8_t* src, bool nn, bool paired, int32_t E, int32_t N, int32_t K,
                                  uint8_t* dst, hipStream_t stream) {
  return launch_tile_weight<1>(src, nn, paired, E, N, K, dst, stream);
}

hipError_t launch_tile_weight_bf16(const uint16_t* src, bool nn, bool paired, int32_t E, int32_t N, int32_t K,
                                   uint16_t* dst, hipStream_t stream) {
  return launch_tile_weight<2>(reinterpret_cast<const uint8_t*>(src), nn, paired, E, N, K,
                               reinterpret_cast<uint8_t*>(dst), stream);
}

hipError_t launch_tile_weight_mx(const uint8_t* codes, const uint8_t* scales, bool paired, int32_t E, int32_t N,
                                 int32_t K, uint8_t* dst_codes, uint8_t* dst_scales, hipStream_t stream) {
  const int32_t NT = paired ? (N / 2) / 128 : (N + kTileN - 1) / kTileN;
  const int64_t n_entries = (int64_t)E * NT * (K / 128) * kTileN;  // one per (tile row, K block)
  if (n_entries == 0) return hipSuccess;
  const int64_t n_chunks = n_entries * 4;
  int blocks = (int)((n_chunks + 255) / 256 < 65536 ? (n_chunks + 255) / 256 : 65536);
  if (paired)
    hipLaunchKernelGGL(tile_weight_mx_kernel<true>, dim3(blocks), dim3(256), 0, stream, codes, N, K, NT, n_chunks,
                       dst_codes);
  else
    hipLaunchKernelGGL(tile_weight_mx_kernel<false>, dim3(blocks), dim3(256), 0, stream, codes, N, K, NT, n_chunks,
                       dst_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  blocks = (int)((n_entries + 255) / 256 < 65536 ? (n_entries + 255) / 256 : 65536);
  if (paired)
    hipLaunchKernelGGL(tile_scale_mx_kernel<true>, dim3(blocks), dim3(256), 0, stream, scales, N, K, NT, n_entries,
                       (uint32_t*)dst_scales);
  else
    hipLaunchKernelGGL(tile_scale_mx_kernel<false>, dim3(blocks), dim3(256), 0, stream, scales, N, K, NT, n_entries,
                       (uint32_t*)dst_scales);
  return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* in, uint8_t* out, int32_t batch, int32_t rows, int32_t cols,
                               hipStream_t stream) {
  return launch_t<uint8_t>(in, out, batch, rows, cols, stream);
}
hipError_t launch_transpose_f32(const float* in, float* out, int32_t batch, int32_t rows, int32_t cols,
                                hipStream_t stream) {
  return launch_t<float>(in, out, batch, rows, cols, stream);
}

}  // namespace moe
