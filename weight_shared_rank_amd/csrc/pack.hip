// Load-time kernels used by theta_bundle_load: zero-fill of the arena (so rank
// padding reads as zero) and the V [K, r] -> V^T [r, K] transpose.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

__global__ void fill_zero_kernel(u32x4 *dst, size_t n16, uint8_t *tail, size_t ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

// 32x32 tiles through LDS: reads of V are coalesced along r, writes of V^T
// along K.
__global__ void transpose_kernel(const uint16_t *V, int K, int r, uint16_t *Vt) {
  __shared__ uint16_t tile[32][33];
  const int k0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: ty in [0, 8)
  for (int i = ty; i < 32; i += 8) {
    const int k = k0 + i, j = r0 + tx;
    tile[i][tx] = (k < K && j < r) ? V[static_cast<size_t>(k) * r + j] : 0;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int j = r0 + i, k = k0 + tx;
    if (j < r && k < K) Vt[static_cast<size_t>(j) * K + k] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_fill_zero(void *dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  // dst is 256-byte aligned by contract of the callers.
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<u32x4 *>(dst), n16, static_cast<uint8_t *>(dst) + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const uint16_t *V, int32_t K, int32_t r, uint16_t *dst, hipStream_t stream) {
  if (K == 0 || r == 0) return hipSuccess;
  const dim3 grid((K + 31) / 32, (r + 31) / 32);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, V, K, r, dst);
  return hipGetLastError();
}

}  // namespace wl
