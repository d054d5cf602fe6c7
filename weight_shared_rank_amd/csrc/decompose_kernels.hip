// Kernels of the GPU decomposition (one band of one family): band mean, the
// per-row least-squares scale, the residual, and an fp32 GEMM with arbitrary
// strides used by the randomized truncated SVD of the residual.  The steps
// are the analytic decomposition of the "Add a new model architecture" page
// ("Decompose HF weights") with these readings: band mean, per-row scale
// s_i = <W_i, W0_i> / <W0_i, W0_i>, rank-r truncated SVD of W - diag(s) W0
// split as U = P sqrt(S), V = Q sqrt(S).  ALS sweeps ("Quality (Gemma 4 31B)"
// page, "ALS optimization barely helps"; read as block-coordinate least
// squares from that start) add the shared-block refit and a scale against
// W0 with the layer's delta U V^T removed.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace wl {

namespace {

// fp64 -> fp32 (nearest even) -> bf16 (nearest even): the stored rounding of
// a value computed in fp64.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) { return f32_to_bf16(static_cast<float>(v)); }

// W0 = bf16(sum_l W_l / m), the sum taken in fp64 in layer order.
__global__ void band_mean_kernel(const uint16_t *W, int m, size_t nk, uint16_t *W0) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nk) return;
  double acc = 0.0;
  for (int l = 0; l < m; ++l) acc += static_cast<double>(bf16_to_f32(W[static_cast<size_t>(l) * nk + i]));
  W0[i] = f64_to_bf16(acc / m);
}

// s_i = <W_i - D_i, W0_i> / <W0_i, W0_i> in fp64 (1 for a zero W0 row),
// stored fp32, with D = U V^T of the layer's current delta (fp32 [N][K]; null
// for none, the one-shot decomposition); then R_i = W_i - s_i W0_i in fp32.
// One workgroup per row.  R may be D: a row's D is read in full before the
// barrier and R written after it.
__global__ void scale_residual_kernel(const uint16_t *W, const uint16_t *W0, int K, const float *D, float *s,
                                      float *R) {
  const int row = blockIdx.x;
  const uint16_t *w = W + static_cast<size_t>(row) * K;
  const uint16_t *w0 = W0 + static_cast<size_t>(row) * K;
  const float *d = D ? D + static_cast<size_t>(row) * K : nullptr;
  double num = 0.0, den = 0.0;
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    const double a = bf16_to_f32(w[j]) - (d ? static_cast<double>(d[j]) : 0.0), b = bf16_to_f32(w0[j]);
    num += a * b;
    den += b * b;
  }
  __shared__ double rn[256], rd[256];
  rn[threadIdx.x] = num;
  rd[threadIdx.x] = den;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (static_cast<int>(threadIdx.x) < st) {
      rn[threadIdx.x] += rn[threadIdx.x + st];
      rd[threadIdx.x] += rd[threadIdx.x + st];
    }
    __syncthreads();
  }
  const float sv = rd[0] == 0.0 ? 1.f : static_cast<float>(rn[0] / rd[0]);
  if (threadIdx.x == 0) s[row] = sv;
  float *r = R + static_cast<size_t>(row) * K;
  for (int j = threadIdx.x; j < K; j += blockDim.x) r[j] = bf16_to_f32(w[j]) - sv * bf16_to_f32(w0[j]);
}

// C[M][N] = sum_k A(m, k) B(k, n), A(m, k) = A[m * sam + k * sak], B(k, n) =
// B[k * sbk + n * sbn]; fp32 on the matrix cores (v_mfma_f32_16x16x4_f32),
// 64 x 64 tiles, 32 k per LDS tile, four waves each owning a 32 x 32 corner
// (2 x 2 MFMA blocks).  The next tile's elements are loaded into registers
// while the current one is multiplied, so a workgroup pays the load latency
// once per tile pair rather than once per tile; products are summed in k
// order, four k per MFMA.  blockIdx.z takes the k range [z kc, (z+1) kc);
// with gridDim.z > 1 each slice writes its own partial C_z at C + z M ldc and
// reduce_kernel adds them in slice order (deterministic).  Tile loads walk the
// operand's unit-stride index fastest (a_m_fast: sam == 1).
constexpr int kF32Kt = 32;
__global__ void gemm_f32_kernel(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn,
                                float *C, int64_t ldc, int M, int N, int K, int kc, int a_m_fast, int b_n_fast) {
  constexpr int EPT = kF32Kt * 64 / 256;  // elements of each operand per thread and tile
  __shared__ float As[kF32Kt][65], Bs[kF32Kt][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int mw = (wave >> 1) * 32, nw = (wave & 1) * 32;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * kc, kend = min(K, kbeg + kc);
  C += static_cast<int64_t>(blockIdx.z) * M * ldc;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ra[EPT], rb[EPT];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = threadIdx.x + q * 256;
      const int kk = a_m_fast ? (e >> 6) : (e & (kF32Kt - 1)), mm = a_m_fast ? (e & 63) : (e / kF32Kt);
      const int gm = m0 + mm, gk = k0 + kk;
      ra[q] = (gm < M && gk < kend) ? A[gm * sam + gk * sak] : 0.f;
      const int kb = b_n_fast ? (e >> 6) : (e & (kF32Kt - 1)), nn = b_n_fast ? (e & 63) : (e / kF32Kt);
      const int gn = n0 + nn, gk2 = k0 + kb;
      rb[q] = (gn < N && gk2 < kend) ? B[gk2 * sbk + gn * sbn] : 0.f;
    }
  };
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kF32Kt) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = threadIdx.x + q * 256;
      const int kk = a_m_fast ? (e >> 6) : (e & (kF32Kt - 1)), mm = a_m_fast ? (e & 63) : (e / kF32Kt);
      As[kk][mm] = ra[q];
      const int kb = b_n_fast ? (e >> 6) : (e & (kF32Kt - 1)), nn = b_n_fast ? (e & 63) : (e / kF32Kt);
      Bs[kb][nn] = rb[q];
    }
    __syncthreads();
    if (k0 + kF32Kt < kend) load(k0 + kF32Kt);  // in flight during the products below
#pragma unroll
    for (int k4 = 0; k4 < kF32Kt; k4 += 4) {
      // A block rows i: lane holds A(mw + 16 i + r16, k4 + g); B columns j: B(k4 + g, nw + 16 j + r16)
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[k4 + g][mw + 16 * i + r16];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[k4 + g][nw + 16 * j + r16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds C(mw + 16 i + 4 g + e, nw + 16 j + r16)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gm = m0 + mw + 16 * i + 4 * g + e;
      if (gm >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gn = n0 + nw + 16 * j + r16;
        if (gn < N) C[gm * ldc + gn] = acc[i][j][e];
      }
    }
}

// C[m][n] = sum over z = 0 .. splits-1, in order, of P[z][m][n] (P dense
// [splits][M][N]).
__global__ void reduce_kernel(const float *P, int splits, int M, int N, float *C, int64_t ldc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t mn = static_cast<int64_t>(M) * N;
  if (i >= mn) return;
  // eight slices' loads in flight at a time (slices past the last re-read it
  // and are dropped); summed in slice order
  float acc = 0.f;
  for (int z0 = 0; z0 < splits; z0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = P[min(z0 + j, splits - 1) * mn + i];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (z0 + j < splits) acc += v[j];
  }
  C[(i / N) * ldc + i % N] = acc;
}

// ALS shared-block step, one layer: num_ij (+)= s_i (W_ij - D_ij), den_i (+)=
// s_i^2 (fp32; layers are added in layer order, first == 1 starts the sums).
// D null: no delta (rank 0).
__global__ void w0_accumulate_kernel(const uint16_t *W, const float *D, const float *s, int N, int K, float *num,
                                     float *den, int first) {
  const size_t nk = static_cast<size_t>(N) * K;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nk) return;
  const int row = static_cast<int>(i / K);
  const float sv = s[row];
  const float v = sv * (bf16_to_f32(W[i]) - (D ? D[i] : 0.f));
  num[i] = first ? v : num[i] + v;
  if (i % K == 0) den[row] = first ? sv * sv : den[row] + sv * sv;
}

// W0_ij = bf16(num_ij / den_i); a row whose scales were all zero keeps W0.
__global__ void w0_finish_kernel(const float *num, const float *den, int K, size_t nk, uint16_t *W0) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nk) return;
  const float d = den[i / K];
  if (d != 0.f) W0[i] = f32_to_bf16(num[i] / d);
}

// bf16 -> fp32, n elements.
__global__ void to_f32_kernel(const uint16_t *src, size_t n, float *dst) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf16_to_f32(src[i]);
}

// fp32 -> bf16 (nearest even), n elements.
__global__ void to_bf16_kernel(const float *src, size_t n, uint16_t *dst) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = f32_to_bf16(src[i]);
}

unsigned blocks_for(size_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

hipError_t launch_band_mean(const uint16_t *W, int m, size_t nk, uint16_t *W0, hipStream_t stream) {
  hipLaunchKernelGGL(band_mean_kernel, dim3(blocks_for(nk)), dim3(256), 0, stream, W, m, nk, W0);
  return hipGetLastError();
}

hipError_t launch_scale_residual(const uint16_t *W, const uint16_t *W0, int N, int K, const float *D, float *s,
                                 float *R, hipStream_t stream) {
  hipLaunchKernelGGL(scale_residual_kernel, dim3(N), dim3(256), 0, stream, W, W0, K, D, s, R);
  return hipGetLastError();
}

hipError_t launch_w0_accumulate(const uint16_t *W, const float *D, const float *s, int N, int K, float *num,
                                float *den, bool first, hipStream_t stream) {
  const size_t nk = static_cast<size_t>(N) * K;
  hipLaunchKernelGGL(w0_accumulate_kernel, dim3(blocks_for(nk)), dim3(256), 0, stream, W, D, s, N, K, num, den,
                     first ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_w0_finish(const float *num, const float *den, int N, int K, uint16_t *W0, hipStream_t stream) {
  const size_t nk = static_cast<size_t>(N) * K;
  hipLaunchKernelGGL(w0_finish_kernel, dim3(blocks_for(nk)), dim3(256), 0, stream, num, den, K, nk, W0);
  return hipGetLastError();
}

hipError_t launch_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(to_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, src, n, dst);
  return hipGetLastError();
}

int gemm_f32_splits(int M, int N, int K, size_t part_elems) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int want = (512 + tiles - 1) / tiles;
  int splits = std::min(want, std::max(1, (K + 63) / 64));
  const size_t mn = static_cast<size_t>(M) * N;
  if (mn == 0 || splits < 2 || part_elems < 2 * mn) return 1;
  splits = static_cast<int>(std::min<size_t>(splits, part_elems / mn));
  return std::max(splits, 1);
}

namespace {
int split_chunk(int K, int &splits) {
  int kc = std::max(K, 1);
  if (splits > 1) {
    kc = ((K + splits - 1) / splits + kF32Kt - 1) / kF32Kt * kF32Kt;  // whole k tiles per slice
    splits = (K + kc - 1) / kc;
  }
  return kc;
}
}  // namespace

hipError_t launch_gemm_f32(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn, float *C,
                           int64_t ldc, int M, int N, int K, float *part, size_t part_elems, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  int splits = part ? gemm_f32_splits(M, N, K, part_elems) : 1;
  const int kc = split_chunk(K, splits);
  const dim3 grid((N + 63) / 64, (M + 63) / 64, splits);
  if (splits == 1) {
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, stream, A, sam, sak, B, sbk, sbn, C, ldc, M, N, K, kc,
                       sam == 1 ? 1 : 0, sbn == 1 ? 1 : 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, stream, A, sam, sak, B, sbk, sbn, part,
                     static_cast<int64_t>(N), M, N, K, kc, sam == 1 ? 1 : 0, sbn == 1 ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t mn = static_cast<size_t>(M) * N;
  hipLaunchKernelGGL(reduce_kernel, dim3(blocks_for(mn)), dim3(256), 0, stream, part, splits, M, N, C, ldc);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float *src, size_t n, uint16_t *dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, src, n, dst);
  return hipGetLastError();
}

}  // namespace wl
