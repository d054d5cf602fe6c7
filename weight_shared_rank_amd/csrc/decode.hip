// Decode-path kernels (T <= 16 tokens): y = s (.) (W0 x) + U (V^T x).
//
// The method's forward for a theta bundle ("Add a new model architecture"
// page, introduction) at decode batch sizes is a bandwidth-bound GEMV: every
// byte of W0 is read once and used for T multiply-adds.  The pages' B200
// custom op ("Quality (Gemma 4 31B)" page, "Custom-op path") put one warp per
// output row and recomputed V^T x per block; here V^T x is computed once per
// call, by a short wide launch, and the main launch streams W0.
//
//   launch 1 (z_partial_kernel): z = V^T x split over (16-rank tiles) x
//     (S slices of K); each workgroup writes one fp32 partial tile
//     zpart[slice][token][rank].  Few bytes (r/N of W0), many workgroups, so
//     it finishes in about one memory round trip.
//   launch 2 (decode_kernel): one workgroup per 16-row tile of W0, W waves
//     splitting K.  The K loop feeds bf16 MFMAs with W0 rows as the A operand
//     and up to 16 tokens of x as the B operand (token columns >= T are
//     zero), so T = 1 and T = 16 run the same code; each lane streams 16-byte
//     loads of W0 straight to registers, four lanes covering 64 contiguous
//     bytes of a row per instruction.  After the K loop each wave adds its
//     share of the rank steps of U z: it sums the S partials of z in slice
//     order, splits the sum into a bf16 hi part and a bf16 lo remainder
//     (z keeps ~16 significant bits) and runs two MFMAs per 32 ranks with U
//     rows as the A operand.  The waves' partial products are reduced through
//     LDS in a fixed order, scaled by s, and y is written once in bf16.
//
// There are no atomics and no waits between workgroups: on this multi-XCD
// device a device-scope atomic (or flag poll) issued by every workgroup of a
// launch serializes on its address and costs far more than a second launch.
// Results are deterministic run to run.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

// One batch of UNROLL complete k-steps (32 k each): loads first, then MFMAs.
template <int UNROLL>
__device__ __forceinline__ void kblock(f32x4 &acc, const uint16_t *arow, const uint16_t *xrow, bool tok_ok,
                                       int s0) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 a[UNROLL], b[UNROLL];
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) a[j] = ld16(arow + (s0 + j) * 32);
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) {
    // unconditional load (row clamped to a valid one), then select: keeps
    // the load sequence branch-free so wait counts stay exact
    const u32x4 v = ld16(xrow + (s0 + j) * 32);
    b[j] = tok_ok ? v : zero4;
  }
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) acc = mfma16x16x32(a[j], b[j], acc);
}

// acc += A[rows of arow] x[tokens]^T over the k-steps [s_begin, s_end) that
// belong to this wave: blocks of UNROLL steps round-robin over W waves, then
// single leftover steps (the last may be partial: K % 32 != 0).
template <int W, int UNROLL>
__device__ __forceinline__ void kloop(f32x4 &acc, const uint16_t *arow, const uint16_t *xrow, bool tok_ok,
                                      int s_begin, int s_end, int K, int wave, int g) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int nfull_end = min(s_end, K >> 5);  // steps fully inside K
  const int nblocks = (nfull_end - s_begin) / UNROLL;
  for (int b = wave; b < nblocks; b += W) kblock<UNROLL>(acc, arow, xrow, tok_ok, s_begin + b * UNROLL);
  for (int s = s_begin + nblocks * UNROLL + wave; s < s_end; s += W) {
    const bool kin = s * 32 + g * 8 < K;
    const u32x4 a = kin ? ld16(arow + s * 32) : zero4;
    const u32x4 v = kin ? ld16(xrow + s * 32) : zero4;
    acc = mfma16x16x32(a, tok_ok ? v : zero4, acc);
  }
}

template <int W>
__device__ __forceinline__ f32x4 reduce_waves(f32x4 (*red)[64], f32x4 v, int wave, int lane) {
  red[wave][lane] = v;
  __syncthreads();
  f32x4 t = red[0][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) t += red[w][lane];
  return t;
}

// grid (ceil(Rz / 16), S): tile of 16 V^T rows x one K slice.
template <int W, int UNROLL>
__global__ __launch_bounds__(W * 64) void z_partial_kernel(CallDesc c, float *zpart, int ldz) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int S = gridDim.y, slice = blockIdx.y;
  const int K = c.K;
  const int nsteps = (K + 31) >> 5;
  const int per = (nsteps + S - 1) / S;
  const int s_begin = min(nsteps, slice * per), s_end = min(nsteps, s_begin + per);
  const int arow_idx = (row0 + r16 < c.Rz) ? row0 + r16 : row0;
  const uint16_t *arow = c.Vt + static_cast<size_t>(arow_idx) * K + g * 8;
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  kloop<W, UNROLL>(acc, arow, xrow, tok_ok, s_begin, s_end, K, wave, g);
  __shared__ f32x4 red[W][64];
  const f32x4 tot = reduce_waves<W>(red, acc, wave, lane);
  if (wave != 0 || !tok_ok) return;
  // lane holds D[m = 4g + i][n = r16]: ranks row0 + 4g + i, token r16
  float *zp = zpart + (static_cast<size_t>(slice) * kDecodeMaxT + r16) * ldz;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = row0 + g * 4 + i;
    if (k < c.Rz) zp[k] = tot[i];
  }
}

// z fragment for the MFMA B operand: ranks kbase + 8g .. +7 of token r16,
// summed over the S slices in order, as a bf16 hi/lo pair.
__device__ __forceinline__ void z_fragment(const float *zpart, int ldz, int S, int r16, int k, bool valid,
                                           u32x4 &hi, u32x4 &lo) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
  if (valid) {
    const float *p = zpart + static_cast<size_t>(r16) * ldz + k;
    for (int s = 0; s < S; ++s) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
      v[0] += a[0]; v[1] += a[1]; v[2] += a[2]; v[3] += a[3];
      v[4] += b[0]; v[5] += b[1]; v[6] += b[2]; v[7] += b[3];
      p += static_cast<size_t>(kDecodeMaxT) * ldz;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = f32_to_bf16(v[2 * e]), h1 = f32_to_bf16(v[2 * e + 1]);
    const uint16_t l0 = f32_to_bf16(v[2 * e] - bf16_to_f32(h0)), l1 = f32_to_bf16(v[2 * e + 1] - bf16_to_f32(h1));
    hi[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
    lo[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
  }
}

template <int W, int UNROLL>
__global__ __launch_bounds__(W * 64) void decode_kernel(CallDesc c, const float *zpart, int ldz, int S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int K = c.K;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Rows past the end read the tile's first row (always valid); their
  // results are never stored.  Token columns >= T are zero.
  const int arow_idx = (row0 + r16 < c.Ntot) ? row0 + r16 : row0;
  const uint16_t *arow = c.W0 + static_cast<size_t>(arow_idx) * K + g * 8;
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  kloop<W, UNROLL>(acc, arow, xrow, tok_ok, 0, (K + 31) >> 5, K, wave, g);

  // delta = U z: this wave's share of the rank steps of every child with
  // rows in this tile (A = U rows of that child, other rows zero).
  f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
  const int arow_g = row0 + r16;
  for (int ci = 0; ci < c.nchild; ++ci) {
    const ChildDesc &ch = c.ch[ci];
    if (ch.rpad == 0 || row0 >= ch.row_start + ch.N || row0 + 16 <= ch.row_start) continue;
    const bool in_child = arow_g >= ch.row_start && arow_g < ch.row_start + ch.N;
    const uint16_t *urow = ch.U + static_cast<size_t>(in_child ? arow_g - ch.row_start : 0) * ch.rpad + g * 8;
    for (int kk = wave * 32; kk < ch.rpad; kk += W * 32) {
      const bool kin = kk + g * 8 < ch.rpad;
      const u32x4 a = (kin && in_child) ? ld16(urow + kk) : zero4;
      u32x4 hi, lo;
      z_fragment(zpart, ldz, S, r16, ch.zoff + kk + g * 8, kin && tok_ok, hi, lo);
      dacc = mfma16x16x32(a, hi, dacc);
      dacc = mfma16x16x32(a, lo, dacc);
    }
  }

  // Cross-wave reduction (K split and rank split), fixed order.
  __shared__ f32x4 red[W][64];
  __shared__ f32x4 dred[W][64];
  red[wave][lane] = acc;
  dred[wave][lane] = dacc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  f32x4 tot = red[0][lane];
  f32x4 dtot = dred[0][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) {
    tot += red[w][lane];
    dtot += dred[w][lane];
  }
  // lane holds D[m = 4g + i][n = r16]: rows row0 + 4g + i, token r16
  uint16_t *yrow = c.y + static_cast<size_t>(r16) * c.ldy;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + g * 4 + i;
    if (row >= c.Ntot) continue;
    int ci = 0;
    while (ci + 1 < c.nchild && row >= c.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = c.ch[ci];
    const uint16_t out = f32_to_bf16(c.s[row] * tot[i] + dtot[i]);
    const int j = row - ch.row_start;
    yrow[ch.y_off + j] = out;
    if (ch.dup_off >= 0) yrow[ch.dup_off + j] = out;
  }
}

}  // namespace

int decode_z_slices(int Rz, int K) {
  // enough (rank tile, K slice) workgroups to cover the device in one round,
  // without slices shorter than 8 k-steps
  const int tiles = (Rz + 15) / 16;
  if (tiles == 0) return 0;
  int S = 256 / tiles;
  const int nsteps = (K + 31) / 32;
  S = min(S, max(1, nsteps / 8));
  return max(1, min(S, kDecodeMaxSlices));
}

hipError_t launch_decode(const CallDesc &c, float *zpart, hipStream_t stream) {
  constexpr int W = 8, UNROLL = 4;
  const int ldz = c.Rz;
  const int S = decode_z_slices(c.Rz, c.K);
  if (c.Rz > 0) {
    hipLaunchKernelGGL((z_partial_kernel<W, UNROLL>), dim3((c.Rz + 15) / 16, S), dim3(W * 64), 0, stream, c, zpart, ldz);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<W, UNROLL>), dim3((c.Ntot + 15) / 16), dim3(W * 64), 0, stream, c,
                     static_cast<const float *>(zpart), ldz, S);
  return hipGetLastError();
}

}  // namespace wl
