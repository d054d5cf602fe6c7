// Decode-path kernels (T <= 16 tokens): y = s (.) (W0 x) + U (V^T x).
//
// The method's forward for a theta bundle ("Add a new model architecture"
// page, introduction) at decode batch sizes is bandwidth-bound: every byte
// of W0 is read once and used for T multiply-adds.  The pages' GEMM path
// ("Quality (Gemma 4 31B)" page, "Kernel optimizations > GEMM path") runs
// two dispatches per stacked call -- one product over W0 and V stacked, one
// block-diagonal U product -- and that is the split kept here, with both
// launches written for gfx950:
//
//   launch 1 (stream_kernel): the rows [W0; V^T] of the call (all children of
//     a stacked call) times x, split over K into KS slices.  A workgroup owns
//     one 16-row tile and one K slice; its W waves take interleaved blocks of
//     UNROLL k-steps, so at any time the workgroup reads each of its 16 rows in
//     contiguous runs of W*UNROLL*64 bytes.  Each lane loads 16 bytes of a row
//     straight to registers (four lanes cover 64 contiguous bytes) and feeds a
//     bf16 MFMA with W0 rows as the A operand and up to 16 tokens of x as the
//     B operand (token columns >= T are zero, so T = 1 and T = 16 run the same
//     code).  The waves' sums are reduced through LDS in a fixed order and the
//     fp32 partial of the tile is written for tokens < T: p_part[slice][t][row]
//     for W0 rows, z_part[t][rank] for V^T rows.
//     The V^T tiles are not split (z needs no summation) and come first in
//     the grid, so they are dispatched early and end well inside the launch.
//   launch 2 (epilogue_kernel): one workgroup per 16-row tile.  Its waves
//     split the rank steps of U z: each splits z into a bf16 hi part and a
//     bf16 lo remainder (z keeps ~16 significant bits) and runs two MFMAs per
//     32 ranks with U rows as the A operand; the waves' sums are reduced
//     through LDS, the KS partials of p are summed in slice order, scaled by
//     s, and y is written once in bf16.  It reads U (r/K of W0's bytes) and
//     the partials.
//
// There are no atomics and no waits between workgroups: on this multi-XCD
// device a device-scope atomic or flag poll issued by every workgroup of a
// launch serializes on its address and costs more than a second launch.
// Results are deterministic run to run.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

constexpr int kStreamWaves = 8;
constexpr int kStreamUnroll = 4;
constexpr int kEpiWaves = 4;

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
    // unconditional load (row clamped to a valid one), then select: keeps the
    // load sequence branch-free so the wait counts stay exact
    const u32x4 v = ld16(xrow + (s0 + j) * 32);
    b[j] = tok_ok ? v : zero4;
  }
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) acc = mfma16x16x32(a[j], b[j], acc);
}

// 1-D grid: first the V^T tiles (full K, so z needs no summation later; they
// are dispatched first and finish well inside the launch), then the W0 tiles,
// each split into KS slices of K.
template <int W, int UNROLL>
__global__ __launch_bounds__(W * 64) void stream_kernel(CallDesc c, float *p_part, float *z_part, int ntile_vt,
                                                        int KS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const bool vt = static_cast<int>(blockIdx.x) < ntile_vt;
  const int widx = blockIdx.x - ntile_vt;
  const int row0 = (vt ? blockIdx.x : widx / KS) * 16;
  const int slice = vt ? 0 : widx % KS;
  const int nslices = vt ? 1 : KS;
  const uint16_t *mat = vt ? c.Vt : c.W0;
  const int nrows = vt ? c.Rz : c.Ntot;
  const int K = c.K;
  const int nsteps = (K + 31) >> 5;
  const int per = (nsteps + nslices - 1) / nslices;
  const int s_begin = min(nsteps, slice * per), s_end = min(nsteps, s_begin + per);

  // Rows past the end read the tile's first row (always valid); their
  // results are never stored.  Token columns >= T are zero.
  const int arow_idx = (row0 + r16 < nrows) ? row0 + r16 : row0;
  const uint16_t *arow = mat + static_cast<size_t>(arow_idx) * K + g * 8;
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nfull_end = min(s_end, K >> 5);  // steps entirely inside K
  const int nblocks = max(0, nfull_end - s_begin) / UNROLL;
  for (int b = wave; b < nblocks; b += W) kblock<UNROLL>(acc, arow, xrow, tok_ok, s_begin + b * UNROLL);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int s = s_begin + nblocks * UNROLL + wave; s < s_end; s += W) {
    const bool kin = s * 32 + g * 8 < K;  // the last step may be partial
    const u32x4 a = kin ? ld16(arow + s * 32) : zero4;
    const u32x4 v = kin ? ld16(xrow + s * 32) : zero4;
    acc = mfma16x16x32(a, tok_ok ? v : zero4, acc);
  }

  __shared__ f32x4 red[W][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  f32x4 tot = red[0][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) tot += red[w][lane];
  // lane holds D[m = 4g + i][n = r16]: rows row0 + 4g + i, token r16
  const int ld = vt ? c.Rz : c.Ntot;
  float *dst = (vt ? z_part : p_part) + (static_cast<size_t>(slice) * c.T + r16) * ld;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + g * 4 + i;
    if (row < nrows) dst[row] = tot[i];
  }
}

// z B-fragment: ranks k .. k+7 of token r16 as a bf16 hi/lo pair.
__device__ __forceinline__ void z_fragment(const float *z_part, int Rz, int r16, int k, bool valid, u32x4 &hi,
                                           u32x4 &lo) {
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float *p = z_part + static_cast<size_t>(r16) * Rz + k;
    a = *reinterpret_cast<const f32x4 *>(p);
    b = *reinterpret_cast<const f32x4 *>(p + 4);
  }
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = f32_to_bf16(v[2 * e]), h1 = f32_to_bf16(v[2 * e + 1]);
    const uint16_t l0 = f32_to_bf16(v[2 * e] - bf16_to_f32(h0)), l1 = f32_to_bf16(v[2 * e + 1] - bf16_to_f32(h1));
    hi[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
    lo[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
  }
}

// One workgroup per 16-row tile; its WE waves split the rank steps of U z.
template <int WE>
__global__ __launch_bounds__(WE * 64) void epilogue_kernel(CallDesc c, const float *p_part, const float *z_part,
                                                           int KS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const bool tok_ok = r16 < c.T;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int rbase = row0 + g * 4;

  // wave 0 starts the loads of the p partials (this lane: rows rbase..+3,
  // token r16) before the delta
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && tok_ok) {
    if (rbase + 3 < c.Ntot && (c.Ntot & 3) == 0) {
      const float *pp = p_part + static_cast<size_t>(r16) * c.Ntot + rbase;
      for (int s = 0; s < KS; ++s) {
        p += *reinterpret_cast<const f32x4 *>(pp);
        pp += static_cast<size_t>(c.T) * c.Ntot;
      }
    } else {
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rbase + i < c.Ntot) p[i] += p_part[(static_cast<size_t>(s) * c.T + r16) * c.Ntot + rbase + i];
    }
  }

  // delta = U z: this wave's rank steps of every child with rows in the tile
  // (A = U rows of that child, rows of other children zero)
  f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
  const int arow_g = row0 + r16;
  for (int ci = 0; ci < c.nchild; ++ci) {
    const ChildDesc &ch = c.ch[ci];
    if (ch.rpad == 0 || row0 >= ch.row_start + ch.N || row0 + 16 <= ch.row_start) continue;
    const bool in_child = arow_g >= ch.row_start && arow_g < ch.row_start + ch.N;
    const uint16_t *urow = ch.U + static_cast<size_t>(in_child ? arow_g - ch.row_start : 0) * ch.rpad + g * 8;
    for (int kk = wave * 32; kk < ch.rpad; kk += 2 * WE * 32) {
      const int k1 = kk + WE * 32;
      const bool in0 = kk + g * 8 < ch.rpad, in1 = k1 + g * 8 < ch.rpad;
      const u32x4 a0 = (in0 && in_child) ? ld16(urow + kk) : zero4;
      const u32x4 a1 = (in1 && in_child) ? ld16(urow + k1) : zero4;
      u32x4 h0, l0, h1, l1;
      z_fragment(z_part, c.Rz, r16, ch.zoff + kk + g * 8, in0 && tok_ok, h0, l0);
      z_fragment(z_part, c.Rz, r16, ch.zoff + k1 + g * 8, in1 && tok_ok, h1, l1);
      dacc = mfma16x16x32(a0, h0, dacc);
      dacc = mfma16x16x32(a0, l0, dacc);
      dacc = mfma16x16x32(a1, h1, dacc);
      dacc = mfma16x16x32(a1, l1, dacc);
    }
  }
  __shared__ f32x4 red[WE][64];
  red[wave][lane] = dacc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  f32x4 d = red[0][lane];
#pragma unroll
  for (int w = 1; w < WE; ++w) d += red[w][lane];

  // lane holds D[m = 4g + i][n = r16]: rows rbase + i, token r16
  uint16_t *yrow = c.y + static_cast<size_t>(r16) * c.ldy;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + i;
    if (row >= c.Ntot) continue;
    int ci = 0;
    while (ci + 1 < c.nchild && row >= c.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = c.ch[ci];
    const uint16_t out = f32_to_bf16(c.s[row] * p[i] + d[i]);
    const int j = row - ch.row_start;
    yrow[ch.y_off + j] = out;
    if (ch.dup_off >= 0) yrow[ch.dup_off + j] = out;
  }
}

}  // namespace

int decode_k_slices(int Ntot, int Rz, int K) {
  // Aim for about 4096 workgroups in the stream launch, with K slices of at
  // least 16 k-steps and at most kDecodeMaxSlices slices.
  const int tiles = (Ntot + 15) / 16 + (Rz + 15) / 16;
  const int nsteps = (K + 31) / 32;
  int ks = (4096 + tiles - 1) / max(1, tiles);
  ks = min(ks, max(1, nsteps / 16));
  return max(1, min(ks, kDecodeMaxSlices));
}

hipError_t launch_decode(const CallDesc &c, float *p_part, float *z_part, hipStream_t stream) {
  const int KS = decode_k_slices(c.Ntot, c.Rz, c.K);
  const int nt_w0 = (c.Ntot + 15) / 16, nt_vt = (c.Rz + 15) / 16;
  hipLaunchKernelGGL((stream_kernel<kStreamWaves, kStreamUnroll>), dim3(nt_vt + nt_w0 * KS), dim3(kStreamWaves * 64),
                     0, stream, c, p_part, z_part, nt_vt, KS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((epilogue_kernel<kEpiWaves>), dim3(nt_w0), dim3(kEpiWaves * 64), 0, stream, c,
                     static_cast<const float *>(p_part), static_cast<const float *>(z_part), KS);
  return hipGetLastError();
}

}  // namespace wl
