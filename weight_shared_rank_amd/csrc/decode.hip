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
//     for W0 rows.  V^T rows hold all of z = V^T x; they store it as a bf16
//     pair, z_hi[t][rank] = bf16(z) and z_lo[t][rank] = bf16(z - z_hi), which
//     keeps ~16 significant bits and is the MFMA operand of launch 2.
//     The V^T tiles come first in the grid, so they are dispatched early.
//     They usually run the whole K (z then needs no summation).  Where a
//     whole-K tile would be the launch's last workgroup, they are split in
//     two K slices instead, and launch 2 adds the two fp32 halves of z.
//     This covers coded W0 at long K and bf16 calls with few rows.
//     With several tokens (bf16 W0) launch 1 is stream_rows_kernel instead:
//     two or four 16-row tiles per workgroup share each x fragment, chosen
//     by T and the call's slice lengths in launch_decode.
//   launch 2 (epilogue_kernel): one workgroup per 16-row tile.  Its waves
//     split the rank steps of U z: two MFMAs per 32 ranks (z_hi, then z_lo,
//     as B operands) with U rows as the A operand; the waves' sums are reduced
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

// Launch shape (overridable at build time for tuning sweeps).
#ifndef WL_STREAM_WAVES
#define WL_STREAM_WAVES 8
#endif
#ifndef WL_STREAM_UNROLL
#define WL_STREAM_UNROLL 4
#endif
#ifndef WL_EPI_WAVES
#define WL_EPI_WAVES 2
#endif
#ifndef WL_DECODE_TARGET_WGS
#define WL_DECODE_TARGET_WGS 3072
#endif
#ifndef WL_STREAM_ROWS
#define WL_STREAM_ROWS 2
#endif
#ifndef WL_STREAM_ROWS_MIN_T
#define WL_STREAM_ROWS_MIN_T 2
#endif
#ifndef WL_STREAM_WIDE_MIN_T
#define WL_STREAM_WIDE_MIN_T 8
#endif
#ifndef WL_STREAM_ROWS4_MIN_T
#define WL_STREAM_ROWS4_MIN_T 8
#endif
#ifndef WL_DECODE_TARGET_WGS_ROWS
#define WL_DECODE_TARGET_WGS_ROWS 2048
#endif
#ifndef WL_DECODE_TARGET_WGS_ROWS4
#define WL_DECODE_TARGET_WGS_ROWS4 1024
#endif
#ifndef WL_FP8_UNROLL
#define WL_FP8_UNROLL 2
#endif
#ifndef WL_FP8_KS_DIV
#define WL_FP8_KS_DIV 1
#endif
constexpr int kStreamWaves = WL_STREAM_WAVES;
constexpr int kStreamUnroll = WL_STREAM_UNROLL;
constexpr int kEpiWaves = WL_EPI_WAVES;
constexpr int kStreamRows = WL_STREAM_ROWS;         // row tiles per stream workgroup for T >= kStreamRowsMinT
constexpr int kStreamRowsMinT = WL_STREAM_ROWS_MIN_T;
constexpr int kStreamWideMinT = WL_STREAM_WIDE_MIN_T;
// from this many tokens on, W0 workgroups own twice kStreamRows row tiles
constexpr int kStreamRows4MinT = WL_STREAM_ROWS4_MIN_T;
constexpr int kTargetWgs = WL_DECODE_TARGET_WGS;
// K slices of the several-token path come from a lower workgroup target:
// each slice writes a T-token-wide fp32 partial that the epilogue re-reads
constexpr int kTargetWgsRows = WL_DECODE_TARGET_WGS_ROWS;
// and the four-tile path's from a lower one still (the 31B q|k|v then runs 4
// slices of 42 k-steps instead of 8 of 21)
constexpr int kTargetWgsRows4 = WL_DECODE_TARGET_WGS_ROWS4;
constexpr int kFp8Unroll = WL_FP8_UNROLL;
// MXFP4 W0: quads of 128 k per wave iteration, and the slice count is the
// bf16 path's divided by kFp4KsDiv (a slice of codes is a quarter of the bytes)
#ifndef WL_FP4_UNROLL
#define WL_FP4_UNROLL 2
#endif
#ifndef WL_FP4_KS_DIV
#define WL_FP4_KS_DIV 2
#endif
constexpr int kFp4Unroll = WL_FP4_UNROLL;
constexpr int kFp4KsDiv = WL_FP4_KS_DIV;
// with an FP8 W0 the one-tile stream launch splits V^T rows in two K slices
// from this K on
#ifndef WL_VT_SPLIT_K
#define WL_VT_SPLIT_K 16384
#endif
constexpr int kVtSplitK = WL_VT_SPLIT_K;
// and with an MXFP4 W0 (a quarter of the bytes) from this K on
#ifndef WL_VT_SPLIT_K_FP4
#define WL_VT_SPLIT_K_FP4 8192
#endif
constexpr int kVtSplitKFp4 = WL_VT_SPLIT_K_FP4;
// from this K on, one-token bf16 calls give the V^T tiles longer k blocks
#ifndef WL_VT_WIDE_K
#define WL_VT_WIDE_K 5120
#endif
constexpr int kVtWideK = WL_VT_WIDE_K;
// bf16 W0: calls with fewer rows than this and K >= WL_VT_SPLIT_MIN_K split
// their V^T tiles in two K slices (their W0 stream is short, and a V^T tile
// over the whole K would be the last workgroup still running)
#ifndef WL_VT_SPLIT_ROWS
#define WL_VT_SPLIT_ROWS 4096
#endif
#ifndef WL_VT_SPLIT_MIN_K
#define WL_VT_SPLIT_MIN_K 2048
#endif
// bf16 W0, one-tile stream launch: slices shorter than this many k-steps
// are merged when the split would need more than WL_RESIDENT_WGS workgroups
// (about one round of resident 8-wave stream workgroups on the chip)
#ifndef WL_SHORT_SLICE_STEPS
#define WL_SHORT_SLICE_STEPS 32
#endif
#ifndef WL_RESIDENT_WGS
#define WL_RESIDENT_WGS 768
#endif

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

// 16 E4M3 codes (one 16-byte load) -> two bf16 MFMA fragments: elements
// 0..7 and 8..15.  v_cvt_scalef32_pk_bf16_fp8 converts two codes per
// instruction; with scale 1 the result is exact (3 mantissa bits fit in 7).
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 w, u32x4 &lo, u32x4 &hi) {
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, false));
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, true));
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte
// i) times their block scale sc -> one bf16 MFMA fragment.  Exact: an E2M1
// value times a power of two inside the bf16 range.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t w, float sc) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3))};
}

// FP8 W0 rows: one 16-byte load per lane covers two 32-k MFMA steps.  Lane
// group g of pair p holds k = 64p + 16g .. +15; step "lo" takes k 64p + 16g
// + 0..7 and step "hi" k 64p + 16g + 8..15 (for all four g these are 32
// distinct k, and x is loaded with the same assignment).
template <int UNROLL>
__device__ __forceinline__ void kblock_fp8(f32x4 &acc, const uint8_t *arow, const uint16_t *xrow, bool tok_ok,
                                           int p0) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 a[UNROLL], b0[UNROLL], b1[UNROLL];
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) a[j] = *reinterpret_cast<const u32x4 *>(arow + (p0 + j) * 64);
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) {
    const u32x4 v0 = ld16(xrow + (p0 + j) * 64), v1 = ld16(xrow + (p0 + j) * 64 + 8);
    b0[j] = tok_ok ? v0 : zero4;
    b1[j] = tok_ok ? v1 : zero4;
  }
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) {
    u32x4 lo, hi;
    fp8x16_to_bf16(a[j], lo, hi);
    acc = mfma16x16x32(lo, b0[j], acc);
    acc = mfma16x16x32(hi, b1[j], acc);
  }
}

// z = V^T x of four ranks rb .. rb+3 of token t, from one V^T workgroup.
// Unsplit (KSV == 1): stored as a bf16 pair, z_hi [T][Rz] = bf16(z) and then
// z_lo [T][Rz] = bf16(z - z_hi) (~16 significant bits), the MFMA operands
// of the epilogue.  Split over K into two slices (KSV == 2, long K): each
// slice's fp32 partial at [slice][T][Rz]; the epilogue adds the two.
__device__ __forceinline__ void store_z(void *zbuf, int KSV, int slice, int T, int Rz, int t, int rb, int nrows,
                                        f32x4 v) {
  if (KSV == 1) {
    uint16_t *zh = static_cast<uint16_t *>(zbuf) + static_cast<size_t>(t) * Rz;
    uint16_t *zl = zh + static_cast<size_t>(T) * Rz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rb + i < nrows) {
        const uint16_t hi = f32_to_bf16(v[i]);
        zh[rb + i] = hi;
        zl[rb + i] = f32_to_bf16(v[i] - bf16_to_f32(hi));
      }
    }
    return;
  }
  float *zp = static_cast<float *>(zbuf) + (static_cast<size_t>(slice) * T + t) * Rz;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (rb + i < nrows) zp[rb + i] = v[i];
}

// Eight consecutive ranks of z for one token (element offset `off` = token
// * Rz + rank in the z region) as the epilogue's two MFMA B operands: the
// stored bf16 pair (KSV == 1), or, split in two (KSV == 2), the sum of the
// two fp32 slice partials (slice 0 first) split into hi = bf16(z) and
// lo = bf16(z - hi).
__device__ __forceinline__ void load_z8(const void *zbuf, int KSV, int T, int Rz, size_t off, u32x4 &h, u32x4 &l) {
  if (KSV == 1) {
    const uint16_t *zh = static_cast<const uint16_t *>(zbuf) + off;
    h = ld16(zh);
    l = ld16(zh + static_cast<size_t>(T) * Rz);
    return;
  }
  const float *zp = static_cast<const float *>(zbuf) + off;
  const size_t sst = static_cast<size_t>(T) * Rz;
  const f32x4 a0 = *reinterpret_cast<const f32x4 *>(zp), b0 = *reinterpret_cast<const f32x4 *>(zp + 4);
  const f32x4 a1 = *reinterpret_cast<const f32x4 *>(zp + sst), b1 = *reinterpret_cast<const f32x4 *>(zp + sst + 4);
  const f32x4 za = a0 + a1, zb = b0 + b1;
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float z0 = i < 2 ? za[2 * i] : zb[2 * i - 4], z1 = i < 2 ? za[2 * i + 1] : zb[2 * i - 3];
    const uint16_t h0 = f32_to_bf16(z0), h1 = f32_to_bf16(z1);
    hw[i] = h0 | (static_cast<uint32_t>(h1) << 16);
    lw[i] = f32_to_bf16(z0 - bf16_to_f32(h0)) | (static_cast<uint32_t>(f32_to_bf16(z1 - bf16_to_f32(h1))) << 16);
  }
  h = u32x4{hw[0], hw[1], hw[2], hw[3]};
  l = u32x4{lw[0], lw[1], lw[2], lw[3]};
}

// 1-D grid: first the V^T tiles (full K, so z needs no summation later; they
// are dispatched first and finish well inside the launch), then the W0 tiles,
// each split into KS slices of K.
// XL (FP8 or MXFP4 W0 at T = 1): x staged in LDS (dynamic shared memory of
// the slice's x row: ceil(pairs / KS) * 128 or ceil(quads / KS) * 256 bytes).
// VTU: k-steps per block for the V^T tiles (bf16 W0), which run the whole K
// while a W0 workgroup runs one slice of it.
template <int W, int UNROLL, bool XL = false, int VTU = UNROLL>
__global__ __launch_bounds__(W * 64) void stream_kernel(CallDesc c, float *p_part, void *zbuf, int nwg_vt, int KSV,
                                                        int KS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  // the first nwg_vt workgroups are the V^T tiles, KSV slices of K each;
  // then the W0 tiles, KS slices each
  const bool vt = static_cast<int>(blockIdx.x) < nwg_vt;
  const int widx = blockIdx.x - nwg_vt;
  const int row0 = (vt ? blockIdx.x / KSV : widx / KS) * 16;
  const int slice = vt ? blockIdx.x % KSV : widx % KS;
  const int nslices = vt ? KSV : KS;
  const uint16_t *mat = vt ? c.Vt : c.W0;  // (null for a coded bundle's W0 tiles, which read W0f8 / W0f4)
  const int nrows = vt ? c.Rz : c.Ntot;
  const int K = c.K;
  const int nsteps = (K + 31) >> 5;
  const int per = (nsteps + nslices - 1) / nslices;
  const int s_begin = min(nsteps, slice * per), s_end = min(nsteps, s_begin + per);

  // Rows past the end read the tile's first row (always valid); their
  // results are never stored.  Token columns >= T are zero.
  const int arow_idx = (row0 + r16 < nrows) ? row0 + r16 : row0;
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  if (!vt && c.W0f8) {
    // FP8 W0: K is walked in pairs of 32-k steps (64 k per 16-byte load);
    // slices split the pairs.  Codes past K are zero (row padding to ldw0),
    // x past K is skipped by the per-half guard.
    const int npairs = (K + 63) >> 6;
    const int pper = (npairs + KS - 1) / KS;
    const int p_begin = min(npairs, slice * pper), p_end = min(npairs, p_begin + pper);
    const uint8_t *arow8 = c.W0f8 + static_cast<size_t>(arow_idx) * c.ldw0 + g * 16;
    const uint16_t *xrow8 = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 16;
    const int pfull_end = min(p_end, K >> 6);  // pairs entirely inside K
    const int npb = max(0, pfull_end - p_begin) / kFp8Unroll;
    if constexpr (XL) {
      // one token: the slice's x row staged in LDS once per workgroup, so
      // the loop issues one global load (16 codes) per two MFMA steps rather
      // than three
      extern __shared__ u32x4 xs[];
      const int nch = (p_end - p_begin) * 8;
      for (int t = threadIdx.x; t < nch; t += W * 64) {
        const int k = p_begin * 64 + t * 8;
        xs[t] = k < K ? ld16(c.x + k) : zero4;
      }
      __syncthreads();
      for (int b = wave; b < npb; b += W) {
        const int p0 = p_begin + b * kFp8Unroll;
        u32x4 av[kFp8Unroll], b0[kFp8Unroll], b1[kFp8Unroll];
#pragma unroll
        for (int j = 0; j < kFp8Unroll; ++j) av[j] = *reinterpret_cast<const u32x4 *>(arow8 + (p0 + j) * 64);
#pragma unroll
        for (int j = 0; j < kFp8Unroll; ++j) {
          const int base = (p0 + j - p_begin) * 8 + g * 2;
          b0[j] = tok_ok ? xs[base] : zero4;
          b1[j] = tok_ok ? xs[base + 1] : zero4;
        }
#pragma unroll
        for (int j = 0; j < kFp8Unroll; ++j) {
          u32x4 lo, hi;
          fp8x16_to_bf16(av[j], lo, hi);
          acc = mfma16x16x32(lo, b0[j], acc);
          acc = mfma16x16x32(hi, b1[j], acc);
        }
      }
    } else {
      for (int b = wave; b < npb; b += W) kblock_fp8<kFp8Unroll>(acc, arow8, xrow8, tok_ok, p_begin + b * kFp8Unroll);
    }
    for (int pp = p_begin + npb * kFp8Unroll + wave; pp < p_end; pp += W) {
      const int k0 = pp * 64 + g * 16;
      const u32x4 a = k0 < c.ldw0 ? *reinterpret_cast<const u32x4 *>(arow8 + pp * 64) : zero4;
      const u32x4 v0 = k0 < K ? ld16(xrow8 + pp * 64) : zero4;
      const u32x4 v1 = k0 + 8 < K ? ld16(xrow8 + pp * 64 + 8) : zero4;
      u32x4 lo, hi;
      fp8x16_to_bf16(a, lo, hi);
      acc = mfma16x16x32(lo, tok_ok ? v0 : zero4, acc);
      acc = mfma16x16x32(hi, tok_ok ? v1 : zero4, acc);
    }
  } else if (!vt && c.W0f4) {
    // MXFP4 W0: K in quads of 128 (four 32-element blocks, one per lane
    // group); lane group g of quad p holds block 4p + g, k = 128p + 32g ..
    // +31, whose four 8-code words feed four MFMA steps: step j takes k =
    // 128p + 32g + 8j .. +7 (32 distinct k over the four lane groups), and x
    // is loaded with the same assignment.  Slices split the quads; codes past
    // K are zero (rows padded to a multiple of 128), x past K is not loaded.
    const int nq = c.ldw0 / 64;
    const int qper = (nq + KS - 1) / KS;
    const int q_begin = min(nq, slice * qper), q_end = min(nq, q_begin + qper);
    const uint8_t *arow4 = c.W0f4 + static_cast<size_t>(arow_idx) * c.ldw0 + g * 16;
    const uint8_t *srow = c.sc4 + static_cast<size_t>(arow_idx) * c.ldsc + g;
    const uint16_t *xrow4 = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 32;
    constexpr int QU = kFp4Unroll;
    // one token (XL): the slice's x row staged in LDS once per workgroup, so
    // the loop issues one global load per 32 codes instead of five
    extern __shared__ u32x4 xs[];
    if constexpr (XL) {
      const int nch = (q_end - q_begin) * 16;
      for (int t = threadIdx.x; t < nch; t += W * 64) {
        const int k = q_begin * 128 + t * 8;
        xs[t] = k < K ? ld16(c.x + k) : zero4;
      }
      __syncthreads();
    }
    for (int q0 = q_begin + wave * QU; q0 < q_end; q0 += W * QU) {
      u32x4 a[QU], xv[QU][4];
      uint32_t b[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int qq = min(q0 + u, q_end - 1);  // a quad past the slice re-reads the last and is dropped
        a[u] = *reinterpret_cast<const u32x4 *>(arow4 + static_cast<size_t>(qq) * 64);
        b[u] = srow[static_cast<size_t>(qq) * 4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (XL) {
            xv[u][j] = xs[(qq - q_begin) * 16 + g * 4 + j];
          } else {
            const int k = qq * 128 + g * 32 + j * 8;
            xv[u][j] = k < K ? ld16(xrow4 + qq * 128 + j * 8) : zero4;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        if (q0 + u >= q_end) break;
        const float sc = __uint_as_float(b[u] << 23);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16x16x32(fp4x8_to_bf16(a[u][j], sc), tok_ok ? xv[u][j] : zero4, acc);
      }
    }
  } else {
    const uint16_t *arow = mat + static_cast<size_t>(arow_idx) * K + g * 8;
    const int nfull_end = min(s_end, K >> 5);  // steps entirely inside K
    int s_tail;
    if (VTU != UNROLL && vt) {
      const int nblocks = max(0, nfull_end - s_begin) / VTU;
      for (int b = wave; b < nblocks; b += W) kblock<VTU>(acc, arow, xrow, tok_ok, s_begin + b * VTU);
      s_tail = s_begin + nblocks * VTU;
    } else {
      const int nblocks = max(0, nfull_end - s_begin) / UNROLL;
      for (int b = wave; b < nblocks; b += W) kblock<UNROLL>(acc, arow, xrow, tok_ok, s_begin + b * UNROLL);
      s_tail = s_begin + nblocks * UNROLL;
    }
    for (int s = s_tail + wave; s < s_end; s += W) {
      const bool kin = s * 32 + g * 8 < K;  // the last step may be partial
      const u32x4 a = kin ? ld16(arow + s * 32) : zero4;
      const u32x4 v = kin ? ld16(xrow + s * 32) : zero4;
      acc = mfma16x16x32(a, tok_ok ? v : zero4, acc);
    }
  }

  __shared__ f32x4 red[W][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  f32x4 tot = red[0][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) tot += red[w][lane];
  // lane holds D[m = 4g + i][n = r16]: rows row0 + 4g + i, token r16
  if (vt) {
    store_z(zbuf, KSV, slice, c.T, c.Rz, r16, row0 + g * 4, nrows, tot);
    return;
  }
  float *dst = p_part + (static_cast<size_t>(slice) * c.T + r16) * c.Ntot;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + g * 4 + i;
    if (row < nrows) dst[row] = tot[i];
  }
}

// The stream launch for several tokens (bf16 W0): like stream_kernel, but a
// workgroup owns R consecutive 16-row tiles and every wave multiplies each x
// fragment it loads into all R of them.  With T > 1 the x fragments are real
// rows (16 cache lines a load, as many as a W0 fragment), and loading them
// once per R row blocks cuts the operand traffic into the CU from 2x to
// (1 + 1/R)x the W0 bytes.  Waves 0..R-1 each reduce one tile.
template <int W, int UNROLL, int R>
__global__ __launch_bounds__(W * 64) void stream_rows_kernel(CallDesc c, float *p_part, void *zbuf,
                                                             int ntile_vt, int KS) {
  static_assert(W >= R, "one reducing wave per tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const bool vt = static_cast<int>(blockIdx.x) < ntile_vt;
  const int widx = blockIdx.x - ntile_vt;
  // V^T tiles (full K) stay 16 rows; W0 workgroups own R tiles
  const int row0 = vt ? blockIdx.x * 16 : (widx / KS) * 16 * R;
  const int nb = vt ? 1 : R;  // tiles of this workgroup
  const int slice = vt ? 0 : widx % KS;
  const int nslices = vt ? 1 : KS;
  const uint16_t *mat = vt ? c.Vt : c.W0;
  const int nrows = vt ? c.Rz : c.Ntot;
  const int K = c.K;
  const int nsteps = (K + 31) >> 5;
  const int per = (nsteps + nslices - 1) / nslices;
  const int s_begin = min(nsteps, slice * per), s_end = min(nsteps, s_begin + per);

  // Rows past the end read the workgroup's first row (always valid); their
  // results are never stored.  Token columns >= T are zero.
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;
  const uint16_t *arow[R];
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const int r = row0 + 16 * b + r16;
    arow[b] = mat + static_cast<size_t>(r < nrows ? r : row0) * K + g * 8;
  }
  f32x4 acc[R];
#pragma unroll
  for (int b = 0; b < R; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int nfull_end = min(s_end, K >> 5);  // steps entirely inside K
  const int nblocks = max(0, nfull_end - s_begin) / UNROLL;
  for (int bk = wave; bk < nblocks; bk += W) {
    const int s0 = s_begin + bk * UNROLL;
    u32x4 a[R][UNROLL], xb[UNROLL];
#pragma unroll
    for (int b = 0; b < R; ++b)
      if (b < nb) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) a[b][j] = ld16(arow[b] + (s0 + j) * 32);
      }
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      // unconditional load (row clamped to a valid one), then select
      const u32x4 v = ld16(xrow + (s0 + j) * 32);
      xb[j] = tok_ok ? v : zero4;
    }
#pragma unroll
    for (int b = 0; b < R; ++b)
      if (b < nb) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) acc[b] = mfma16x16x32(a[b][j], xb[j], acc[b]);
      }
  }
  for (int s = s_begin + nblocks * UNROLL + wave; s < s_end; s += W) {
    const bool kin = s * 32 + g * 8 < K;  // the last step may be partial
    const u32x4 v = kin ? ld16(xrow + s * 32) : zero4;
#pragma unroll
    for (int b = 0; b < R; ++b)
      if (b < nb) {
        const u32x4 a = kin ? ld16(arow[b] + s * 32) : zero4;
        acc[b] = mfma16x16x32(a, tok_ok ? v : zero4, acc[b]);
      }
  }

  __shared__ f32x4 red[W][R][64];
#pragma unroll
  for (int b = 0; b < R; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave >= nb || !tok_ok) return;
  const int b = wave;  // this wave reduces tile b (waves in a fixed order)
  f32x4 tot = red[0][b][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) tot += red[w][b][lane];
  const int tile0 = row0 + 16 * b;
  // lane holds D[m = 4g + i][n = r16]: rows tile0 + 4g + i, token r16
  if (vt) {
    store_z(zbuf, 1, 0, c.T, c.Rz, r16, tile0 + g * 4, nrows, tot);
    return;
  }
  float *dst = p_part + (static_cast<size_t>(slice) * c.T + r16) * c.Ntot;
  const int rb = tile0 + g * 4;
  if (rb + 3 < nrows && ((reinterpret_cast<uintptr_t>(dst + rb)) & 15) == 0) {
    *reinterpret_cast<f32x4 *>(dst + rb) = tot;  // four rows with one store
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb + i;
    if (row < nrows) dst[row] = tot[i];
  }
}

// One workgroup per 16-row tile; its WE waves split the rank steps of U z.
// KSM >= KS bounds the K slices whose partials wave 0 holds (so a call
// with few slices keeps few registers and more workgroups resident).
template <int WE, int KSM>
__global__ __launch_bounds__(WE * 64) void epilogue_kernel(CallDesc c, const float *p_part, const void *zbuf,
                                                           int KSV, int KS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const bool tok_ok = r16 < c.T;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int rbase = row0 + g * 4;

  // wave 0 loads the p partials and s of this lane's rows rbase..+3, token
  // r16; they are summed (in slice order) only after the delta, so these
  // loads and those of U and z are in flight together.  Slices past KS are
  // not loaded; rows past Ntot re-read a valid address and are dropped.
  f32x4 part[KSM];
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && tok_ok) {
    const size_t sstride = static_cast<size_t>(c.T) * c.Ntot;
    const float *pp = p_part + static_cast<size_t>(r16) * c.Ntot;
    // an FP8 bundle's rows carry their W0 scale q too: s q p
    const float *qrow = c.q;
    if (rbase + 3 < c.Ntot && (c.Ntot & 3) == 0 &&
        ((reinterpret_cast<uintptr_t>(c.s) | reinterpret_cast<uintptr_t>(qrow)) & 15) == 0) {
#pragma unroll
      for (int s = 0; s < KSM; ++s)
        part[s] = s < KS ? *reinterpret_cast<const f32x4 *>(pp + static_cast<size_t>(s) * sstride + rbase) : f32x4{0.f, 0.f, 0.f, 0.f};
      sc = *reinterpret_cast<const f32x4 *>(c.s + rbase);
      if (qrow) sc *= *reinterpret_cast<const f32x4 *>(qrow + rbase);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = min(rbase + i, c.Ntot - 1);
#pragma unroll
        for (int s = 0; s < KSM; ++s) part[s][i] = s < KS ? pp[static_cast<size_t>(s) * sstride + row] : 0.f;
        sc[i] = c.s[row] * (qrow ? qrow[row] : 1.f);
      }
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
    // z of this lane's token (token 0 stands in for columns >= T)
    const size_t zrow = static_cast<size_t>(tok_ok ? r16 : 0) * c.Rz + ch.zoff + g * 8;
    // kk and k1 are multiples of 32 and rpad is too, so a step is either
    // wholly inside the padded rank or wholly outside.  Every load is
    // unconditional (an outside step re-reads step kk) and issued before the
    // MFMAs, so all of a wave's loads are in flight together.
    for (int kk = wave * 32; kk < ch.rpad; kk += 2 * WE * 32) {
      const int k1 = kk + WE * 32;
      const bool in1 = k1 < ch.rpad;
      const int k1c = in1 ? k1 : kk;
      const u32x4 ua0 = ld16(urow + kk), ua1 = ld16(urow + k1c);
      u32x4 h0, l0, h1, l1;
      load_z8(zbuf, KSV, c.T, c.Rz, zrow + kk, h0, l0);
      load_z8(zbuf, KSV, c.T, c.Rz, zrow + k1c, h1, l1);
      const u32x4 a0 = in_child ? ua0 : zero4;
      const u32x4 a1 = (in1 && in_child) ? ua1 : zero4;
      dacc = mfma16x16x32(a0, tok_ok ? h0 : zero4, dacc);
      dacc = mfma16x16x32(a0, tok_ok ? l0 : zero4, dacc);
      dacc = mfma16x16x32(a1, (in1 && tok_ok) ? h1 : zero4, dacc);
      dacc = mfma16x16x32(a1, (in1 && tok_ok) ? l1 : zero4, dacc);
    }
  }
  __shared__ f32x4 red[WE][64];
  red[wave][lane] = dacc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  f32x4 d = red[0][lane];
#pragma unroll
  for (int w = 1; w < WE; ++w) d += red[w][lane];
  f32x4 p = part[0];
#pragma unroll
  for (int s = 1; s < KSM; ++s)
    if (s < KS) p += part[s];

  // lane holds D[m = 4g + i][n = r16]: rows rbase + i, token r16
  uint16_t *yrow = c.y + static_cast<size_t>(r16) * c.ldy;
  {
    // four rows of one child with 8-byte aligned destinations: one store each
    int ci = 0;
    while (ci + 1 < c.nchild && rbase >= c.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = c.ch[ci];
    const int j = rbase - ch.row_start;
    uint16_t *y0 = yrow + ch.y_off + j;
    uint16_t *y1 = ch.dup_off >= 0 ? yrow + ch.dup_off + j : y0;
    if (j + 3 < ch.N && ((reinterpret_cast<uintptr_t>(y0) | reinterpret_cast<uintptr_t>(y1)) & 7) == 0) {
      u32x2 o;
      o[0] = f32_to_bf16(sc[0] * p[0] + d[0]) | (static_cast<uint32_t>(f32_to_bf16(sc[1] * p[1] + d[1])) << 16);
      o[1] = f32_to_bf16(sc[2] * p[2] + d[2]) | (static_cast<uint32_t>(f32_to_bf16(sc[3] * p[3] + d[3])) << 16);
      *reinterpret_cast<u32x2 *>(y0) = o;
      if (ch.dup_off >= 0) *reinterpret_cast<u32x2 *>(y1) = o;
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + i;
    if (row >= c.Ntot) continue;
    int ci = 0;
    while (ci + 1 < c.nchild && row >= c.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = c.ch[ci];
    const uint16_t out = f32_to_bf16(sc[i] * p[i] + d[i]);
    const int j = row - ch.row_start;
    yrow[ch.y_off + j] = out;
    if (ch.dup_off >= 0) yrow[ch.dup_off + j] = out;
  }
}

// Fused gate|up epilogue: h[t][j] = act(gate_j) * up_j with gate_j =
// s_j p_j + (U_gate z_gate)_j and up_j the same on row N_g + j (children 0 and
// 1 of the call, N_g rows each).  One workgroup per 16 values of j; its WE
// waves split the rank steps of both deltas.
template <int WE, int KSM>
__global__ __launch_bounds__(WE * 64) void act_epilogue_kernel(CallDesc c, const float *p_part,
                                                               const void *zbuf, int KSV, int KS, int act,
                                                               uint16_t *h, int ldh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int Ng = c.ch[0].N;
  const int j0 = blockIdx.x * 16;
  const bool tok_ok = r16 < c.T;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // wave 0: p partials (slices < KS) and s of rows j0 + 4g + i of both halves
  // (rows past N_g re-read row N_g - 1 of the half and are dropped); summed
  // after the deltas so all loads are in flight together
  float part[2][KSM][4];
  float sc[2][4];
  if (wave == 0 && tok_ok) {
    const size_t sstride = static_cast<size_t>(c.T) * c.Ntot;
    const float *pp = p_part + static_cast<size_t>(r16) * c.Ntot;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = c.ch[hf].row_start + min(j0 + 4 * g + i, Ng - 1);
#pragma unroll
        for (int s = 0; s < KSM; ++s)
          part[hf][s][i] = s < KS ? pp[static_cast<size_t>(s) * sstride + row] : 0.f;
        sc[hf][i] = c.s[row] * (c.q ? c.q[row] : 1.f);
      }
  }

  f32x4 dacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const bool in_rows = j0 + r16 < Ng;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const ChildDesc &ch = c.ch[hf];
    if (ch.rpad == 0) continue;
    const uint16_t *urow = ch.U + static_cast<size_t>(in_rows ? j0 + r16 : 0) * ch.rpad + g * 8;
    const size_t zrow = static_cast<size_t>(tok_ok ? r16 : 0) * c.Rz + ch.zoff + g * 8;
    for (int kk = wave * 32; kk < ch.rpad; kk += 2 * WE * 32) {
      const int k1 = kk + WE * 32;
      const bool in1 = k1 < ch.rpad;
      const int k1c = in1 ? k1 : kk;
      const u32x4 ua0 = ld16(urow + kk), ua1 = ld16(urow + k1c);
      u32x4 h0, l0, h1, l1;
      load_z8(zbuf, KSV, c.T, c.Rz, zrow + kk, h0, l0);
      load_z8(zbuf, KSV, c.T, c.Rz, zrow + k1c, h1, l1);
      const u32x4 a0 = in_rows ? ua0 : zero4;
      const u32x4 a1 = (in1 && in_rows) ? ua1 : zero4;
      dacc[hf] = mfma16x16x32(a0, tok_ok ? h0 : zero4, dacc[hf]);
      dacc[hf] = mfma16x16x32(a0, tok_ok ? l0 : zero4, dacc[hf]);
      dacc[hf] = mfma16x16x32(a1, (in1 && tok_ok) ? h1 : zero4, dacc[hf]);
      dacc[hf] = mfma16x16x32(a1, (in1 && tok_ok) ? l1 : zero4, dacc[hf]);
    }
  }
  __shared__ f32x4 red[WE][2][64];
  red[wave][0][lane] = dacc[0];
  red[wave][1][lane] = dacc[1];
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  float y[2][4];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 d = red[0][hf][lane];
#pragma unroll
    for (int w = 1; w < WE; ++w) d += red[w][hf][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p = part[hf][0][i];
#pragma unroll
      for (int s = 1; s < KSM; ++s)
        if (s < KS) p += part[hf][s][i];
      y[hf][i] = sc[hf][i] * p + d[i];
    }
  }
  uint16_t *hrow = h + static_cast<size_t>(r16) * ldh;
  const int jb = j0 + 4 * g;
  if (jb + 3 < Ng && (reinterpret_cast<uintptr_t>(hrow + jb) & 7) == 0) {
    // four values with one 8-byte store
    u32x2 o;
    o[0] = f32_to_bf16(activation(act, y[0][0]) * y[1][0]) |
           (static_cast<uint32_t>(f32_to_bf16(activation(act, y[0][1]) * y[1][1])) << 16);
    o[1] = f32_to_bf16(activation(act, y[0][2]) * y[1][2]) |
           (static_cast<uint32_t>(f32_to_bf16(activation(act, y[0][3]) * y[1][3])) << 16);
    *reinterpret_cast<u32x2 *>(hrow + jb) = o;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = jb + i;
    if (j < Ng) hrow[j] = f32_to_bf16(activation(act, y[0][i]) * y[1][i]);
  }
}

}  // namespace

namespace {
int k_slices_for(int Ntot, int Rz, int K, int target) {
  // Aim for about `target` workgroups in the stream launch, with K slices
  // of at least 16 k-steps and at most kDecodeMaxSlices slices.
  const int tiles = (Ntot + 15) / 16 + (Rz + 15) / 16;
  const int nsteps = (K + 31) / 32;
  int ks = (target + tiles - 1) / max(1, tiles);
  ks = min(ks, max(1, nsteps / 16));
  return max(1, min(ks, kDecodeMaxSlices));
}
}  // namespace

int decode_k_slices(int Ntot, int Rz, int K) { return k_slices_for(Ntot, Rz, K, kTargetWgs); }

template <int KSM>
hipError_t launch_epilogue(const CallDesc &c, const float *p_part, const void *zbuf, int KSV, int KS,
                           hipStream_t stream, int act, uint16_t *h, int ldh) {
  if (act < 0) {
    hipLaunchKernelGGL((epilogue_kernel<kEpiWaves, KSM>), dim3((c.Ntot + 15) / 16), dim3(kEpiWaves * 64), 0, stream,
                       c, p_part, zbuf, KSV, KS);
  } else {
    hipLaunchKernelGGL((act_epilogue_kernel<kEpiWaves, KSM>), dim3((c.ch[0].N + 15) / 16), dim3(kEpiWaves * 64), 0,
                       stream, c, p_part, zbuf, KSV, KS, act, h, ldh);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const CallDesc &c, float *p_part, void *z_pair, hipStream_t stream, int act,
                         uint16_t *h, int ldh) {
  const int nt_w0 = (c.Ntot + 15) / 16;
  int KS, KSV = 1;
  const int KS1 = decode_k_slices(c.Ntot, c.Rz, c.K);
  constexpr int R = kStreamRows, R4 = 2 * kStreamRows;
  const int ks_rows = min(KS1, k_slices_for(c.Ntot, c.Rz, c.K, kTargetWgsRows));
  const int ks_rows4 = min(KS1, k_slices_for(c.Ntot, c.Rz, c.K, kTargetWgsRows4));
  if (c.W0 != nullptr && c.T >= kStreamRows4MinT && R4 * ks_rows4 <= kDecodeMaxSlices) {
    // eight or more tokens: R4 row tiles per W0 workgroup share each x
    // fragment (the x bytes pulled from L2 per W0 byte halve again), with R4
    // times the slices of the four-tile target; blocks of two k-steps
    // where every wave gets at least two such blocks of a slice, else single
    // steps, so the slice's steps stay spread over all waves
    KS = R4 * ks_rows4;
    const int per = ((c.K + 31) / 32 + KS - 1) / KS;
    const int nw_w0 = (c.Ntot + 16 * R4 - 1) / (16 * R4), nt_vt = (c.Rz + 15) / 16;
    if (per >= 2 * 2 * kStreamWaves)
      hipLaunchKernelGGL((stream_rows_kernel<kStreamWaves, 2, R4>), dim3(nt_vt + nw_w0 * KS),
                         dim3(kStreamWaves * 64), 0, stream, c, p_part, z_pair, nt_vt, KS);
    else
      hipLaunchKernelGGL((stream_rows_kernel<kStreamWaves, 1, R4>), dim3(nt_vt + nw_w0 * KS),
                         dim3(kStreamWaves * 64), 0, stream, c, p_part, z_pair, nt_vt, KS);
  } else if (c.W0 != nullptr && c.T >= kStreamRowsMinT && KS1 * R <= kDecodeMaxSlices) {
    // several tokens: R row tiles per W0 workgroup share each x fragment,
    // with R times the slices of the lower several-token target (never more
    // than the R * KS1 <= kDecodeMaxSlices checked above)
    KS = R * ks_rows;
    const int nw_w0 = (c.Ntot + 16 * R - 1) / (16 * R), nt_vt = (c.Rz + 15) / 16;
    hipLaunchKernelGGL((stream_rows_kernel<kStreamWaves, kStreamUnroll, R>), dim3(nt_vt + nw_w0 * KS),
                       dim3(kStreamWaves * 64), 0, stream, c, p_part, z_pair, nt_vt, KS);
  } else if (c.W0 != nullptr && c.T >= kStreamWideMinT && KS1 == kDecodeMaxSlices &&
             ((c.K + 31) / 32 + KS1 - 1) / KS1 >= 2 * kStreamWaves * 2) {
    // several tokens, long K slices (o- and down-shaped calls): R4 row tiles
    // per workgroup on twice the waves at the full slice count, in 2-step
    // blocks (every wave gets at least one)
    KS = KS1;
    const int nw4 = (c.Ntot + 16 * R4 - 1) / (16 * R4), nt_vt = (c.Rz + 15) / 16;
    hipLaunchKernelGGL((stream_rows_kernel<2 * kStreamWaves, 2, R4>), dim3(nt_vt + nw4 * KS),
                       dim3(2 * kStreamWaves * 64), 0, stream, c, p_part, z_pair, nt_vt, KS);
  } else {
    KS = c.W0f8   ? max(1, decode_k_slices(c.Ntot, c.Rz, c.K) / WL_FP8_KS_DIV)
         : c.W0f4 ? max(1, (decode_k_slices(c.Ntot, c.Rz, c.K) + kFp4KsDiv - 1) / kFp4KsDiv)
                  : decode_k_slices(c.Ntot, c.Rz, c.K);
    if (c.W0 != nullptr) {
      // short slices: when the K split would take the launch past one round
      // of resident workgroups, fewer slices (each wave then streams more
      // of its rows) and a single round
      const int tiles = (c.Ntot + 15) / 16 + (c.Rz + 15) / 16, nsteps = (c.K + 31) / 32;
      if (nsteps / KS < WL_SHORT_SLICE_STEPS && tiles * KS > WL_RESIDENT_WGS && tiles <= WL_RESIDENT_WGS)
        KS = max(1, WL_RESIDENT_WGS / tiles);
    }
    // with a coded W0 (FP8, MXFP4) the W0 workgroups stream a half or a
    // quarter of the bytes, and over a long K (>= kVtSplitK, or
    // kVtSplitKFp4 for MXFP4) a V^T tile over the whole K is the last
    // workgroup still streaming: its rows are then split in two K slices
    // (FP8 down call 40.1 -> 33.7 us; MXFP4 o 22.0 -> 19.8 us, where the FP8
    // o call was 1.4 us slower split).  With bf16 W0 the split saves less in
    // the stream launch than the epilogue's extra z loads cost, except on
    // calls with few rows: the Gemma-3 down call, 1152 rows at K = 4096,
    // ran its two 128 KB V^T tiles for most of its stream launch.
    KSV = (((c.W0f8 != nullptr && c.K >= kVtSplitK) || (c.W0f4 != nullptr && c.K >= kVtSplitKFp4)) && KS >= 2)
              ? 2 : 1;
    if (c.W0 != nullptr && c.Ntot < WL_VT_SPLIT_ROWS && c.K >= WL_VT_SPLIT_MIN_K && KS >= 2) KSV = 2;
    const int nwg_vt = (c.Rz + 15) / 16 * KSV;
    if (c.T == 1 && (c.W0f8 != nullptr || c.W0f4 != nullptr)) {
      // x slice in LDS: 64 k (128 bytes) per FP8 pair, 128 k per MXFP4 quad
      size_t xbytes;
      if (c.W0f8) {
        const int npairs = (c.K + 63) / 64;
        xbytes = static_cast<size_t>((npairs + KS - 1) / KS) * 128;
      } else {
        const int nq = c.ldw0 / 64;
        xbytes = static_cast<size_t>((nq + KS - 1) / KS) * 256;
      }
      hipLaunchKernelGGL((stream_kernel<kStreamWaves, kStreamUnroll, true>), dim3(nwg_vt + nt_w0 * KS),
                         dim3(kStreamWaves * 64), xbytes, stream, c, p_part, z_pair, nwg_vt, KSV, KS);
    } else if (c.T == 1 && c.W0 != nullptr && c.K >= kVtWideK) {
      // one token, long K: the V^T tiles (whole K) take blocks of twice the
      // k-steps, so more of their bytes are in flight
      hipLaunchKernelGGL((stream_kernel<kStreamWaves, kStreamUnroll, false, 2 * kStreamUnroll>),
                         dim3(nwg_vt + nt_w0 * KS), dim3(kStreamWaves * 64), 0, stream, c, p_part, z_pair, nwg_vt,
                         KSV, KS);
    } else {
      hipLaunchKernelGGL((stream_kernel<kStreamWaves, kStreamUnroll>), dim3(nwg_vt + nt_w0 * KS),
                         dim3(kStreamWaves * 64), 0, stream, c, p_part, z_pair, nwg_vt, KSV, KS);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float *pp = static_cast<const float *>(p_part);
  if (KS <= 2) return launch_epilogue<2>(c, pp, z_pair, KSV, KS, stream, act, h, ldh);
  if (KS <= 4) return launch_epilogue<4>(c, pp, z_pair, KSV, KS, stream, act, h, ldh);
  return launch_epilogue<kDecodeMaxSlices>(c, pp, z_pair, KSV, KS, stream, act, h, ldh);
}

}  // namespace wl
