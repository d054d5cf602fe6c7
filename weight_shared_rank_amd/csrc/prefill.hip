// Prefill-path kernels (T > 16 tokens): two launches of one bf16 MFMA GEMM.
//
//   launch 1:  Z[T, Rz] = X[T, K] V              (the thin reduction, bf16 out)
//   launch 2:  Y[T, N]  = (X W0^T) (.) s + Z U^T   (scale and rank-r delta fused
//              into the epilogue of the shared-block GEMM; y written once)
//
// The forward is the theta-bundle forward ("Add a new model architecture"
// page, introduction); as in the pages' GEMM formulation the operands stay
// bf16 with fp32 accumulation ("Quality (Gemma 4 31B)" page, "Kernel
// optimizations > GEMM path").
//
// GEMM core (gfx950).  A workgroup owns a BM x BN output tile: BM weight rows
// ("features", MFMA A operand) by BN tokens (B operand).  Both operands are
// K-contiguous rows.  Tiles of 32 k are moved global -> LDS by
// global_load_lds_dwordx4 (no VGPR staging) into an NST-stage ring, so loads
// run NST-1 k-tiles ahead of the MFMAs.  Each wave instruction fills 16
// rows x 64 bytes (1 KB, lane i at byte 16 i); a lane fetches 16-byte chunk
// c = (i % 4) ^ ((i / 8) % 4) of row i / 4.  This XOR-swizzles the LDS rows
// (slot = chunk ^ ((row / 2) % 4)) so that each 8-lane phase of a 16-byte
// fragment read (8 consecutive rows, one chunk) covers the 32 LDS banks
// exactly once: no bank conflicts.  Lanes whose row or k lies outside the operand fetch a row of zeros
// kept in the arena, which is how tails and foreign rows are masked (an LDS
// DMA lane cannot be zero-filled).  Large tiles use eight waves (two per
// SIMD, 64 x 128 or 64 x 64 each), small ones four.
//
// Scheduling.  Workgroups are numbered XCD-major: hardware assigns
// workgroup w to XCD w % 8, and the tile order is remapped so that each XCD
// walks a contiguous range of (feature tile, K slice, token tile), token tile
// fastest: the token tiles that share a block of W0 run at the same time on
// one XCD and read it from HBM once (later reads hit that XCD's L2).
// Each launch takes the largest tile shape (256x256 down to 64x64) that
// still gives every CU a workgroup.  K is never split across workgroups:
// combining partial tiles across XCDs needs device-scope release/acquire,
// which on this part writes back / invalidates a whole L2 and costs more than
// the smaller tile.
//
// Epilogue of launch 2: the fp32 accumulators are scaled by s per feature
// row, then the same staged loop runs over the ranks of every child whose
// rows meet the tile (A = that child's U rows, other rows read the zero row;
// B = the child's columns of Z), so U z is added at MFMA rate before y is
// rounded to bf16 and stored.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kNST = 4;       // LDS ring stages
constexpr int kBK = 32;       // k per stage
constexpr int kRowBytes = 64; // kBK bf16 per LDS row

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

struct GemmArgs {
  // main segment: rows of A (weights) against rows of B (tokens), K long
  const uint16_t *A;
  int32_t M;
  int64_t lda;
  const uint16_t *B;
  int32_t T;
  int64_t ldb;
  int32_t K;
  const uint16_t *zero_row;  // >= 16 zero bytes
  // tiling
  int32_t nM, nT;     // feature tiles, token tiles
  // epilogue
  int32_t mode;       // 0: Y = bf16(acc) [T][ldy]; 1: scale + delta + child map
  uint16_t *Y;
  int32_t ldy;
  const float *s;
  const uint16_t *Z;  // [T][ldz] (mode 1)
  int32_t ldz;
  int32_t nchild;
  ChildDesc ch[kMaxChildren];
};

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int GA = BM / 16, GB = BN / 16;
  static constexpr int LPW = (GA + GB) / NW;  // LDS-DMA instructions per wave per stage
  static constexpr int STAGE = (BM + BN) * kRowBytes;
  static_assert((GA + GB) % NW == 0, "16-row groups must split evenly over the waves");
};

// One staged GEMM segment: acc += A[arow0 + ..] B[brow0 + ..]^T over k-steps
// [s_begin, s_end) of 32.  Row pointers are per load instruction, chosen by
// the caller (already offset to the lane's chunk); a null row pointer reads
// the zero row.  klen bounds the valid k (tail chunks read the zero row).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void segment(f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                        const uint16_t *const (&rp)[(BM + BN) / 16 / (WM * WN)], int klen,
                                        int s_begin, int s_end, const uint16_t *zero_row, uint8_t *lds) {
  using TL = Tile<BM, BN, WM, WN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lchunk = (lane & 3) ^ ((lane >> 3) & 3);
  const int nk = s_end - s_begin;
  int ldsoff[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    const int gq = wave * TL::LPW + q;
    ldsoff[q] = gq < TL::GA ? gq * 1024 : BM * kRowBytes + (gq - TL::GA) * 1024;
  }
  auto issue = [&](int stage, int step) {
    const int k = step * kBK + lchunk * 8;
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      const uint16_t *src = (rp[q] != nullptr && k < klen) ? rp[q] + step * kBK : zero_row;
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                       (lds_void *)(lds + stage * TL::STAGE + ldsoff[q]), 16, 0, 0);
    }
  };
  const int swz = (g ^ ((r16 >> 1) & 3)) * 16;
  const int aoff = (wm * TL::TM + r16) * kRowBytes + swz;
  const int boff = BM * kRowBytes + (wn * TL::TN + r16) * kRowBytes + swz;

#pragma unroll
  for (int st = 0; st < kNST - 1; ++st)
    if (st < nk) issue(st, s_begin + st);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of k-tile kt are done once at most (NST-2) tiles of
    // loads remain outstanding; the barrier then makes every wave's part of
    // the tile visible, and tells that stage kt-1 is no longer being read
    if (kt + kNST - 2 < nk)
      wait_vmcnt<(kNST - 2) * TL::LPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + kNST - 1 < nk) issue((kt + kNST - 1) % kNST, s_begin + kt + kNST - 1);
    const uint8_t *sb = lds + (kt % kNST) * TL::STAGE;
    u32x4 fa[TL::FM], fb[TL::FN];
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) fa[i] = *reinterpret_cast<const u32x4 *>(sb + aoff + i * 16 * kRowBytes);
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) fb[j] = *reinterpret_cast<const u32x4 *>(sb + boff + j * 16 * kRowBytes);
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
  }
  // every wave is done with the ring before it is refilled
  __builtin_amdgcn_s_barrier();
}

// Workgroup index -> (feature tile, token tile), XCD-major: hardware sends
// workgroup w to XCD w % 8; XCD x is given the contiguous unit range
// [x * per + min(x, rem), ...) so the token tiles of one feature tile run
// together on one XCD.
__device__ __forceinline__ void unit_of(int id, int total, int nT, int &f, int &t) {
  const int x = id & 7, j = id >> 3;
  const int per = total >> 3, rem = total & 7;
  const int u = x * per + min(x, rem) + j;
  f = u / nT;
  t = u % nT;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(GemmArgs a) {
  using TL = Tile<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 3) & 3);
  int f, t;
  unit_of(blockIdx.x, gridDim.x, a.nT, f, t);
  const int m0 = f * BM, n0 = t * BN;

  f32x4 acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // main segment row pointers: rows of A (features) then of B (tokens)
  {
    const uint16_t *rp[TL::LPW];
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      const int gq = wave * TL::LPW + q;
      if (gq < TL::GA) {
        const int row = m0 + gq * 16 + lrow;
        rp[q] = row < a.M ? a.A + row * a.lda + lchunk * 8 : nullptr;
      } else {
        const int row = n0 + (gq - TL::GA) * 16 + lrow;
        rp[q] = row < a.T ? a.B + row * a.ldb + lchunk * 8 : nullptr;
      }
    }
    segment<BM, BN, WM, WN>(acc, rp, a.K, 0, (a.K + kBK - 1) / kBK, a.zero_row, lds);
  }

  if (a.mode == 1) {
    // scale by s (rows outside [0, M) are never stored)
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int row = m0 + wm * TL::TM + i * 16 + g * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sc = row + e < a.M ? a.s[row + e] : 0.f;
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j][e] *= sc;
      }
    }
    // delta = Z U^T for every child with rows in this tile
    for (int ci = 0; ci < a.nchild; ++ci) {
      const ChildDesc &ch = a.ch[ci];
      if (ch.rpad == 0 || m0 >= ch.row_start + ch.N || m0 + BM <= ch.row_start) continue;
      const uint16_t *rp[TL::LPW];
#pragma unroll
      for (int q = 0; q < TL::LPW; ++q) {
        const int gq = wave * TL::LPW + q;
        if (gq < TL::GA) {
          const int row = m0 + gq * 16 + lrow;
          const bool in = row >= ch.row_start && row < ch.row_start + ch.N;
          rp[q] = in ? ch.U + static_cast<int64_t>(row - ch.row_start) * ch.rpad + lchunk * 8 : nullptr;
        } else {
          const int row = n0 + (gq - TL::GA) * 16 + lrow;
          rp[q] = row < a.T ? a.Z + static_cast<int64_t>(row) * a.ldz + ch.zoff + lchunk * 8 : nullptr;
        }
      }
      segment<BM, BN, WM, WN>(acc, rp, ch.rpad, 0, (ch.rpad + kBK - 1) / kBK, a.zero_row, lds);
    }
  }

  // store: lane holds rows m0 + wm*TM + 16i + 4g + e, token n0 + wn*TN + 16j + r16
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) {
    const int tok = n0 + wn * TL::TN + j * 16 + r16;
    if (tok >= a.T) continue;
    uint16_t *yrow = a.Y + static_cast<int64_t>(tok) * a.ldy;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int row = m0 + wm * TL::TM + i * 16 + g * 4;
      if (row >= a.M) continue;
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(acc[i][j][e]);
      if (a.mode == 0) {
        if (row + 3 < a.M && ((a.ldy | row) & 3) == 0) {
          *reinterpret_cast<uint2 *>(yrow + row) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
        } else {
          for (int e = 0; e < 4; ++e)
            if (row + e < a.M) yrow[row + e] = o[e];
        }
      } else {
        for (int e = 0; e < 4; ++e) {
          const int r = row + e;
          if (r >= a.M) break;
          int ci = 0;
          while (ci + 1 < a.nchild && r >= a.ch[ci + 1].row_start) ++ci;
          const ChildDesc &ch = a.ch[ci];
          const int jj = r - ch.row_start;
          yrow[ch.y_off + jj] = o[e];
          if (ch.dup_off >= 0) yrow[ch.dup_off + jj] = o[e];
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(kNST) * Tile<BM, BN, WM, WN>::STAGE;
  auto kern = gemm_kernel<BM, BN, WM, WN>;
  static bool attr_set = false;  // per instance; setting it twice is harmless
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(a.nM * a.nT), dim3(WM * WN * 64), lds, stream, a);
  return hipGetLastError();
}

// Tile shapes, largest first: (BM features, BN tokens, waves).
struct TileCfg {
  int BM, BN;
};
constexpr TileCfg kTiles[] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}, {64, 64}};

// The largest tile that still gives every CU a workgroup; else the smallest.
int pick_tile(int M, int T) {
  constexpr int kCUs = 256;
  const int n = sizeof(kTiles) / sizeof(kTiles[0]);
  for (int i = 0; i < n; ++i) {
    const long tiles = static_cast<long>((M + kTiles[i].BM - 1) / kTiles[i].BM) * ((T + kTiles[i].BN - 1) / kTiles[i].BN);
    if (tiles >= kCUs) return i;
  }
  return n - 1;
}

hipError_t launch_tiled(GemmArgs a, hipStream_t stream) {
  const int i = pick_tile(a.M, a.T);
  a.nM = (a.M + kTiles[i].BM - 1) / kTiles[i].BM;
  a.nT = (a.T + kTiles[i].BN - 1) / kTiles[i].BN;
  switch (i) {
    case 0: return launch_gemm<256, 256, 4, 2>(a, stream);
    case 1: return launch_gemm<256, 128, 4, 2>(a, stream);
    case 2: return launch_gemm<128, 128, 2, 2>(a, stream);
    case 3: return launch_gemm<128, 64, 2, 2>(a, stream);
    default: return launch_gemm<64, 64, 2, 2>(a, stream);
  }
}

}  // namespace

hipError_t launch_prefill(const CallDesc &c, uint16_t *zbuf, const uint16_t *zero_row, hipStream_t stream) {
  hipError_t e;
  if (c.Rz > 0) {
    GemmArgs a{};
    a.A = c.Vt;
    a.M = c.Rz;
    a.lda = c.K;
    a.B = c.x;
    a.T = c.T;
    a.ldb = c.K;
    a.K = c.K;
    a.zero_row = zero_row;
    a.mode = 0;
    a.Y = zbuf;
    a.ldy = c.Rz;
    e = launch_tiled(a, stream);
    if (e != hipSuccess) return e;
  }
  GemmArgs a{};
  a.A = c.W0;
  a.M = c.Ntot;
  a.lda = c.K;
  a.B = c.x;
  a.T = c.T;
  a.ldb = c.K;
  a.K = c.K;
  a.zero_row = zero_row;
  a.mode = 1;
  a.Y = c.y;
  a.ldy = c.ldy;
  a.s = c.s;
  a.Z = zbuf;
  a.ldz = c.Rz;
  a.nchild = c.nchild;
  for (int i = 0; i < c.nchild; ++i) a.ch[i] = c.ch[i];
  return launch_tiled(a, stream);
}

}  // namespace wl
