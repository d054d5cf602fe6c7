// Prefill-path kernels (T > 16 tokens): bf16 MFMA GEMMs.
//
//   Z[T, Rz] = X[T, K] V                          (the thin reduction, bf16)
//   Y[T, N]  = (X W0^T) (.) s + Z U^T               (scale and rank-r delta in
//              the epilogue of the shared-block GEMM; y written once)
//
// The forward is the theta-bundle forward ("Add a new model architecture"
// page, introduction); as in the pages' GEMM formulation the operands stay
// bf16 with fp32 accumulation ("Quality (Gemma 4 31B)" page, "Kernel
// optimizations > GEMM path").
//
// GEMM core (gfx950).  A workgroup owns a BM x BN output tile: BM weight rows
// ("features", MFMA A operand) by BN tokens (B operand).  Both operands are
// K-contiguous rows.  Stages of 64 k (128 bytes per row) move global -> LDS by
// buffer_load_dwordx4 ... lds (no VGPR staging) into an NST-stage ring.  One
// wave instruction fills 8 rows x 128 bytes: lane i writes LDS slot i % 8 of row
// i / 8 and fetches 16-byte chunk c = (i % 8) ^ (row % 8) of that row, so
// chunk c of row r sits in slot c ^ (r % 8).  A 16-byte fragment read (8
// lanes per LDS phase: 8 consecutive rows, one chunk) then touches 8
// different slots, i.e. all 32 banks once.  Whole 128-byte rows per request
// halve the per-CU request count of 64-byte rows, and the request rate per CU,
// not the MFMA rate, is what bounds the operand stream at a few hundred
// tokens.  Lanes whose row or k lies outside the operand take an offset past
// the load's buffer range, which the buffer unit returns as zeros.
//
// Scheduling.  Workgroups are numbered XCD-major: hardware assigns workgroup
// w to XCD w % 8, and the unit order is remapped so that each XCD walks a
// contiguous range of (feature tile, K slice, token tile), token tile
// fastest: the token tiles that share a block of W0 run together on one XCD
// and read it from HBM once (later reads hit that XCD's L2).
//
// Tile and split choice (plan_gemm).  Big tiles (256 x 128 on eight waves)
// stream the fewest bytes per flop and win when they fill the chip; GEMMs
// with few rows (o, down, and Z = X V) split K into KS slices instead, so
// that every CU streams.  Slices write fp32 partial tiles to the workspace;
// a later launch sums them in slice order (deterministic): a reduce kernel
// for Z, and for the main GEMM an elementwise finish kernel.  On a split main
// GEMM the last slice of each tile also computes the delta Z U^T (another K
// range of the same product, with U and Z as the operands) into a partial of
// its own, and takes that many fewer K steps, so the slices are balanced;
// the finish kernel forms s (.) sum(K partials) + delta.
// Partials are combined across launches, never across workgroups of one
// launch: that would need device-scope release/acquire, which writes back /
// invalidates a whole L2 on this part.
//
// Epilogue of the main GEMM: the fp32 accumulators are scaled by s per
// feature row, then the same staged loop runs over the ranks of every child
// whose rows meet the tile (A = that child's U rows, other rows read
// zeros; B = the child's columns of Z), so U z is added at MFMA rate
// before y is rounded to bf16 and stored.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "internal.h"

namespace wl {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 64;         // k per stage
constexpr int kRowBytes = 128;  // kBK bf16 per LDS row
constexpr int kMinSliceSteps = 4;
// A 64-k step of any tile costs at least this (in units of a 256 x 128 step
// at full streaming rate): with few workgroups per CU a step waits out the
// memory latency of its loads rather than the stream rate.
constexpr double kStepFloor = 0.55;
// Cost (same units) of the extra launch that sums split-K partials.
constexpr double kSplitLaunch = 4.0;
constexpr int kMaxSplit = 16;
constexpr int kCUs = 256;

// LDS-DMA stage loads.  They are buffer loads into LDS (buffer_load_dwordx4
// ... lds), not global_load_lds: with the latter in flight the compiler
// drains every outstanding LDS read (s_waitcnt lgkmcnt(0)) before each use of
// a fragment, with the former it counts them (lgkmcnt(n)), so fragment reads
// stay in flight under the MFMAs (same results; the 31B prefill GEMMs ran
// 2-7% faster).  One load instruction of a wave (8 rows x 128 bytes) reads
// through one descriptor whose base is its first live lane's address less
// 128 bytes; each lane adds a 32-bit byte offset.  The rows of one
// instruction ascend with the lane (every caller maps lane >> 3 to
// consecutive rows of one operand), so every live offset is positive and
// small.  A lane without a row takes an offset past the descriptor's range,
// which the buffer unit returns as zeros.
constexpr int kBufWord3 = 0x00020000;          // raw gfx9 descriptor: no swizzle, stride 0
constexpr int kBufRange = 0x40000000;          // bytes the offsets are checked against
constexpr uint32_t kBufNoRow = 0x7ffffff0u;    // past the range: reads zeros

struct RowLoad {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off;  // this lane's byte offset (kBufNoRow: no row)
};

// p: this lane's source address, or null for no row; fallback: any valid
// address, the base when no lane of the wave has a row.
__device__ __forceinline__ RowLoad row_load(const uint16_t *p, const uint16_t *fallback) {
  const uint64_t live = __builtin_amdgcn_ballot_w64(p != nullptr);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(p);
  uintptr_t base = reinterpret_cast<uintptr_t>(fallback);
  if (live) {
    const int first = __builtin_ctzll(live);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(addr), first);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(addr >> 32), first);
    base = ((static_cast<uintptr_t>(hi) << 32) | lo) - kRowBytes;
  }
  return RowLoad{__builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, kBufRange, kBufWord3),
                 p != nullptr ? static_cast<uint32_t>(addr - base) : kBufNoRow};
}

__device__ __forceinline__ void load_rows(const RowLoad &r, uint32_t off, uint8_t *dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rsrc, (lds_void *)dst, 16, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

enum Mode : int32_t {
  kStoreBf16 = 0,  // Y = bf16(acc), [T][ldy]
  kFused = 1,      // Y = child map of bf16(s (.) acc + Z U^T)
  kPartial = 2,    // P[slice][T][M] = acc (fp32); the last slice also writes P[ksplit] = Z U^T (if nchild)
  kAddScaled = 3,  // Y = bf16(acc + s[t] * W[t][m]), [T][ldy] (effective-weight materialization)
  kFusedAct = 4,   // paired gate|up rows: H = bf16(act(s (.) gate + dg) * (s (.) up + du)), [T][ldh]
};

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
  int32_t nM, nT, ksplit, steps_per_slice;
  // epilogue
  int32_t mode;
  uint16_t *Y;
  int32_t ldy;
  const float *s;
  const uint16_t *Z;  // [T][ldz]
  int32_t ldz;
  float *P;           // partials [ksplit (+1 for the delta)][T][M]
  const uint16_t *W;  // kAddScaled: [T][ldw] bf16, scaled by s[t] and added
  int64_t ldw;
  int32_t pair;       // > 0: rows are paired gate|up with this many gate rows
  int32_t act;        // kFusedAct: activation code
  uint16_t *H;        // kFusedAct: [T][ldh] bf16
  int32_t ldh;
  int32_t nchild;
  ChildDesc ch[kMaxChildren];
  // fused thin reduction (gemm_fz_kernel): V^T rows [rz][ldv] of the call
  const uint16_t *Vt;
  int64_t ldv;
  int32_t rz;
};

// RZ > 0 (fused thin reduction): every stage also holds RZ rows of V^T
// after the BM weight rows, and the waves accumulate Z = X V for the tile's
// tokens beside the main product (FZ 16-rank fragments per wave).
template <int BM, int BN, int WM, int WN, int NST, int RZ = 0>
struct Tile {
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int AR = BM + RZ;               // A rows of a stage
  static constexpr int FZ = RZ / 16 / WM;          // Z fragments per wave
  static constexpr int GA = AR / 8, GB = BN / 8;  // 8-row load groups
  static constexpr int LPW = (GA + GB) / NW;      // LDS-DMA instructions per wave per stage
  static constexpr int STAGE = (AR + BN) * kRowBytes;
  static constexpr size_t LDS = static_cast<size_t>(NST) * STAGE;
  static_assert((GA + GB) % NW == 0, "8-row groups must split evenly over the waves");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tiles are whole MFMA blocks");
  static_assert(RZ % (16 * WM) == 0, "the Z rows split evenly over the wave rows");
};

// One staged GEMM segment: acc += A B^T over 64-k steps [s_begin, s_end).
// Row pointers are per load instruction (already offset to the lane's chunk);
// a null row pointer reads zeros.  klen bounds the valid k (chunks at or past
// klen read zeros).  With RZ > 0 the A rows BM .. BM+RZ-1 are
// V^T rows whose products go to zacc.
template <int BM, int BN, int WM, int WN, int NST, int RZ>
__device__ __forceinline__ void segment_rz(f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                           f32x4 (&zacc)[RZ ? RZ / 16 / WM : 1][BN / WN / 16],
                                           const uint16_t *const (&rp)[(BM + RZ + BN) / 8 / (WM * WN)], int klen,
                                           int s_begin, int s_end, const uint16_t *zero_row, uint8_t *lds) {
  using TL = Tile<BM, BN, WM, WN, NST, RZ>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lchunk = (lane & 7) ^ ((lane >> 3) & 7);
  const int nk = s_end - s_begin;
  int ldsoff[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    const int gq = wave * TL::LPW + q;
    ldsoff[q] = gq < TL::GA ? gq * 1024 : TL::AR * kRowBytes + (gq - TL::GA) * 1024;
  }
  // Running source offsets, one per load instruction, advanced by one stage
  // per issue (stages are issued in order); a lane without a row reads zeros
  // and never advances.  Only a last step that reaches past klen (K not a
  // multiple of 64) needs the per-chunk bound.
  RowLoad src[TL::LPW];
  uint32_t inc[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    src[q] = row_load(rp[q] != nullptr ? rp[q] + s_begin * kBK : nullptr, zero_row);
    inc[q] = rp[q] != nullptr ? kRowBytes : 0;
  }
  const int full_steps = klen / kBK;
  // loads q0 .. q1-1 of a stage
  auto issue_part = [&](int stage, int step, int q0, int q1) {
    const bool tail = step >= full_steps;
    const int k = step * kBK + lchunk * 8;
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      if (q < q0 || q >= q1) continue;
      load_rows(src[q], (tail && k >= klen) ? kBufNoRow : src[q].off, lds + stage * TL::STAGE + ldsoff[q]);
      src[q].off += inc[q];
    }
  };
  auto issue = [&](int stage, int step) { issue_part(stage, step, 0, TL::LPW); };
  const int arow = (wm * TL::TM + r16) * kRowBytes;
  const int zrow = (BM + wm * TL::FZ * 16 + r16) * kRowBytes;
  const int brow = TL::AR * kRowBytes + (wn * TL::TN + r16) * kRowBytes;
  const int sw0 = ((0 + g) ^ (r16 & 7)) * 16, sw1 = ((4 + g) ^ (r16 & 7)) * 16;
  (void)zrow;

#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nk) issue(st, s_begin + st);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done once at most NST-2 stages of
    // loads remain outstanding; the barrier then makes every wave's part of
    // the stage visible, and tells that stage kt-1 is no longer being read
    if (kt + NST - 2 < nk)
      wait_vmcnt<(NST - 2) * TL::LPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // the next stage's loads go out in two halves, before and between the
    // two 32-k halves of this stage's MFMAs, so they interleave with the
    // matrix work rather than queue up at once
    const bool more = kt + NST - 1 < nk;
    const int nstage = (kt + NST - 1) % NST, nstep = s_begin + kt + NST - 1;
    if (more) issue_part(nstage, nstep, 0, TL::LPW / 2);
    const uint8_t *sb = lds + (kt % NST) * TL::STAGE;
    // both halves' fragments are read up front (registers allow it: at most
    // two waves per SIMD), so the LDS latency is paid once per stage
    u32x4 fa[2][TL::FM], fb[2][TL::FN], fz[2][TL::FZ ? TL::FZ : 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sw = h ? sw1 : sw0;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
        fa[h][i] = *reinterpret_cast<const u32x4 *>(sb + arow + i * 16 * kRowBytes + sw);
#pragma unroll
      for (int i = 0; i < TL::FZ; ++i)
        fz[h][i] = *reinterpret_cast<const u32x4 *>(sb + zrow + i * 16 * kRowBytes + sw);
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
        fb[h][j] = *reinterpret_cast<const u32x4 *>(sb + brow + j * 16 * kRowBytes + sw);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = mfma16x16x32(fa[h][i], fb[h][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < TL::FZ; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) zacc[i][j] = mfma16x16x32(fz[h][i], fb[h][j], zacc[i][j]);
      if (h == 0 && more) issue_part(nstage, nstep, TL::LPW / 2, TL::LPW);
    }
  }
  // every wave is done with the ring before it is refilled
  __builtin_amdgcn_s_barrier();
}

template <int BM, int BN, int WM, int WN, int NST>
__device__ __forceinline__ void segment(f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                        const uint16_t *const (&rp)[(BM + BN) / 8 / (WM * WN)], int klen,
                                        int s_begin, int s_end, const uint16_t *zero_row, uint8_t *lds) {
  f32x4 none[1][BN / WN / 16];
  segment_rz<BM, BN, WM, WN, NST, 0>(acc, none, rp, klen, s_begin, s_end, zero_row, lds);
}

// The two deltas of a paired gate|up tile in one pass.  Tile rows v < BM/2
// are gate rows (A = U_gate rows, B = the Z_gate columns) and v >= BM/2 the
// matching up rows (U_up, Z_up); a stage holds both B blocks, so every wave
// multiplies only its own child's rows, where two separate segments would
// each run half the tile on zero rows.  Two 64-k stages of BM + 2 BN rows in
// the ring (which has room for them for every tile shape).  Rank steps past
// a child's padded rank read zeros.
template <int BM, int BN, int WM, int WN, int NST>
__device__ __forceinline__ void paired_delta(f32x4 (&acc)[BM / WM / 16][BN / WN / 16], const GemmArgs &a, int f,
                                             int n0, uint8_t *lds) {
  using TL = Tile<BM, BN, WM, WN, NST>;
  constexpr int HB = BM / 2;
  constexpr int GA = BM / 8, GB2 = 2 * BN / 8;  // 8-row load groups: A, then both B blocks
  constexpr int LPW2 = (GA + GB2) / TL::NW;
  constexpr int STAGE2 = (BM + 2 * BN) * kRowBytes;
  static_assert((GA + GB2) % TL::NW == 0, "8-row groups must split evenly over the waves");
  static_assert(2 * STAGE2 <= TL::LDS, "two paired-delta stages must fit the ring");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lrow & 7);
  const ChildDesc &cg = a.ch[0], &cu = a.ch[1];
  const int nsteps = (max(cg.rpad, cu.rpad) + kBK - 1) / kBK;
  const uint16_t *rp[LPW2];
  int klen[LPW2], ldsoff[LPW2];
  RowLoad src[LPW2];
#pragma unroll
  for (int q = 0; q < LPW2; ++q) {
    const int gq = wave * LPW2 + q;
    if (gq < GA) {
      const int v = gq * 8 + lrow;
      const bool up = v >= HB;
      const ChildDesc &ch = up ? cu : cg;
      const int j = f * HB + (v & (HB - 1));
      rp[q] = j < a.pair ? ch.U + static_cast<int64_t>(j) * ch.rpad + lchunk * 8 : nullptr;
      klen[q] = ch.rpad;
      ldsoff[q] = gq * 1024;
    } else {
      const int gb = gq - GA, up = gb >= BN / 8;
      const ChildDesc &ch = up ? cu : cg;
      const int row = n0 + (gb - (up ? BN / 8 : 0)) * 8 + lrow;
      rp[q] = row < a.T ? a.Z + static_cast<int64_t>(row) * a.ldz + ch.zoff + lchunk * 8 : nullptr;
      klen[q] = ch.rpad;
      ldsoff[q] = BM * kRowBytes + gb * 1024;
    }
  }
#pragma unroll
  for (int q = 0; q < LPW2; ++q) src[q] = row_load(rp[q], a.zero_row);
  auto issue = [&](int stage, int step) __attribute__((always_inline)) {
    const int k = step * kBK + lchunk * 8;
#pragma unroll
    for (int q = 0; q < LPW2; ++q)
      load_rows(src[q], (rp[q] != nullptr && k < klen[q]) ? src[q].off + step * kRowBytes : kBufNoRow,
                lds + stage * STAGE2 + ldsoff[q]);
  };
  const int arow = (wm * TL::TM + r16) * kRowBytes;
  const int region = wm * TL::TM < HB ? 0 : 1;  // gate waves read Z_gate, up waves Z_up
  const int brow = (BM + region * BN + wn * TL::TN + r16) * kRowBytes;
  const int sw0 = ((0 + g) ^ (r16 & 7)) * 16, sw1 = ((4 + g) ^ (r16 & 7)) * 16;
  if (nsteps > 0) issue(0, 0);
  for (int kt = 0; kt < nsteps; ++kt) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // stage kt visible; stage kt-1 no longer read
    if (kt + 1 < nsteps) issue((kt + 1) & 1, kt + 1);
    const uint8_t *sb = lds + (kt & 1) * STAGE2;
    u32x4 fa[2][TL::FM], fb[2][TL::FN];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sw = h ? sw1 : sw0;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
        fa[h][i] = *reinterpret_cast<const u32x4 *>(sb + arow + i * 16 * kRowBytes + sw);
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
        fb[h][j] = *reinterpret_cast<const u32x4 *>(sb + brow + j * 16 * kRowBytes + sw);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = mfma16x16x32(fa[h][i], fb[h][j], acc[i][j]);
  }
  // every wave is done with the ring before it is refilled
  __builtin_amdgcn_s_barrier();
}

// Workgroup index -> (feature tile, K slice, token tile), XCD-major: hardware
// sends workgroup w to XCD w % 8; XCD x is given the contiguous unit range
// [x * per + min(x, rem), ...) of the total units, token tile fastest.
__device__ __forceinline__ void unit_of(int id, int total, int nT, int nslices, int &f, int &sl, int &t) {
  const int x = id & 7, j = id >> 3;
  const int per = total >> 3, rem = total & 7;
  const int u = x * per + min(x, rem) + j;
  f = u / (nslices * nT);
  const int r = u % (nslices * nT);
  sl = r / nT;
  t = r % nT;
}

// fp32 partial of a tile (rows of the operand only) at P [T][M]: lane holds
// tile rows v = wm*TM + 16i + 4g + e, token n0 + wn*TN + 16j + r16, mapped to
// operand rows as in the kernel (plain or gate|up paired).
template <int BM, int BN, int WM, int WN, int NST>
__device__ __forceinline__ void store_partial_tile(const f32x4 (&acc)[BM / WM / 16][BN / WN / 16], float *P,
                                                   const GemmArgs &a, int f, int n0) {
  using TL = Tile<BM, BN, WM, WN, NST>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN, r16 = lane & 15, g = lane >> 4;
  constexpr int HB = BM / 2;
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) {
    const int tok = n0 + wn * TL::TN + j * 16 + r16;
    if (tok >= a.T) continue;
    float *prow = P + static_cast<size_t>(tok) * a.M;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int v = wm * TL::TM + i * 16 + g * 4;
      const int row = a.pair ? (v >= HB ? a.pair : 0) + f * HB + (v & (HB - 1)) : f * BM + v;
      const int lim = a.pair ? a.pair - (f * HB + (v & (HB - 1))) : a.M - (f * BM + v);
      const int nv = max(0, min(4, lim));
      if (nv == 4 && ((a.M | row) & 3) == 0) {
        *reinterpret_cast<f32x4 *>(prow + row) = acc[i][j];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) prow[row + e] = acc[i][j][e];
      }
    }
  }
}

// Store a fused (non-paired) tile: rows f*BM + v, y through the child map
// (its K=V copy too), staged through LDS.  Each lane's four bf16 (features
// 4g.., one token) go to a token-major tile in LDS, then the workgroup writes
// whole 16-byte chunks of token rows (8 consecutive features), so a store
// instruction covers full 128-byte lines of y rather than 32-byte pieces of
// 16 rows (the Gemma-3 gate call's store phase 5.7 -> 3.5 us, same bits).  A chunk whose 8 features do not lie in one child, or whose
// address is not 16-byte aligned, or that crosses M, goes out element by
// element.  lds: >= BN * (2 BM + 16) bytes, free of other use.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void store_fused_tile_staged(const f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                                        const GemmArgs &a, int f, int n0, uint8_t *lds) {
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int PITCH = 2 * BM + 16;  // bytes per token row in LDS (16-byte pad against bank conflicts)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN, r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int tl = wn * TN + j * 16 + r16, fl = wm * TM + i * 16 + g * 4;
      *reinterpret_cast<uint2 *>(lds + tl * PITCH + fl * 2) =
          make_uint2(f32_to_bf16(acc[i][j][0]) | (static_cast<uint32_t>(f32_to_bf16(acc[i][j][1])) << 16),
                     f32_to_bf16(acc[i][j][2]) | (static_cast<uint32_t>(f32_to_bf16(acc[i][j][3])) << 16));
    }
  __syncthreads();
  constexpr int CPR = BM / 8;  // 16-byte chunks per token row
  for (int c = threadIdx.x; c < BN * CPR; c += WM * WN * 64) {
    const int tl = c / CPR, fl = (c % CPR) * 8;
    const int tok = n0 + tl, row = f * BM + fl;
    if (tok >= a.T || row >= a.M) continue;
    const uint4 v = *reinterpret_cast<const uint4 *>(lds + tl * PITCH + fl * 2);
    uint16_t *yrow = a.Y + static_cast<int64_t>(tok) * a.ldy;
    int ci = 0;
    while (ci + 1 < a.nchild && row >= a.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = a.ch[ci];
    const int jj = row - ch.row_start;
    uint16_t *p0 = yrow + ch.y_off + jj, *p1 = ch.dup_off >= 0 ? yrow + ch.dup_off + jj : p0;
    if (row + 8 <= a.M && jj + 8 <= ch.N &&
        ((reinterpret_cast<uintptr_t>(p0) | reinterpret_cast<uintptr_t>(p1)) & 15) == 0) {
      *reinterpret_cast<uint4 *>(p0) = v;
      if (ch.dup_off >= 0) *reinterpret_cast<uint4 *>(p1) = v;
    } else {
      const uint16_t *o = reinterpret_cast<const uint16_t *>(&v);
      for (int e = 0; e < 8 && row + e < a.M; ++e) {
        const int r = row + e;
        int cj = ci;
        while (cj + 1 < a.nchild && r >= a.ch[cj + 1].row_start) ++cj;
        const ChildDesc &c2 = a.ch[cj];
        const int j2 = r - c2.row_start;
        yrow[c2.y_off + j2] = o[e];
        if (c2.dup_off >= 0) yrow[c2.dup_off + j2] = o[e];
      }
    }
  }
}

// At most two waves per SIMD (the LDS ring allows one workgroup per CU for
// the big tiles), so the compiler may use up to 256 VGPRs per lane.
// PAIRED: the instantiation for paired gate|up calls (rows of a tile split
// between the two children), which runs both deltas in one pass; the
// others never contain that code, so their register allocation is their own.
template <int BM, int BN, int WM, int WN, int NST, bool PAIRED>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(GemmArgs a) {
  using TL = Tile<BM, BN, WM, WN, NST>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lrow & 7);
  // units: the K slices of every tile (XCD-major); on a split GEMM the last
  // slice of a tile also computes the delta, so its K range is shorter by
  // the delta's steps and every unit has about the same work
  int f, sl, t;
  const int nslices = a.mode == kPartial ? a.ksplit : 1;
  unit_of(blockIdx.x, a.nM * a.nT * nslices, a.nT, nslices, f, sl, t);
  const int n0 = t * BN;
  // Tile rows.  Plain: rows f*BM + v.  Paired (gate|up with the activation
  // fused): v < BM/2 is gate row f*BM/2 + v and v >= BM/2 is up row
  // pair + f*BM/2 + v - BM/2, so gate and up of one output column meet in
  // one tile.  valid() counts rows of the operand; 4-row groups never
  // straddle the two halves.
  constexpr int HB = BM / 2;
  auto actual = [&](int v) -> int {
    return a.pair ? (v >= HB ? a.pair : 0) + f * HB + (v & (HB - 1)) : f * BM + v;
  };
  auto nvalid = [&](int v, int n) -> int {  // how many of rows v..v+n-1 exist
    const int lim = a.pair ? a.pair - (f * HB + (v & (HB - 1))) : a.M - (f * BM + v);
    return max(0, min(n, lim));
  };

  f32x4 acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    // main segment (this workgroup's K slice): rows of A (features) then of B (tokens)
    const uint16_t *rp[TL::LPW];
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      const int gq = wave * TL::LPW + q;
      if (gq < TL::GA) {
        const int v = gq * 8 + lrow;
        rp[q] = nvalid(v, 1) ? a.A + actual(v) * a.lda + lchunk * 8 : nullptr;
      } else {
        const int row = n0 + (gq - TL::GA) * 8 + lrow;
        rp[q] = row < a.T ? a.B + row * a.ldb + lchunk * 8 : nullptr;
      }
    }
    const int nsteps = (a.K + kBK - 1) / kBK;
    const int sb = min(nsteps, sl * a.steps_per_slice), se = min(nsteps, sb + a.steps_per_slice);
    segment<BM, BN, WM, WN, NST>(acc, rp, a.K, sb, se, a.zero_row, lds);
  }

  // A split GEMM's unit stores its fp32 partial; the last slice of a tile
  // then computes the delta into a zeroed accumulator and stores it as
  // partial ksplit.
  const bool delta_slice = a.mode == kPartial && sl == a.ksplit - 1 && a.nchild > 0;
  if (a.mode == kPartial) {
    store_partial_tile<BM, BN, WM, WN, NST>(acc, a.P + static_cast<size_t>(sl) * a.T * a.M, a, f, n0);
    if (!delta_slice) return;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const bool fused = a.mode == kFused || a.mode == kFusedAct;
  if (fused) {
    // scale by s (rows outside the operand are never stored)
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int v = wm * TL::TM + i * 16 + g * 4;
      const int nv = nvalid(v, 4), row = actual(v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sc = e < nv ? a.s[row + e] : 0.f;
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j][e] *= sc;
      }
    }
  }
  if (PAIRED && (fused || delta_slice)) {
    // paired gate|up tile: both deltas in one pass
    if constexpr (PAIRED) paired_delta<BM, BN, WM, WN, NST>(acc, a, f, n0, lds);
  } else if (fused || delta_slice) {
    // delta = Z U^T for every child with rows in this tile
    for (int ci = 0; ci < a.nchild; ++ci) {
      const ChildDesc &ch = a.ch[ci];
      if (ch.rpad == 0) continue;
      if (!a.pair && (f * BM >= ch.row_start + ch.N || f * BM + BM <= ch.row_start)) continue;
      const uint16_t *rp[TL::LPW];
#pragma unroll
      for (int q = 0; q < TL::LPW; ++q) {
        const int gq = wave * TL::LPW + q;
        if (gq < TL::GA) {
          const int v = gq * 8 + lrow;
          const int row = actual(v);
          const bool in = nvalid(v, 1) && row >= ch.row_start && row < ch.row_start + ch.N;
          rp[q] = in ? ch.U + static_cast<int64_t>(row - ch.row_start) * ch.rpad + lchunk * 8 : nullptr;
        } else {
          const int row = n0 + (gq - TL::GA) * 8 + lrow;
          rp[q] = row < a.T ? a.Z + static_cast<int64_t>(row) * a.ldz + ch.zoff + lchunk * 8 : nullptr;
        }
      }
      segment<BM, BN, WM, WN, NST>(acc, rp, ch.rpad, 0, (ch.rpad + kBK - 1) / kBK, a.zero_row, lds);
    }
  }

  if (delta_slice) {
    store_partial_tile<BM, BN, WM, WN, NST>(acc, a.P + static_cast<size_t>(a.ksplit) * a.T * a.M, a, f, n0);
    return;
  }

  if (a.mode == kFusedAct) {
    // the up half's waves hand their values to the gate half's waves (same
    // lane, same i and j) through LDS, which the K loop no longer uses
    f32x4 *xch = reinterpret_cast<f32x4 *>(lds);
    const bool up_half = wm >= WM / 2;
    const int pw = (wm % (WM / 2)) * WN + wn;
    if (up_half) {
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) xch[((pw * TL::FM + i) * TL::FN + j) * 64 + lane] = acc[i][j];
    }
    __syncthreads();
    if (up_half) return;
    // h = act(gate) * up into a token-major tile after the exchange area,
    // then whole 16-byte chunks of H rows (as the fused y store)
    constexpr int XCH = (WM / 2) * WN * TL::FM * TL::FN * 64 * static_cast<int>(sizeof(f32x4));
    constexpr int HPITCH = 2 * HB + 16;  // bytes per token row (16-byte pad against bank conflicts)
    static_assert(XCH + BN * HPITCH <= static_cast<int>(TL::LDS), "exchange and h tile fit the ring");
    uint8_t *ht = lds + XCH;
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        const f32x4 u = xch[((pw * TL::FM + i) * TL::FN + j) * 64 + lane];
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(activation(a.act, acc[i][j][e]) * u[e]);
        // tile row: token; column: gate row v = wm TM + 16 i + 4 g (< BM/2)
        *reinterpret_cast<uint2 *>(ht + (wn * TL::TN + j * 16 + r16) * HPITCH + (wm * TL::TM + i * 16 + g * 4) * 2) =
            make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      }
    __syncthreads();  // the gate half's waves only: the up half has left
    constexpr int CPR = HB / 8;                    // 16-byte chunks per token row
    constexpr int NTHR = (WM / 2) * WN * 64;       // the gate half's threads, 0 .. NTHR-1
    for (int c = threadIdx.x; c < BN * CPR; c += NTHR) {
      const int tl = c / CPR, v = (c % CPR) * 8;
      const int tok = n0 + tl;
      const int nv = nvalid(v, 8), jj = actual(v);
      if (tok >= a.T || nv == 0) continue;
      const uint4 x = *reinterpret_cast<const uint4 *>(ht + tl * HPITCH + v * 2);
      uint16_t *hrow = a.H + static_cast<int64_t>(tok) * a.ldh;
      if (nv == 8 && (reinterpret_cast<uintptr_t>(hrow + jj) & 15) == 0) {
        *reinterpret_cast<uint4 *>(hrow + jj) = x;
      } else {
        const uint16_t *o = reinterpret_cast<const uint16_t *>(&x);
        for (int e = 0; e < nv; ++e) hrow[jj + e] = o[e];
      }
    }
    return;
  }

  if (a.mode == kFused && !a.pair) {
    // the ring is idle (every segment ends on a barrier)
    static_assert(BN * (2 * BM + 16) <= TL::LDS, "the staged output tile fits the ring");
    store_fused_tile_staged<BM, BN, WM, WN>(acc, a, f, n0, lds);
    return;
  }
  // store: y through the child map (fused), or plain rows
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) {
    const int tok = n0 + wn * TL::TN + j * 16 + r16;
    if (tok >= a.T) continue;
    uint16_t *yrow = a.Y + static_cast<int64_t>(tok) * a.ldy;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int v = wm * TL::TM + i * 16 + g * 4;
      const int nv = nvalid(v, 4), row = actual(v);
      if (nv == 0) continue;
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(acc[i][j][e]);
      if (a.mode == kAddScaled) {
        // here the B rows ("tokens") are the rows of the weight and the A rows
        // its columns: y[t][m] = acc + s[t] * W[t][m]
        const float sc = a.s[tok];
        const uint16_t *wrow = a.W + static_cast<int64_t>(tok) * a.ldw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) o[e] = f32_to_bf16(acc[i][j][e] + sc * bf16_to_f32(wrow[row + e]));
      }
      if (a.mode == kStoreBf16 || a.mode == kAddScaled) {
        if (nv == 4 && (reinterpret_cast<uintptr_t>(yrow + row) & 7) == 0) {
          *reinterpret_cast<uint2 *>(yrow + row) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nv) yrow[row + e] = o[e];
        }
      } else {
        int ci = 0;
        while (ci + 1 < a.nchild && row >= a.ch[ci + 1].row_start) ++ci;
        const ChildDesc &ch = a.ch[ci];
        const int jj = row - ch.row_start;
        uint16_t *p0 = yrow + ch.y_off + jj, *p1 = ch.dup_off >= 0 ? yrow + ch.dup_off + jj : p0;
        if (nv == 4 && jj + 4 <= ch.N && ((reinterpret_cast<uintptr_t>(p0) | reinterpret_cast<uintptr_t>(p1)) & 7) == 0) {
          // the four rows are one child's: one 8-byte store (and its K=V copy)
          const uint2 pk = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                                      o[2] | (static_cast<uint32_t>(o[3]) << 16));
          *reinterpret_cast<uint2 *>(p0) = pk;
          if (ch.dup_off >= 0) *reinterpret_cast<uint2 *>(p1) = pk;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (e >= nv) break;
            const int r = row + e;
            int cj = ci;
            while (cj + 1 < a.nchild && r >= a.ch[cj + 1].row_start) ++cj;
            const ChildDesc &c2 = a.ch[cj];
            const int j2 = r - c2.row_start;
            yrow[c2.y_off + j2] = o[e];
            if (c2.dup_off >= 0) yrow[c2.dup_off + j2] = o[e];
          }
        }
      }
    }
  }
}

// One launch for a whole call with a small total rank (Rz <= RZ, RZ 64 or
// 128): the workgroup of a BM x BN tile also computes its tokens' Z = X V.
// Every stage of the main loop holds, after the BM rows of W0, the RZ rows
// of V^T (rows past Rz read zeros), so the X rows already staged for
// the main product serve the thin reduction too; the waves accumulate
// W0 x and V^T x side by side.  Then Z is rounded to bf16 (as between the
// two launches of the unfused path) into LDS, token-major with 16-byte
// chunk c of token t at slot c ^ (t % 8), the main accumulator is scaled by
// s, and each child's U rows (A, streamed 64 ranks per step; ranks past the
// child's padded rank read zeros) multiply its columns of Z (B, from
// LDS) into it before the bf16 store.  Each token tile's Z is recomputed by
// every feature tile of its column: RZ / BM more MFMA work, traded for the
// two launches (the Z product and its sum) it saves.
template <int BM, int BN, int WM, int WN, int NST, int RZ>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN > 8 ? WM * WN / 4 : 1, WM * WN > 8 ? WM * WN / 4 : 2))) void gemm_fz_kernel(GemmArgs a) {
  using TL = Tile<BM, BN, WM, WN, NST, RZ>;
  static_assert(RZ % 64 == 0, "Z rows are whole 64-rank blocks (the chunk swizzle stays inside a row)");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, g = lane >> 4;
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lrow & 7);
  int f, sl, t;
  unit_of(blockIdx.x, a.nM * a.nT, a.nT, 1, f, sl, t);
  const int n0 = t * BN;

  f32x4 acc[TL::FM][TL::FN], zacc[TL::FZ][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TL::FZ; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) zacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const uint16_t *rp[TL::LPW];
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      const int gq = wave * TL::LPW + q;
      if (gq < TL::GA) {
        const int v = gq * 8 + lrow;
        if (v < BM) {
          const int row = f * BM + v;
          rp[q] = row < a.M ? a.A + row * a.lda + lchunk * 8 : nullptr;
        } else {
          const int zr = v - BM;
          rp[q] = zr < a.rz ? a.Vt + zr * a.ldv + lchunk * 8 : nullptr;
        }
      } else {
        const int row = n0 + (gq - TL::GA) * 8 + lrow;
        rp[q] = row < a.T ? a.B + row * a.ldb + lchunk * 8 : nullptr;
      }
    }
    segment_rz<BM, BN, WM, WN, NST, RZ>(acc, zacc, rp, a.K, 0, (a.K + kBK - 1) / kBK, a.zero_row, lds);
  }
  // (the segment ends with a barrier: the ring is free)
  // Z tile -> LDS: lane holds ranks wm*FZ*16 + 16i + 4g .. +3 of token
  // wn*TN + 16j + r16
  constexpr int ZROW = RZ * 2;  // bytes per token row
#pragma unroll
  for (int i = 0; i < TL::FZ; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int rk = wm * TL::FZ * 16 + i * 16 + g * 4;
      const int tk = wn * TL::TN + j * 16 + r16;
      const int off = tk * ZROW + (((rk >> 3) ^ (tk & 7)) << 4) + (rk & 4) * 2;
      *reinterpret_cast<uint2 *>(lds + off) =
          make_uint2(f32_to_bf16(zacc[i][j][0]) | (static_cast<uint32_t>(f32_to_bf16(zacc[i][j][1])) << 16),
                     f32_to_bf16(zacc[i][j][2]) | (static_cast<uint32_t>(f32_to_bf16(zacc[i][j][3])) << 16));
    }
  // scale by s (rows outside the operand are never stored)
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) {
    const int v = f * BM + wm * TL::TM + i * 16 + g * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sc = v + e < a.M ? a.s[v + e] : 0.f;
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[i][j][e] *= sc;
    }
  }
  __syncthreads();
  // delta: U rows of each child meeting the tile, 64 ranks per step
  constexpr int ZBYTES = ((BN * ZROW + 1023) / 1024) * 1024;
  static_assert(ZBYTES + BM * kRowBytes <= TL::LDS, "Z tile and one U stage fit the ring");
  constexpr int GU = BM / 8, LPU = GU / TL::NW;
  static_assert(GU % TL::NW == 0, "U rows split evenly over the waves");
  uint8_t *ubuf = lds + ZBYTES;
  const int arow = (wm * TL::TM + r16) * kRowBytes;
  const int sw0 = ((0 + g) ^ (r16 & 7)) * 16, sw1 = ((4 + g) ^ (r16 & 7)) * 16;
  for (int ci = 0; ci < a.nchild; ++ci) {
    const ChildDesc &ch = a.ch[ci];
    if (ch.rpad == 0 || f * BM >= ch.row_start + ch.N || f * BM + BM <= ch.row_start) continue;
    RowLoad usrc[LPU];
#pragma unroll
    for (int q = 0; q < LPU; ++q) {
      const int row = f * BM + (wave * LPU + q) * 8 + lrow;
      const bool in = row < a.M && row >= ch.row_start && row < ch.row_start + ch.N;
      usrc[q] = row_load(in ? ch.U + static_cast<int64_t>(row - ch.row_start) * ch.rpad + lchunk * 8 : nullptr,
                         a.zero_row);
    }
    for (int st = 0; st * kBK < ch.rpad; ++st) {
#pragma unroll
      for (int q = 0; q < LPU; ++q) {
        const int k = st * kBK + lchunk * 8;
        load_rows(usrc[q], k < ch.rpad ? usrc[q].off + st * kRowBytes : kBufNoRow, ubuf + (wave * LPU + q) * 1024);
      }
      wait_vmcnt<0>();
      __syncthreads();
      u32x4 fa[2][TL::FM], fb[2][TL::FN];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sw = h ? sw1 : sw0;
#pragma unroll
        for (int i = 0; i < TL::FM; ++i)
          fa[h][i] = *reinterpret_cast<const u32x4 *>(ubuf + arow + i * 16 * kRowBytes + sw);
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) {
          const int tk = wn * TL::TN + j * 16 + r16;
          // ranks past Rz (the last child's step beyond its padded rank) meet
          // zero U columns; any chunk of the row serves as their operand
          const int cz = ((((ch.zoff + st * kBK + h * 32) >> 3) + g) & (RZ / 8 - 1));
          fb[h][j] = *reinterpret_cast<const u32x4 *>(lds + tk * ZROW + ((cz ^ (tk & 7)) << 4));
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TL::FM; ++i)
#pragma unroll
          for (int j = 0; j < TL::FN; ++j) acc[i][j] = mfma16x16x32(fa[h][i], fb[h][j], acc[i][j]);
      __syncthreads();  // every wave is done with ubuf before the next step refills it
    }
  }
  static_assert(BN * (2 * BM + 16) <= TL::LDS, "the staged output tile fits the ring");
  store_fused_tile_staged<BM, BN, WM, WN>(acc, a, f, n0, lds);
}

// Z[i] = bf16(sum over slices of P[slice][i]), slices in order; n is a
// multiple of 4 (T * Rz with Rz a multiple of 32).
__global__ void reduce_z_kernel(const float *P, int ksplit, size_t n, uint16_t *Z) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v = *reinterpret_cast<const f32x4 *>(P + i);
  for (int s = 1; s < ksplit; ++s) v += *reinterpret_cast<const f32x4 *>(P + static_cast<size_t>(s) * n + i);
  *reinterpret_cast<uint2 *>(Z + i) =
      make_uint2(f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                 f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
}

// y = bf16(s (.) sum_{slice < ksplit} P[slice] + P[ksplit] (the delta, if
// any)) for one (token, 4 rows) per thread, stored through the child map.
struct FinishArgs {
  const float *P;
  int32_t ksplit, has_delta, T, M;
  const float *s;
  uint16_t *Y;
  int32_t ldy;
  int32_t nchild;
  ChildDesc ch[kMaxChildren];
  int32_t act, pair;  // act >= 0: h = act(gate) * up into H, pair = gate rows
  uint16_t *H;
  int32_t ldh;
};

// One output value of the split path at row r, token tok:
// s_r sum_{slice < ksplit} P[slice][tok][r] + P[ksplit][tok][r] (the delta).
__device__ __forceinline__ float finished(const FinishArgs &a, int tok, int r) {
  const size_t plane = static_cast<size_t>(a.T) * a.M;
  const float *p = a.P + static_cast<size_t>(tok) * a.M + r;
  const float d = a.has_delta ? p[a.ksplit * plane] : 0.f;
  float acc = 0.f;
  for (int s0 = 0; s0 < a.ksplit; s0 += 4) {  // four loads in flight, summed in slice order
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = p[min(s0 + j, a.ksplit - 1) * plane];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < a.ksplit) acc += v[j];
  }
  return a.s[r] * acc + d;
}

// h[tok][j] = act(gate_j) * up_j for the paired gate|up call on the split path.
__global__ void finish_act_kernel(FinishArgs a) {
  const long id = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long>(a.pair) * a.T) return;
  const int tok = static_cast<int>(id / a.pair), j = static_cast<int>(id % a.pair);
  const float gv = finished(a, tok, j), uv = finished(a, tok, a.pair + j);
  a.H[static_cast<size_t>(tok) * a.ldh + j] = f32_to_bf16(activation(a.act, gv) * uv);
}

__global__ void finish_kernel(FinishArgs a) {
  const int groups = (a.M + 3) / 4;
  const long id = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long>(groups) * a.T) return;
  const int tok = static_cast<int>(id / groups), row = static_cast<int>(id % groups) * 4;
  const size_t plane = static_cast<size_t>(a.T) * a.M;
  const float *p = a.P + static_cast<size_t>(tok) * a.M + row;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
  // the 16-byte loads need s 16-byte aligned too: a single-family call's s
  // is a row slice of its group's s (q with a ragged N shifts k's)
  if (row + 3 < a.M && (a.M & 3) == 0 && (reinterpret_cast<uintptr_t>(a.s) & 15) == 0) {
    if (a.has_delta) d = *reinterpret_cast<const f32x4 *>(p + a.ksplit * plane);
    sc = *reinterpret_cast<const f32x4 *>(a.s + row);
    // four slices' loads in flight at a time (slices past the last re-read
    // it and are dropped); summed in slice order
    for (int s0 = 0; s0 < a.ksplit; s0 += 4) {
      f32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const f32x4 *>(p + min(s0 + j, a.ksplit - 1) * plane);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < a.ksplit) acc += v[j];
    }
  } else {
    for (int e = 0; e < 4 && row + e < a.M; ++e) {
      for (int s = 0; s < a.ksplit; ++s) acc[e] += p[s * plane + e];
      if (a.has_delta) d[e] = p[a.ksplit * plane + e];
      sc[e] = a.s[row + e];
    }
  }
  uint16_t *yrow = a.Y + static_cast<size_t>(tok) * a.ldy;
  {
    // four rows of one child with 8-byte aligned destinations: one store each
    int ci = 0;
    while (ci + 1 < a.nchild && row >= a.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = a.ch[ci];
    const int jj = row - ch.row_start;
    uint16_t *y0 = yrow + ch.y_off + jj;
    uint16_t *y1 = ch.dup_off >= 0 ? yrow + ch.dup_off + jj : y0;
    if (jj + 3 < ch.N && ((reinterpret_cast<uintptr_t>(y0) | reinterpret_cast<uintptr_t>(y1)) & 7) == 0) {
      u32x2 o;
      o[0] = f32_to_bf16(sc[0] * acc[0] + d[0]) | (static_cast<uint32_t>(f32_to_bf16(sc[1] * acc[1] + d[1])) << 16);
      o[1] = f32_to_bf16(sc[2] * acc[2] + d[2]) | (static_cast<uint32_t>(f32_to_bf16(sc[3] * acc[3] + d[3])) << 16);
      *reinterpret_cast<u32x2 *>(y0) = o;
      if (ch.dup_off >= 0) *reinterpret_cast<u32x2 *>(y1) = o;
      return;
    }
  }
  for (int e = 0; e < 4; ++e) {
    const int r = row + e;
    if (r >= a.M) break;
    int ci = 0;
    while (ci + 1 < a.nchild && r >= a.ch[ci + 1].row_start) ++ci;
    const ChildDesc &ch = a.ch[ci];
    const uint16_t o = f32_to_bf16(sc[e] * acc[e] + d[e]);
    const int jj = r - ch.row_start;
    yrow[ch.y_off + jj] = o;
    if (ch.dup_off >= 0) yrow[ch.dup_off + jj] = o;
  }
}

// Raise a kernel's dynamic-LDS limit to what its ring needs, once per kernel
// and device (the attribute belongs to the device the call runs on).
template <auto KERN>
hipError_t ensure_lds(size_t bytes) {
  static std::atomic<uint64_t> done{0};  // bit d: set on device d (d < 64)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(bytes));
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// The stage loads address 8 rows of an operand from one buffer descriptor:
// the offsets of a load instruction must stay inside its range over the
// whole K (8 row strides plus the row length, in bytes).  Far beyond any
// model shape; checked so that a larger stride fails rather than reads zeros.
bool buffer_offsets_fit(const GemmArgs &a) {
  int64_t ld = std::max<int64_t>({a.lda, a.ldb, a.ldz, a.ldv});
  int64_t len = a.K;
  for (int i = 0; i < a.nchild; ++i) {
    ld = std::max<int64_t>(ld, a.ch[i].rpad);
    len = std::max<int64_t>(len, a.ch[i].rpad);
  }
  return 2 * (8 * ld + len) + 2 * kRowBytes <= kBufRange;
}

template <int BM, int BN, int WM, int WN, int NST, bool PAIRED>
hipError_t launch_gemm_inst(const GemmArgs &a, hipStream_t stream) {
  using TL = Tile<BM, BN, WM, WN, NST>;
  if (!buffer_offsets_fit(a)) return hipErrorInvalidValue;
  auto kern = gemm_kernel<BM, BN, WM, WN, NST, PAIRED>;
  const hipError_t e = ensure_lds<gemm_kernel<BM, BN, WM, WN, NST, PAIRED>>(TL::LDS);
  if (e != hipSuccess) return e;
  const int units = a.nM * a.nT * (a.mode == kPartial ? a.ksplit : 1);
  hipLaunchKernelGGL(kern, dim3(units), dim3(WM * WN * 64), TL::LDS, stream, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NST>
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  return (a.pair && a.nchild == 2) ? launch_gemm_inst<BM, BN, WM, WN, NST, true>(a, stream)
                                   : launch_gemm_inst<BM, BN, WM, WN, NST, false>(a, stream);
}

// Tile shapes: BM features x BN tokens.  eff ranks the shapes by measured
// streaming efficiency (bigger tiles move fewer bytes per flop).  Every
// shape runs on at least eight waves (the fused-Z 128 x 64 tile at rank <=
// 64 on sixteen): the small tiles hold one workgroup per CU for their ring,
// and a step of the K loop (waits, barrier, load issue, fragment reads,
// MFMAs) ran 9-15% faster with more waves to interleave than with four.
struct TileCfg {
  int BM, BN;
  double eff;
};
constexpr TileCfg kTiles[] = {{256, 128, 1.0}, {128, 128, 0.75}, {128, 64, 0.5}, {64, 64, 0.3}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

struct Plan {
  int tile, ksplit, steps_per_slice, nM, nT;
  double cost;
};

// Choose the tile shape and the K split of one GEMM (M rows, K deep, T
// tokens, plus dsteps 64-k steps of rank-r delta per tile): minimise the
// estimated makespan -- rounds of workgroups over the CUs times the work of
// one workgroup, scaled by the tile's efficiency -- plus, when K is split, the
// cost of writing and re-reading the fp32 partials and of the finish launch.
// On a split GEMM the last slice of a tile also runs the delta: the slices
// split the K steps plus the delta steps evenly, the last one taking that
// many fewer K steps.  Unit: one 64-k step of a 256 x 128 tile (48 KB
// streamed per CU).
Plan plan_gemm(int M, int K, int T, int dsteps, bool allow_split = true) {
  const int nsteps = (K + kBK - 1) / kBK;
  Plan best{kNumTiles - 1, 1, nsteps, (M + 63) / 64, (T + 63) / 64, 1e300};
  double best_cost = 1e300;
  // smallest tile first: on equal cost (latency-bound small GEMMs) the tile
  // that wastes no rows wins
  for (int i = kNumTiles - 1; i >= 0; --i) {
    if (i != kNumTiles - 1 && kTiles[i].BM >= 2 * M) continue;  // at least half the rows would be empty
    const int nM = (M + kTiles[i].BM - 1) / kTiles[i].BM, nT = (T + kTiles[i].BN - 1) / kTiles[i].BN;
    const long tiles = static_cast<long>(nM) * nT;
    const double scale = std::max(kStepFloor, (kTiles[i].BM * kTiles[i].BN) / (256.0 * 128.0) / kTiles[i].eff);
    const int max_split = allow_split ? std::min(kMaxSplit, std::max(1, nsteps / kMinSliceSteps)) : 1;
    for (int ks = 1; ks <= max_split; ++ks) {
      const int work = ks == 1 ? nsteps : nsteps + dsteps;  // steps one tile's slices share
      const int per = (work + ks - 1) / ks;
      // every slice but the last takes per K steps; the last takes the rest
      // of K (possibly none) and the delta
      if (ks > 1) {
        const int last_k = nsteps - (ks - 1) * per;
        if (last_k < 0 || (last_k == 0 && dsteps == 0)) continue;  // a slice would be empty
      }
      const long rounds = (tiles * ks + kCUs - 1) / kCUs;
      double cost;
      if (ks == 1) {
        cost = static_cast<double>(rounds) * (per + dsteps) * scale;
      } else {
        cost = static_cast<double>(rounds) * per * scale;
        cost += 2.0 * (ks + (dsteps > 0 ? 1 : 0)) * static_cast<double>(T) * M * 4 / (kCUs * 48.0 * 1024) + kSplitLaunch;
      }
      if (cost < best_cost) {
        best_cost = cost;
        best = Plan{i, ks, per, nM, nT, cost};
      }
    }
  }
  return best;
}

int delta_steps(const CallDesc &c) {
  int r = 0;
  for (int i = 0; i < c.nchild; ++i) r = std::max(r, static_cast<int>(c.ch[i].rpad));
  return (r + kBK - 1) / kBK;
}

hipError_t launch_planned(GemmArgs a, const Plan &p, hipStream_t stream) {
  a.nM = p.nM;
  a.nT = p.nT;
  a.ksplit = p.ksplit;
  a.steps_per_slice = p.steps_per_slice;
  switch (p.tile) {
    case 0: return launch_gemm<256, 128, 4, 2, 3>(a, stream);
    case 1: return launch_gemm<128, 128, 4, 2, 4>(a, stream);
    case 2: return launch_gemm<128, 64, 4, 2, 4>(a, stream);
    default: return launch_gemm<64, 64, 4, 2, 4>(a, stream);
  }
}

// Fused thin reduction (gemm_fz_kernel): tile shapes, the stage depth each
// holds with RZ rows of V^T added, and their relative streaming efficiency.
// (A 256 x 128 tile has room for only two stages with the V^T rows added,
// spills registers, and measured slower than the unfused path on the
// Gemma-3 gate and up calls: 64 us against 56; it is not offered.)
constexpr TileCfg kFzTiles[] = {{128, 128, 0.75}, {128, 64, 0.5}, {64, 64, 0.3}};
constexpr int kNumFzTiles = sizeof(kFzTiles) / sizeof(kFzTiles[0]);
// Cost of one more dependent launch, in the planner's units (a 64-k step of
// a 256 x 128 tile): the unfused path's separate Z product.
constexpr double kLaunch = 6.0;
constexpr int kMaxFusedRank = 128;

// The fused plan of a call with Rz total padded ranks (RZ = 64 or 128 rows of
// V^T per stage): K unsplit; each step streams BM + RZ + BN rows instead of
// BM + BN, and the tile adds its delta steps.
Plan plan_fused_z(int M, int K, int T, int RZ, int dsteps) {
  const int nsteps = (K + kBK - 1) / kBK;
  Plan best{kNumFzTiles - 1, 1, nsteps, (M + 63) / 64, (T + 63) / 64, 1e300};
  for (int i = kNumFzTiles - 1; i >= 0; --i) {
    const TileCfg &tc = kFzTiles[i];
    if (i != kNumFzTiles - 1 && tc.BM >= 2 * M) continue;
    const int nM = (M + tc.BM - 1) / tc.BM, nT = (T + tc.BN - 1) / tc.BN;
    const long rounds = (static_cast<long>(nM) * nT + kCUs - 1) / kCUs;
    const double scale = std::max(kStepFloor, (tc.BM * tc.BN) / (256.0 * 128.0) / tc.eff);
    const double stream = static_cast<double>(tc.BM + RZ + tc.BN) / (tc.BM + tc.BN);
    const double cost = static_cast<double>(rounds) * (nsteps * stream + dsteps) * scale;
    if (cost < best.cost) best = Plan{i, 1, nsteps, nM, nT, cost};
  }
  return best;
}

template <int BM, int BN, int WM, int WN, int NST, int RZ>
hipError_t launch_fz_inst(const GemmArgs &a, hipStream_t stream) {
  using TL = Tile<BM, BN, WM, WN, NST, RZ>;
  if (!buffer_offsets_fit(a)) return hipErrorInvalidValue;
  auto kern = gemm_fz_kernel<BM, BN, WM, WN, NST, RZ>;
  const hipError_t e = ensure_lds<gemm_fz_kernel<BM, BN, WM, WN, NST, RZ>>(TL::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.nM * a.nT), dim3(WM * WN * 64), TL::LDS, stream, a);
  return hipGetLastError();
}

hipError_t launch_fused_z(GemmArgs a, const Plan &p, int RZ, hipStream_t stream) {
  a.nM = p.nM;
  a.nT = p.nT;
  a.ksplit = 1;
  a.steps_per_slice = p.steps_per_slice;
  const bool r64 = RZ == 64;
  switch (p.tile) {
    case 0:
      // With at least two tiles per CU, a two-stage ring (80 KB) lets two
      // workgroups share each CU, 16 waves instead of 8 (Gemma-3 gate / up
      // at T = 2048: 51 -> 39 us).  With fewer tiles the deeper ring of one
      // workgroup per CU is faster.
      if (r64 && static_cast<long>(p.nM) * p.nT >= 2L * kCUs) return launch_fz_inst<128, 128, 4, 2, 2, 64>(a, stream);
      return r64 ? launch_fz_inst<128, 128, 4, 2, 3, 64>(a, stream) : launch_fz_inst<128, 128, 4, 2, 3, 128>(a, stream);
    case 1: return r64 ? launch_fz_inst<128, 64, 4, 4, 4, 64>(a, stream) : launch_fz_inst<128, 64, 2, 4, 3, 128>(a, stream);
    default: return r64 ? launch_fz_inst<64, 64, 4, 2, 4, 64>(a, stream) : launch_fz_inst<64, 64, 4, 2, 4, 128>(a, stream);
  }
}

size_t partial_bytes(const Plan &p, int M, int T, bool delta) {
  return p.ksplit > 1 ? static_cast<size_t>(p.ksplit + (delta ? 1 : 0)) * T * M * 4 : 0;
}

}  // namespace

size_t prefill_partial_bytes(int Ntot, int Rz, int rmax, int K, int T) {
  const int dsteps = (rmax + kBK - 1) / kBK;
  size_t n = partial_bytes(plan_gemm(Ntot, K, T, dsteps), Ntot, T, dsteps > 0);
  if (Rz > 0) n = std::max(n, partial_bytes(plan_gemm(Rz, K, T, 0), Rz, T, false));
  return n;
}

hipError_t launch_prefill(const CallDesc &c, uint16_t *zbuf, float *pbuf, const uint16_t *zero_row,
                          hipStream_t stream, int act, uint16_t *h, int ldh) {
  hipError_t e;
  if (act < 0 && c.Rz > 0 && c.Rz <= kMaxFusedRank) {
    // small total rank: one launch that computes each tile's Z itself, where
    // the planner's estimate beats the separate Z product and its launches
    const int RZ = c.Rz <= 64 ? 64 : 128;
    const int dsteps = delta_steps(c);
    const Plan pf = plan_fused_z(c.Ntot, c.K, c.T, RZ, dsteps);
    const Plan pz = plan_gemm(c.Rz, c.K, c.T, 0);
    const Plan pm = plan_gemm(c.Ntot, c.K, c.T, dsteps);
    const double unfused = pz.cost + (pz.ksplit > 1 ? kSplitLaunch : 0.0) + pm.cost + kLaunch;
    if (pf.cost < unfused) {
      GemmArgs a{};
      a.A = c.W0;
      a.M = c.Ntot;
      a.lda = c.K;
      a.B = c.x;
      a.T = c.T;
      a.ldb = c.K;
      a.K = c.K;
      a.zero_row = zero_row;
      a.mode = kFused;
      a.Y = c.y;
      a.ldy = c.ldy;
      a.s = c.s;
      a.Vt = c.Vt;
      a.ldv = c.K;
      a.rz = c.Rz;
      a.nchild = c.nchild;
      for (int i = 0; i < c.nchild; ++i) a.ch[i] = c.ch[i];
      return launch_fused_z(a, pf, RZ, stream);
    }
  }
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
    a.Y = zbuf;
    a.ldy = c.Rz;
    a.P = pbuf;
    const Plan p = plan_gemm(c.Rz, c.K, c.T, 0);
    a.mode = p.ksplit > 1 ? kPartial : kStoreBf16;
    e = launch_planned(a, p, stream);
    if (e != hipSuccess) return e;
    if (p.ksplit > 1) {
      const size_t n = static_cast<size_t>(c.T) * c.Rz;
      const unsigned blocks = static_cast<unsigned>((n / 4 + 255) / 256);
      hipLaunchKernelGGL(reduce_z_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const float *>(pbuf),
                         p.ksplit, n, zbuf);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
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
  a.Y = c.y;
  a.ldy = c.ldy;
  a.s = c.s;
  a.Z = zbuf;
  a.ldz = c.Rz;
  a.P = pbuf;
  a.nchild = c.nchild;
  for (int i = 0; i < c.nchild; ++i) a.ch[i] = c.ch[i];
  Plan p = plan_gemm(c.Ntot, c.K, c.T, delta_steps(c));
  if (act >= 0) {
    // gate|up with the activation fused: tiles hold BM/2 gate rows and the
    // matching BM/2 up rows
    a.pair = c.ch[0].N;
    a.act = act;
    a.H = h;
    a.ldh = ldh;
    p.nM = (a.pair + kTiles[p.tile].BM / 2 - 1) / (kTiles[p.tile].BM / 2);
  }
  if (p.ksplit == 1) {
    a.mode = act >= 0 ? kFusedAct : kFused;
    return launch_planned(a, p, stream);
  }
  // K slices; the last slice of each tile also computes the delta (if any
  // child has a rank) into its own partial
  const bool any_rank = delta_steps(c) > 0;
  if (!any_rank) a.nchild = 0;
  a.mode = kPartial;
  e = launch_planned(a, p, stream);
  if (e != hipSuccess) return e;
  FinishArgs fa{};
  fa.P = pbuf;
  fa.ksplit = p.ksplit;
  fa.has_delta = any_rank ? 1 : 0;
  fa.T = c.T;
  fa.M = c.Ntot;
  fa.s = c.s;
  fa.Y = c.y;
  fa.ldy = c.ldy;
  fa.nchild = c.nchild;
  for (int i = 0; i < c.nchild; ++i) fa.ch[i] = c.ch[i];
  if (act >= 0) {
    fa.act = act;
    fa.pair = c.ch[0].N;
    fa.H = h;
    fa.ldh = ldh;
    const long threads = static_cast<long>(fa.pair) * c.T;
    hipLaunchKernelGGL(finish_act_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream,
                       fa);
    return hipGetLastError();
  }
  const long threads = static_cast<long>((c.Ntot + 3) / 4) * c.T;
  hipLaunchKernelGGL(finish_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, fa);
  return hipGetLastError();
}

hipError_t launch_materialize(const uint16_t *V, const uint16_t *U, int32_t N, int32_t K, int32_t rpad,
                              const float *s, const uint16_t *W0, uint16_t *out, const uint16_t *zero_row,
                              hipStream_t stream) {
  // out[i][j] = s[i] W0[i][j] + sum_k U[i][k] V[j][k]: A = V rows (the K
  // columns of W_eff), B = U rows (its N rows), reduction over the ranks
  GemmArgs a{};
  a.A = V;
  a.M = K;
  a.lda = rpad;
  a.B = U;
  a.T = N;
  a.ldb = rpad;
  a.K = rpad;
  a.zero_row = zero_row;
  a.mode = kAddScaled;
  a.Y = out;
  a.ldy = K;
  a.s = s;
  a.W = W0;
  a.ldw = K;
  return launch_planned(a, plan_gemm(K, rpad, N, 0, false), stream);
}

}  // namespace wl
