// Prefill-path kernels (T > 16 tokens): two bf16 MFMA GEMMs.
//
//   launch 1:  Z[T, Rz] = X[T, K] V          (bf16 out, the thin reduction)
//   launch 2:  Y[T, N]  = (X W0^T) (.) s + Z U^T   (scale and rank-r delta
//              fused into the epilogue of the shared-block GEMM; y is written
//              once, in bf16)
//
// The forward is the method's theta-bundle forward ("Add a new model
// architecture" page, introduction); the pages' GEMM formulation keeps bf16
// operands with fp32 accumulation ("Quality (Gemma 4 31B)" page, "Kernel
// optimizations > GEMM path"), as these kernels do.
//
// Both launches use one LDS-tiled kernel.  A workgroup owns a BM x BN tile of
// the output: BM rows of the weight matrix (W0 or V^T: "features", the MFMA
// A operand) by BN tokens (the B operand).  All operands are K-contiguous, so
// every global load is a 16-byte row chunk and every LDS fragment read is one
// 16-byte ds_read.  Tiles of A and B are staged through registers into a
// double-buffered LDS ring (rows padded by 16 bytes against bank conflicts).
// The epilogue of launch 2 scales the fp32 accumulators by s per feature row
// and then runs the same staged loop over the ranks of each child (A = U
// rows of that child, B = Z columns of that child), so the delta is computed
// on the MFMA at the GEMM's own rate before y is rounded and stored.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

constexpr int BM = 128;   // features per workgroup
constexpr int BN = 128;   // tokens per workgroup
constexpr int BK = 64;    // k per stage
constexpr int LDSW = BK + 8;  // padded LDS row, in bf16 elements (144 bytes)
constexpr int NTHR = 256;
// each thread stages BM*BK/8/NTHR = 4 vectors of A and 4 of B per stage
constexpr int VPT_A = BM * BK / 8 / NTHR;
constexpr int VPT_B = BN * BK / 8 / NTHR;

struct Operand {
  const uint16_t *ptr;  // element (row 0, col 0) of the operand matrix
  int64_t ld;           // row stride in elements
  int32_t row_lo, row_hi;  // valid rows [row_lo, row_hi) (others read as zero)
};

// Stage one BK-wide slice [k0, k0 + BK) of `rows` rows starting at row0 into
// registers; columns >= klen and rows outside [row_lo, row_hi) are zero.
template <int ROWS, int VPT>
__device__ __forceinline__ void stage_load(u32x4 (&v)[VPT], const Operand &op, int row0, int k0, int klen) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = t + i * NTHR;
    const int row = row0 + idx / (BK / 8);
    const int col = k0 + (idx % (BK / 8)) * 8;
    const bool ok = row >= op.row_lo && row < op.row_hi && col < klen;
    v[i] = ok ? ld16(op.ptr + static_cast<int64_t>(row) * op.ld + col) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int ROWS, int VPT>
__device__ __forceinline__ void stage_store(uint16_t *lds, const u32x4 (&v)[VPT]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = t + i * NTHR;
    const int row = idx / (BK / 8);
    const int col = (idx % (BK / 8)) * 8;
    *reinterpret_cast<u32x4 *>(lds + row * LDSW + col) = v[i];
  }
}

// acc[fm][fn] += A[rows of this wave] * B[tokens of this wave]^T over klen,
// A rows from a.row0.., B rows from b.row0.. (the tile origins).
__device__ __forceinline__ void gemm_segment(f32x4 (&acc)[4][4], const Operand &a, int arow0,
                                             const Operand &b, int brow0, int klen,
                                             uint16_t *ldsA, uint16_t *ldsB) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int nk = (klen + BK - 1) / BK;
  u32x4 va[VPT_A], vb[VPT_B];

  stage_load<BM, VPT_A>(va, a, arow0, 0, klen);
  stage_load<BN, VPT_B>(vb, b, brow0, 0, klen);
  stage_store<BM, VPT_A>(ldsA, va);
  stage_store<BN, VPT_B>(ldsB, vb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      stage_load<BM, VPT_A>(va, a, arow0, (kt + 1) * BK, klen);
      stage_load<BN, VPT_B>(vb, b, brow0, (kt + 1) * BK, klen);
    }
    const uint16_t *sA = ldsA + cur * BM * LDSW;
    const uint16_t *sB = ldsB + cur * BN * LDSW;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        fa[f] = *reinterpret_cast<const u32x4 *>(sA + (wm * 64 + f * 16 + r16) * LDSW + kk + g * 8);
        fb[f] = *reinterpret_cast<const u32x4 *>(sB + (wn * 64 + f * 16 + r16) * LDSW + kk + g * 8);
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = mfma16x16x32(fa[fm], fb[fn], acc[fm][fn]);
    }
    if (more) {
      stage_store<BM, VPT_A>(ldsA + (cur ^ 1) * BM * LDSW, va);
      stage_store<BN, VPT_B>(ldsB + (cur ^ 1) * BN * LDSW, vb);
    }
    __syncthreads();
  }
}

// EPI = false: plain bf16 store of the product (launch 1, Z = X V).
// EPI = true: scale by s, add the per-child rank-r delta, store y.
template <bool EPI>
__global__ __launch_bounds__(NTHR) void gemm_kernel(CallDesc c, const uint16_t *zbuf, int ldz) {
  __shared__ __attribute__((aligned(16))) uint16_t ldsA[2 * BM * LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t ldsB[2 * BN * LDSW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * BM;   // first feature row
  const int n0 = blockIdx.y * BN;   // first token

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const Operand A{c.W0, c.K, 0, c.Ntot};
  const Operand X{c.x, c.K, 0, c.T};
  gemm_segment(acc, A, m0, X, n0, c.K, ldsA, ldsB);

  if (EPI) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + fm * 16 + g * 4 + i;
        const float sc = row < c.Ntot ? c.s[row] : 0.f;
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) acc[fm][fn][i] *= sc;
      }
    for (int ci = 0; ci < c.nchild; ++ci) {
      const ChildDesc &ch = c.ch[ci];
      if (ch.rpad == 0 || m0 >= ch.row_start + ch.N || m0 + BM <= ch.row_start) continue;
      // U rows are indexed by feature row: element (row, k) at
      // U + (row - row_start) * rpad + k; rows outside the child are zero.
      const Operand Uop{ch.U - static_cast<int64_t>(ch.row_start) * ch.rpad, ch.rpad, ch.row_start,
                        ch.row_start + ch.N};
      const Operand Zop{zbuf + ch.zoff, ldz, 0, c.T};
      gemm_segment(acc, Uop, m0, Zop, n0, ch.rpad, ldsA, ldsB);
    }
  }

  // Store: this lane holds rows m0 + wm*64 + fm*16 + 4g + i, token n0 + wn*64 + fn*16 + r16.
#pragma unroll
  for (int fn = 0; fn < 4; ++fn) {
    const int tok = n0 + wn * 64 + fn * 16 + r16;
    if (tok >= c.T) continue;
    uint16_t *yrow = c.y + static_cast<int64_t>(tok) * c.ldy;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + fm * 16 + g * 4 + i;
        if (row >= c.Ntot) continue;
        const uint16_t out = f32_to_bf16(acc[fm][fn][i]);
        if (!EPI) {
          yrow[row] = out;
        } else {
          int ci = 0;
          while (ci + 1 < c.nchild && row >= c.ch[ci + 1].row_start) ++ci;
          const ChildDesc &ch = c.ch[ci];
          const int j = row - ch.row_start;
          yrow[ch.y_off + j] = out;
          if (ch.dup_off >= 0) yrow[ch.dup_off + j] = out;
        }
      }
  }
}

}  // namespace

hipError_t launch_prefill(const CallDesc &c, uint16_t *zbuf, hipStream_t stream) {
  const dim3 block(NTHR);
  if (c.Rz > 0) {
    CallDesc zc = c;
    zc.W0 = c.Vt;
    zc.Ntot = c.Rz;
    zc.s = nullptr;
    zc.y = zbuf;
    zc.ldy = c.Rz;
    zc.nchild = 1;
    zc.ch[0] = ChildDesc{nullptr, 0, c.Rz, 0, 0, 0, -1};
    const dim3 gz((c.Rz + BM - 1) / BM, (c.T + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_kernel<false>), gz, block, 0, stream, zc, nullptr, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((c.Ntot + BM - 1) / BM, (c.T + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<true>), grid, block, 0, stream, c, zbuf, c.Rz);
  return hipGetLastError();
}

}  // namespace wl
