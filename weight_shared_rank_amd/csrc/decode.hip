// Decode-path kernel (T <= 16 tokens): y = s (.) (W0 x) + U (V^T x) in ONE launch.
//
// The method's forward for a theta bundle ("Add a new model architecture"
// page, introduction) at decode batch sizes is a bandwidth-bound GEMV: every
// byte of W0 is read once and used for T multiply-adds.  The pages' B200
// custom op (page "Quality (Gemma 4 31B)", "Custom-op path") put one warp per
// output row and recomputed V^T x per block; here V^T x is computed once per
// call and handed to the epilogue through the workspace.
//
// Layout of the launch (one workgroup = one 16-row tile, W waves split K):
//   * workgroups [0, nz) own 16-row tiles of V^T and produce z = V^T x
//     (fp32, stored as a bf16 hi/lo pair so the epilogue can use the MFMA);
//     each publishes completion by a release increment of ctrl[ZReady];
//   * workgroups [nz, nz + nw) own 16-row tiles of W0.  Their K loop feeds
//     bf16 MFMAs with W0 rows as the A operand and up to 16 tokens of x as the
//     B operand (token columns >= T are zero), so T = 1 and T = 16 run the
//     same code; the K loop is pure streaming: 16-byte loads of W0 straight
//     to registers, four lanes covering 64 contiguous bytes of a row per
//     instruction.  The epilogue waits (acquire) until all nz z-tiles are
//     published, then adds U z with two more MFMAs per 32 ranks (z hi and z
//     lo parts, so z keeps ~16 bits) and scales by s, writing y once in bf16.
//   * Hardware dispatches a kernel's workgroups in increasing index order on
//     each XCD, so every z-tile is dispatched no later than any W0 tile that
//     waits for it, and z-tiles never wait: the wait always ends.  It is also
//     bounded (kSpinLimit sleeps); on timeout the workgroup sets a sticky bit
//     in ctrl[Error] and goes on.
//   * The last workgroup to finish (ctrl[Done] reaching the tile count)
//     resets ctrl[ZReady] and ctrl[Done] to zero, so the workspace is ready
//     for the next call, including replays of a captured graph.
#include "common.h"
#include "internal.h"

namespace wl {

namespace {

constexpr int kSpinLimit = 1 << 21;

template <int W, int UNROLL>
__global__ __launch_bounds__(W * 64) void decode_kernel(CallDesc c, DecodeWs ws, int nz, int ntiles) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bid = blockIdx.x;
  const bool ztile = bid < nz;
  const int row0 = (ztile ? bid : bid - nz) * 16;
  const uint16_t *mat = ztile ? c.Vt : c.W0;
  const int nrows = ztile ? c.Rz : c.Ntot;
  const int r16 = lane & 15;   // A row within the tile / B token column
  const int g = lane >> 4;     // k-slot group: k = 32*step + 8*g
  const int K = c.K;

  // Rows past the end read the tile's first row (always valid); their
  // results are never stored.  Token columns >= T are zero.
  const int arow_idx = (row0 + r16 < nrows) ? row0 + r16 : row0;
  const uint16_t *arow = mat + static_cast<size_t>(arow_idx) * K + g * 8;
  const bool tok_ok = r16 < c.T;
  const uint16_t *xrow = c.x + static_cast<size_t>(tok_ok ? r16 : 0) * K + g * 8;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = (K + 31) >> 5;
  const int nfull = K >> 5;
  const int nblocks = (nsteps + UNROLL - 1) / UNROLL;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int b = wave; b < nblocks; b += W) {
    const int s0 = b * UNROLL;
    u32x4 av[UNROLL], bv[UNROLL];
    if (s0 + UNROLL <= nfull) {
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) av[j] = ld16(arow + (s0 + j) * 32);
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) bv[j] = tok_ok ? ld16(xrow + (s0 + j) * 32) : zero4;
    } else {
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int k = (s0 + j) * 32 + g * 8;
        const bool kin = k < K;
        av[j] = kin ? ld16(arow + (s0 + j) * 32) : zero4;
        bv[j] = (kin && tok_ok) ? ld16(xrow + (s0 + j) * 32) : zero4;
      }
    }
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) acc = mfma16x16x32(av[j], bv[j], acc);
  }

  // Cross-wave reduction of the K split, in a fixed order (deterministic).
  __shared__ f32x4 red[W][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 tot = red[0][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) tot += red[w][lane];

  // This lane holds D[m = 4g + i][n = r16]: rows row0 + 4g + i, token r16.
  if (ztile) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = row0 + g * 4 + i;
      if (k < c.Rz) {
        const float v = tot[i];
        const uint16_t hi = f32_to_bf16(v);
        const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
        ws.zhi[r16 * ws.ldz + k] = hi;
        ws.zlo[r16 * ws.ldz + k] = lo;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) __hip_atomic_fetch_add(ws.ctrl + kCtrlZReady, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
    if (nz > 0) {
      int spins = 0;
      while (__hip_atomic_load(ws.ctrl + kCtrlZReady, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
             static_cast<uint32_t>(nz)) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          if (lane == 0) __hip_atomic_fetch_or(ws.ctrl + kCtrlError, kErrZWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // delta = U z for every child with rows in this tile.  A = U rows of the
      // child (rows of other children are zero), B = z columns of the child.
      const int arow_g = row0 + r16;
      const uint16_t *zh = ws.zhi + r16 * ws.ldz + g * 8;
      const uint16_t *zl = ws.zlo + r16 * ws.ldz + g * 8;
      for (int ci = 0; ci < c.nchild; ++ci) {
        const ChildDesc &ch = c.ch[ci];
        if (ch.rpad == 0 || row0 >= ch.row_start + ch.N || row0 + 16 <= ch.row_start) continue;
        const bool in_child = arow_g >= ch.row_start && arow_g < ch.row_start + ch.N;
        const uint16_t *urow = ch.U + static_cast<size_t>(in_child ? arow_g - ch.row_start : 0) * ch.rpad + g * 8;
        for (int kk = 0; kk < ch.rpad; kk += 32) {
          const bool kin = kk + g * 8 < ch.rpad;
          const u32x4 a = (kin && in_child) ? ld16(urow + kk) : zero4;
          const u32x4 bh = kin ? ld16(zh + ch.zoff + kk) : zero4;
          const u32x4 bl = kin ? ld16(zl + ch.zoff + kk) : zero4;
          dacc = mfma16x16x32(a, bh, dacc);
          dacc = mfma16x16x32(a, bl, dacc);
        }
      }
    }
    if (tok_ok) {
      uint16_t *yrow = c.y + static_cast<size_t>(r16) * c.ldy;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + g * 4 + i;
        if (row >= c.Ntot) continue;
        int ci = 0;
        while (ci + 1 < c.nchild && row >= c.ch[ci + 1].row_start) ++ci;
        const ChildDesc &ch = c.ch[ci];
        const uint16_t out = f32_to_bf16(c.s[row] * tot[i] + dacc[i]);
        const int j = row - ch.row_start;
        yrow[ch.y_off + j] = out;
        if (ch.dup_off >= 0) yrow[ch.dup_off + j] = out;
      }
    }
  }

  // Completion count; the last workgroup resets the synchronization words.
  if (lane == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ws.ctrl + kCtrlDone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == static_cast<uint32_t>(ntiles - 1)) {
      __hip_atomic_store(ws.ctrl + kCtrlZReady, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ws.ctrl + kCtrlDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_decode(const CallDesc &c, const DecodeWs &ws, hipStream_t stream) {
  constexpr int W = 4, UNROLL = 8;
  const int nz = (c.Rz + 15) / 16;
  const int nw = (c.Ntot + 15) / 16;
  const int ntiles = nz + nw;
  hipLaunchKernelGGL((decode_kernel<W, UNROLL>), dim3(ntiles), dim3(W * 64), 0, stream, c, ws, nz, ntiles);
  return hipGetLastError();
}

}  // namespace wl
