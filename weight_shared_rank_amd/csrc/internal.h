// Internal declarations shared by the host side of the library and its HIP
// kernels.  Not part of the public ABI (include/weightless.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wl {

// Decode path limit: T <= kDecodeMaxT tokens run the one-launch decode kernel.
constexpr int kDecodeMaxT = 16;
constexpr int kMaxChildren = 3;

// Decode path: the stream launch splits K into at most kDecodeMaxSlices
// slices and writes fp32 partials [slice][token][row] of W0 x and V^T x.
#ifndef WL_DECODE_MAX_SLICES
#define WL_DECODE_MAX_SLICES 8
#endif
constexpr int kDecodeMaxSlices = WL_DECODE_MAX_SLICES;

// One child projection of a (possibly stacked) call, as the kernels see it.
struct ChildDesc {
  const uint16_t *U;   // [N, rpad] bf16, row-major (padded ranks are zero)
  int32_t row_start;   // first row of this child among the call's rows
  int32_t N;           // rows of this child
  int32_t rpad;        // rank rounded up to a multiple of 32 (U row stride)
  int32_t zoff;        // first V^T row / z column of this child
  int32_t y_off;       // first output column of this child in y
  int32_t dup_off;     // second output column offset (K=V tying) or -1
};

// One call: rows [0, Ntot) of W0 and s, ranks [0, Rz) of V^T and z.
struct CallDesc {
  const uint16_t *x;   // [T, K] bf16
  const uint16_t *W0;  // [Ntot, K] bf16 (null for an FP8 bundle's decode call)
  const uint8_t *W0f8; // FP8 bundle: [Ntot, ldw0] E4M3 codes, else null
  const float *q;      // FP8 bundle: [Ntot] per-row scale of W0f8, else null
  int32_t ldw0;        // row stride of W0f8 / W0f4 in bytes
  const uint8_t *W0f4; // MXFP4 bundle: [Ntot, ldw0] E2M1 codes, two per byte (element 2i low), else null
  const uint8_t *sc4;  // MXFP4 bundle: [Ntot, ldsc] E8M0 scale bytes, one per 32 elements
  int32_t ldsc;        // row stride of sc4 in bytes
  const float *s;      // [Ntot]
  const uint16_t *Vt;  // [Rz, K] bf16
  uint16_t *y;         // [T, ldy] bf16
  int32_t T, K, Ntot, Rz, ldy;
  int32_t nchild;
  ChildDesc ch[kMaxChildren];
};

// Decode path (T <= 16): launch 1 streams [W0; V^T] x into the K-slice
// partials p_part [KS][T][Ntot] (fp32) and z = V^T x into zbuf: a bf16
// hi/lo pair [2][T][Rz] when the V^T rows run over the whole K, or two fp32
// slice partials [2][T][Rz] when a long K splits them; launch 2 sums the
// partials and applies the scale and the U z epilogue.
// act >= 0: the call is gate|up (children 0 and 1 with equal N) and the
// epilogue writes h [T][ldh] = act(gate) * up instead of y.
int decode_k_slices(int Ntot, int Rz, int K);
hipError_t launch_decode(const CallDesc &c, float *p_part, void *zbuf, hipStream_t stream, int act = -1,
                         uint16_t *h = nullptr, int ldh = 0);

// Prefill path (T > 16): Z = X V into zbuf [T][Rz] (bf16), then the main
// GEMM with the scale and rank-r epilogue.  GEMMs with few rows split K and
// use pbuf for fp32 partials (prefill_partial_bytes bytes for a call of
// Ntot rows, Rz total padded ranks, largest padded child rank rmax).
// zero_row points at >= 16 zero bytes (used to mask rows and k columns
// outside an operand).
size_t prefill_partial_bytes(int Ntot, int Rz, int rmax, int K, int T);
// act >= 0: gate|up call (children 0 and 1 with equal N) writing
// h [T][ldh] = act(gate) * up instead of y.
hipError_t launch_prefill(const CallDesc &c, uint16_t *zbuf, float *pbuf, const uint16_t *zero_row,
                          hipStream_t stream, int act = -1, uint16_t *h = nullptr, int ldh = 0);

// Effective weight: out[N][K] (bf16) = s (.) W0 + U V^T, with V given as
// rows [K][rpad] (ranks contiguous) and U as [N][rpad]; rpad may be 0.
hipError_t launch_materialize(const uint16_t *V, const uint16_t *U, int32_t N, int32_t K, int32_t rpad,
                              const float *s, const uint16_t *W0, uint16_t *out, const uint16_t *zero_row,
                              hipStream_t stream);

// FP8 shared block: rows of src bf16 [N][K] -> E4M3 codes dst [N][Kp] (Kp a
// multiple of 16, padding zero) and per-row power-of-two scales q [N];
// and back to bf16 [N][K] (value * q).
hipError_t launch_quantize_rows(const uint16_t *src, int32_t N, int32_t K, uint8_t *dst, int32_t Kp, float *q,
                                hipStream_t stream);
hipError_t launch_dequantize_rows(const uint8_t *src, int32_t Kp, const float *q, int32_t N, int32_t K,
                                  uint16_t *dst, hipStream_t stream);
// MXFP4 shared block: rows of src bf16 [N][K] -> E2M1 codes [N][Kq / 2]
// (two per byte) and E8M0 block scales [N][Kq / 32] (Kq a multiple of 128,
// padding zero codes), and back to bf16 [N][K].
hipError_t launch_quantize_mxfp4(const uint16_t *src, int32_t N, int32_t K, uint8_t *codes, int32_t Kq,
                                 uint8_t *scales, hipStream_t stream);
hipError_t launch_dequantize_mxfp4(const uint8_t *codes, int32_t Kq, const uint8_t *scales, int32_t N, int32_t K,
                                   uint16_t *dst, hipStream_t stream);

// Decomposition (one band of one family): W0 = bf16(mean of the m layers
// W [m][nk]); per layer s [N] (LS row scale of W - D against W0, fp32; D =
// the layer's delta U V^T in fp32 [N][K], or NULL) and R = W - s W0 (fp32
// [N][K]; may be D); a strided fp32 GEMM C = A B with A(m,k) = A[m*sam +
// k*sak] and B(k,n) = B[k*sbk + n*sbn], splitting K over up to part_elems /
// (M N) slices whose fp32 partials go to part (NULL: no split); fp32 -> bf16
// and back.  ALS shared-block step: per layer num (+)= diag(s) (W - D), den
// (+)= s^2 (first starts the sums), then W0 = bf16(num / den) on rows with
// den != 0.
hipError_t launch_band_mean(const uint16_t *W, int m, size_t nk, uint16_t *W0, hipStream_t stream);
hipError_t launch_scale_residual(const uint16_t *W, const uint16_t *W0, int N, int K, const float *D, float *s,
                                 float *R, hipStream_t stream);
hipError_t launch_w0_accumulate(const uint16_t *W, const float *D, const float *s, int N, int K, float *num,
                                float *den, bool first, hipStream_t stream);
hipError_t launch_w0_finish(const float *num, const float *den, int N, int K, uint16_t *W0, hipStream_t stream);
hipError_t launch_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t stream);
hipError_t launch_gemm_f32(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn,
                           float *C, int64_t ldc, int M, int N, int K, float *part, size_t part_elems,
                           hipStream_t stream);
hipError_t launch_to_bf16(const float *src, size_t n, uint16_t *dst, hipStream_t stream);

// Text of wl_last_error() for failures reported outside weightless.cpp.
void set_last_error(const char *msg);

// Load-time helpers.
hipError_t launch_fill_zero(void *dst, size_t bytes, hipStream_t stream);
// V [K, r] (row-major, bf16) -> V^T rows [r, K] at dst (row stride K).
hipError_t launch_transpose_v(const uint16_t *V, int32_t K, int32_t r, uint16_t *dst,
                              hipStream_t stream);

}  // namespace wl
