// GPU decomposition of one band of one family into a theta bundle: the band
// mean W0, per layer the least-squares row scale s and the rank-r delta U V^T
// of the residual ("Add a new model architecture" page, "Decompose HF
// weights"; readings as in the oracle: contiguous bands, LS scale, symmetric
// sqrt(S) split, bf16 storage with W0 rounded before s is fitted).
//
// The truncated SVD of each residual R [N, K] is randomized subspace
// iteration (Halko, Martinsson and Tropp, "Finding structure with
// randomness", 2011): Y = R Omega with l = r + p columns, q rounds of
// Z = R^T Y, Y = R Z, each product orthonormalized by Cholesky-QR (one pass
// between products, three on the final basis); then B = Q^T R, the small symmetric eigenproblem B B^T = W Lambda W^T on
// the host in double (cyclic Jacobi), sigma = sqrt(Lambda), U = Q W_r
// sqrt(sigma_r), V = B^T W_r / sqrt(sigma_r).  The products run on the GPU in
// fp32; the host sees only l x l matrices.  The test matrix Omega is the
// caller's (random numbers are inputs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.h"
#include "weightless.h"

namespace {

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// In-place Cholesky A = L L^T of a symmetric positive-definite n x n matrix
// (row-major, lower triangle written); false if a pivot is not positive.
bool cholesky(std::vector<double> &a, int n) {
  for (int j = 0; j < n; ++j) {
    double d = a[j * n + j];
    for (int k = 0; k < j; ++k) d -= a[j * n + k] * a[j * n + k];
    if (!(d > 0.0)) return false;
    const double ljj = std::sqrt(d);
    a[j * n + j] = ljj;
    for (int i = j + 1; i < n; ++i) {
      double v = a[i * n + j];
      for (int k = 0; k < j; ++k) v -= a[i * n + k] * a[j * n + k];
      a[i * n + j] = v / ljj;
    }
  }
  return true;
}

// T = L^{-T} (upper triangular), row-major n x n, from the lower factor L.
std::vector<double> inv_lower_transpose(const std::vector<double> &L, int n) {
  // X = L^{-1} (lower) by forward substitution, then T = X^T
  std::vector<double> X(static_cast<size_t>(n) * n, 0.0);
  for (int c = 0; c < n; ++c) {
    for (int i = c; i < n; ++i) {
      double v = (i == c) ? 1.0 : 0.0;
      for (int k = c; k < i; ++k) v -= L[i * n + k] * X[k * n + c];
      X[i * n + c] = v / L[i * n + i];
    }
  }
  std::vector<double> T(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) T[i * n + j] = X[j * n + i];
  return T;
}

// Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix (row-major):
// eigenvalues descending in lam, eigenvectors as columns of V.
void jacobi_eigen(std::vector<double> a, int n, std::vector<double> &lam, std::vector<double> &V) {
  V.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) V[i * n + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        tot += a[i * n + j] * a[i * n + j];
        if (i != j) off += a[i * n + j] * a[i * n + j];
      }
    if (off <= 1e-30 * tot || off == 0.0) break;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) {
        const double apq = a[p * n + q];
        if (apq == 0.0) continue;
        const double theta = (a[q * n + q] - a[p * n + p]) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; ++k) {  // rotate columns p, q
          const double akp = a[k * n + p], akq = a[k * n + q];
          a[k * n + p] = c * akp - s * akq;
          a[k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {  // rotate rows p, q
          const double apk = a[p * n + k], aqk = a[q * n + k];
          a[p * n + k] = c * apk - s * aqk;
          a[q * n + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < n; ++k) {
          const double vkp = V[k * n + p], vkq = V[k * n + q];
          V[k * n + p] = c * vkp - s * vkq;
          V[k * n + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int x, int y) { return a[x * n + x] > a[y * n + y]; });
  lam.resize(n);
  std::vector<double> Vs(static_cast<size_t>(n) * n);
  for (int c = 0; c < n; ++c) {
    lam[c] = a[order[c] * n + order[c]];
    for (int k = 0; k < n; ++k) Vs[k * n + c] = V[k * n + order[c]];
  }
  V.swap(Vs);
}

struct Dev {
  hipStream_t s;
  hipError_t err = hipSuccess;
  float *part = nullptr;  // split-K partials of the fp32 GEMMs
  size_t part_elems = 0;
  std::vector<float> up_t, up_u, up_v;  // host sources of in-flight uploads (alive until the next sync)
  bool ok() const { return err == hipSuccess; }
  hipError_t gemm(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn, float *C,
                  int64_t ldc, int M, int N, int K) {
    return wl::launch_gemm_f32(A, sam, sak, B, sbk, sbn, C, ldc, M, N, K, part, part_elems, s);
  }
  // Asynchronous upload from a host vector that stays alive until the next sync.
  void put_async(float *d, std::vector<float> &keep, const std::vector<double> &h) {
    if (!ok()) return;
    keep.assign(h.begin(), h.end());
    err = hipMemcpyAsync(d, keep.data(), keep.size() * 4, hipMemcpyHostToDevice, s);
  }
  std::vector<double> get(const float *d, size_t n) {
    std::vector<float> f(n);
    if (ok()) err = hipMemcpyAsync(f.data(), d, n * 4, hipMemcpyDeviceToHost, s);
    if (ok()) err = hipStreamSynchronize(s);
    return std::vector<double>(f.begin(), f.end());
  }
};

// Y [n x l] <- Y T with Y^T Y = L L^T and T = L^-T, repeated `passes` times
// (Cholesky-QR).  The l x l Gram matrix is formed on the device and factored
// on the host in fp64 (for the l of a sketch, one host round trip measured
// faster than a one-wavefront device factorization).  A rank-deficient Y
// gets a small diagonal shift (shifted Cholesky-QR); the following pass
// restores orthonormality.  tmp is another n x l buffer.
enum Orth { kOrthOk, kOrthZero, kOrthFail };
Orth orthonormalize(Dev &d, float *&Y, float *&tmp, int n, int l, float *small, int passes) {
  for (int pass = 0; pass < passes && d.ok(); ++pass) {
    d.err = d.gemm(Y, 1, l, Y, l, 1, small, l, l, l, n);  // G = Y^T Y
    std::vector<double> G = d.get(small, static_cast<size_t>(l) * l);
    if (!d.ok()) return kOrthFail;
    double tr = 0.0;
    for (int i = 0; i < l; ++i) tr += G[i * l + i];
    if (tr == 0.0) return kOrthZero;
    if (!std::isfinite(tr)) return kOrthFail;
    std::vector<double> L = G;
    bool good = cholesky(L, l);
    for (int attempt = 1; !good && attempt < 8; ++attempt) {
      L = G;
      const double shift = tr / l * std::pow(10.0, -8 + attempt);
      for (int i = 0; i < l; ++i) L[i * l + i] += shift;
      good = cholesky(L, l);
    }
    if (!good) return kOrthFail;
    // the upload needs no wait: the product below is ordered after it on the
    // stream, and the next get() synchronizes before up_t is reused
    d.put_async(small, d.up_t, inv_lower_transpose(L, l));
    if (d.ok()) d.err = d.gemm(Y, l, 1, small, l, 1, tmp, l, n, l, l);  // Y T
    std::swap(Y, tmp);
  }
  return d.ok() ? kOrthOk : kOrthFail;
}

// Split-K partials: up to 16 slices of the largest product output (max(N, K) x l).
size_t part_elems(int N, int K, size_t l) { return 16 * static_cast<size_t>(std::max(N, K)) * l; }

wl_status report(wl_status st, const char *what, int layer, hipError_t e) {
  char buf[256];
  if (st == WL_EHIP)
    std::snprintf(buf, sizeof buf, "weightless_decompose: layer %d: %s", layer, hipGetErrorString(e));
  else
    std::snprintf(buf, sizeof buf, "weightless_decompose: layer %d: %s", layer, what);
  wl::set_last_error(buf);
  return st;
}

size_t base_workspace_bytes(int32_t N, int32_t K, int32_t rank, int32_t oversample) {
  if (N <= 0 || K <= 0 || rank < 0 || oversample < 0) return 0;
  const size_t l = static_cast<size_t>(std::min<int64_t>(static_cast<int64_t>(rank) + oversample, std::min(N, K)));
  size_t n = align256(static_cast<size_t>(N) * K * 4);        // R
  n += 2 * align256(static_cast<size_t>(N) * l * 4);          // Y, spare
  n += 2 * align256(static_cast<size_t>(K) * l * 4);          // Z, spare
  n += align256(l * K * 4);                                   // B
  n += align256(l * l * 4);                                   // small
  n += align256(static_cast<size_t>(N) * rank * 4);                // U in fp32
  n += align256(static_cast<size_t>(K) * rank * 4);                // V in fp32
  n += align256(part_elems(N, K, l) * 4);                          // split-K partials
  return n;
}

// The ALS shared-block step's sums: num (fp32 [N][K]) and den (fp32 [N]).
size_t als_extra_bytes(int32_t N, int32_t K) {
  return align256(static_cast<size_t>(N) * K * 4) + align256(static_cast<size_t>(N) * 4);
}

// The one-shot decomposition of a band, then `sweeps` ALS sweeps: the shared
// block refit from every layer's s and U V^T (fp32 sums in layer order,
// rounded to bf16), then per layer the scale against W0 with the current
// delta removed and the truncated SVD of the new residual, as in the one-shot
// pass.  The deltas are recomputed in fp32 from the stored bf16 U and V.
wl_status decompose_band(const void *d_w, int32_t m, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                         int32_t power_iters, int32_t sweeps, const float *d_omega, void *d_w0, float *d_s,
                         void *d_u, void *d_v, void *d_ws, size_t ws_bytes, void *stream) {
  if (m < 1 || N < 1 || K < 1 || rank < 0 || oversample < 0 || power_iters < 0 || power_iters > 16)
    return report(WL_EINVAL, "need m, N, K >= 1, rank, oversample >= 0 and 0 <= power_iters <= 16", -1, hipSuccess);
  if (sweeps < 0 || sweeps > 64) return report(WL_EINVAL, "need 0 <= sweeps <= 64", -1, hipSuccess);
  if (rank > std::min(N, K)) return report(WL_ESHAPE, "rank exceeds min(N, K)", -1, hipSuccess);
  if (!d_w || !d_w0 || !d_s || !d_ws || (rank > 0 && (!d_u || !d_v || !d_omega)))
    return report(WL_EINVAL, "NULL pointer", -1, hipSuccess);
  if (reinterpret_cast<uintptr_t>(d_ws) % 256) return report(WL_EINVAL, "workspace not 256-byte aligned", -1, hipSuccess);
  const size_t need = base_workspace_bytes(N, K, rank, oversample) + (sweeps > 0 ? als_extra_bytes(N, K) : 0);
  if (ws_bytes < need) return report(WL_ENOSPACE, "workspace too small", -1, hipSuccess);
  const int l = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(rank) + oversample, std::min(N, K)));
  Dev d;
  d.s = static_cast<hipStream_t>(stream);
  uint8_t *ws = static_cast<uint8_t *>(d_ws);
  auto take = [&ws](size_t elems) {
    float *p = reinterpret_cast<float *>(ws);
    ws += align256(elems * 4);
    return p;
  };
  float *R = take(static_cast<size_t>(N) * K);
  float *Y = take(static_cast<size_t>(N) * l), *Y2 = take(static_cast<size_t>(N) * l);
  float *Z = take(static_cast<size_t>(K) * l), *Z2 = take(static_cast<size_t>(K) * l);
  float *B = take(static_cast<size_t>(l) * K);
  float *small = take(static_cast<size_t>(l) * l);
  float *F = take(static_cast<size_t>(N) * rank), *F2 = take(static_cast<size_t>(K) * rank);
  d.part_elems = part_elems(N, K, l);
  d.part = take(d.part_elems);
  float *num = sweeps > 0 ? take(static_cast<size_t>(N) * K) : nullptr;
  float *den = sweeps > 0 ? take(static_cast<size_t>(N)) : nullptr;

  const uint16_t *W = static_cast<const uint16_t *>(d_w);
  uint16_t *W0 = static_cast<uint16_t *>(d_w0);
  uint16_t *Uo = static_cast<uint16_t *>(d_u), *Vo = static_cast<uint16_t *>(d_v);
  const size_t nk = static_cast<size_t>(N) * K;

  // U V^T of R's layer (the residual R, already formed) -> the layer's bf16 U, V
  auto svd_layer = [&](int layer) -> wl_status {
    uint16_t *u = Uo + static_cast<size_t>(layer) * N * rank, *v = Vo + static_cast<size_t>(layer) * K * rank;
    // range finder: Y = R Omega, then q rounds of Z = R^T Y, Y = R Z.  The
    // bases between products only need to stay well conditioned (one
    // Cholesky-QR pass); the final one, which B = Q^T R and U = Q W use,
    // gets three (shifted Cholesky-QR3 when the first pass needs a shift).
    d.err = d.gemm(R, K, 1, d_omega, l, 1, Y, l, N, l, K);
    Orth o = d.ok() ? orthonormalize(d, Y, Y2, N, l, small, power_iters == 0 ? 3 : 1) : kOrthFail;
    for (int it = 0; it < power_iters && o == kOrthOk; ++it) {
      d.err = d.gemm(R, 1, K, Y, l, 1, Z, l, K, l, N);  // Z = R^T Y
      o = d.ok() ? orthonormalize(d, Z, Z2, K, l, small, 1) : kOrthFail;
      if (o != kOrthOk) break;
      d.err = d.gemm(R, K, 1, Z, l, 1, Y, l, N, l, K);  // Y = R Z
      o = d.ok() ? orthonormalize(d, Y, Y2, N, l, small, it + 1 == power_iters ? 3 : 1) : kOrthFail;
    }
    if (!d.ok()) return report(WL_EHIP, "", layer, d.err);
    if (o == kOrthFail)
      return report(WL_EINVAL, "range basis is not numerically positive definite (non-finite weights?)", layer,
                    hipSuccess);
    if (o == kOrthZero) {  // R Omega = 0: the residual is zero, so is its delta
      d.err = hipMemsetAsync(u, 0, static_cast<size_t>(N) * rank * 2, d.s);
      if (d.ok()) d.err = hipMemsetAsync(v, 0, static_cast<size_t>(K) * rank * 2, d.s);
      return d.ok() ? WL_OK : report(WL_EHIP, "", layer, d.err);
    }
    // B = Q^T R [l, K]; B B^T = W Lambda W^T on the host
    d.err = d.gemm(Y, 1, l, R, K, 1, B, K, l, K, N);
    if (d.ok()) d.err = d.gemm(B, K, 1, B, 1, K, small, l, l, l, K);
    std::vector<double> C = d.get(small, static_cast<size_t>(l) * l), lam, Wv;
    if (!d.ok()) return report(WL_EHIP, "", layer, d.err);
    jacobi_eigen(C, l, lam, Wv);
    std::vector<double> Su(static_cast<size_t>(l) * rank), Sv(static_cast<size_t>(l) * rank);
    for (int c = 0; c < rank; ++c) {
      const double sig = std::sqrt(std::max(lam[c], 0.0));
      const double root = std::sqrt(sig);
      for (int i = 0; i < l; ++i) {
        Su[static_cast<size_t>(i) * rank + c] = Wv[static_cast<size_t>(i) * l + c] * root;
        Sv[static_cast<size_t>(i) * rank + c] = sig > 0.0 ? Wv[static_cast<size_t>(i) * l + c] / root : 0.0;
      }
    }
    // U = Q Su [N, r], V = B^T Sv [K, r], rounded to bf16 (no sync: the next
    // layer's round trip, or the final sync, completes them)
    d.put_async(small, d.up_u, Su);
    if (d.ok()) d.err = d.gemm(Y, l, 1, small, rank, 1, F, rank, N, rank, l);
    if (d.ok()) d.err = wl::launch_to_bf16(F, static_cast<size_t>(N) * rank, u, d.s);
    d.put_async(Z2, d.up_v, Sv);
    if (d.ok()) d.err = d.gemm(B, 1, K, Z2, rank, 1, F2, rank, K, rank, l);
    if (d.ok()) d.err = wl::launch_to_bf16(F2, static_cast<size_t>(K) * rank, v, d.s);
    return d.ok() ? WL_OK : report(WL_EHIP, "", layer, d.err);
  };
  // D = U V^T of a layer's stored (bf16) delta, fp32 into R; NULL for rank 0
  auto delta_into_R = [&](int layer) -> const float * {
    if (rank == 0) return nullptr;
    const uint16_t *u = Uo + static_cast<size_t>(layer) * N * rank, *v = Vo + static_cast<size_t>(layer) * K * rank;
    d.err = wl::launch_to_f32(u, static_cast<size_t>(N) * rank, F, d.s);
    if (d.ok()) d.err = wl::launch_to_f32(v, static_cast<size_t>(K) * rank, F2, d.s);
    if (d.ok()) d.err = d.gemm(F, rank, 1, F2, 1, rank, R, K, N, K, rank);
    return R;
  };

  d.err = wl::launch_band_mean(W, m, nk, W0, d.s);
  if (!d.ok()) return report(WL_EHIP, "", -1, d.err);
  for (int layer = 0; layer < m; ++layer) {
    d.err = wl::launch_scale_residual(W + layer * nk, W0, N, K, nullptr, d_s + static_cast<size_t>(layer) * N, R, d.s);
    if (!d.ok()) return report(WL_EHIP, "", layer, d.err);
    if (rank == 0) continue;
    const wl_status st = svd_layer(layer);
    if (st != WL_OK) return st;
  }
  for (int sweep = 0; sweep < sweeps; ++sweep) {
    for (int layer = 0; layer < m; ++layer) {
      const float *D = delta_into_R(layer);
      if (d.ok())
        d.err = wl::launch_w0_accumulate(W + layer * nk, D, d_s + static_cast<size_t>(layer) * N, N, K, num, den,
                                         layer == 0, d.s);
      if (!d.ok()) return report(WL_EHIP, "", layer, d.err);
    }
    d.err = wl::launch_w0_finish(num, den, N, K, W0, d.s);
    if (!d.ok()) return report(WL_EHIP, "", -1, d.err);
    for (int layer = 0; layer < m; ++layer) {
      const float *D = delta_into_R(layer);
      if (d.ok())
        d.err = wl::launch_scale_residual(W + layer * nk, W0, N, K, D, d_s + static_cast<size_t>(layer) * N, R, d.s);
      if (!d.ok()) return report(WL_EHIP, "", layer, d.err);
      if (rank == 0) continue;
      const wl_status st = svd_layer(layer);
      if (st != WL_OK) return st;
    }
  }
  d.err = hipStreamSynchronize(d.s);
  if (!d.ok()) return report(WL_EHIP, "", m - 1, d.err);
  wl::set_last_error("");
  return WL_OK;
}

}  // namespace

extern "C" {

size_t weightless_decompose_workspace_bytes(int32_t N, int32_t K, int32_t rank, int32_t oversample) {
  return base_workspace_bytes(N, K, rank, oversample);
}

wl_status weightless_decompose(const void *d_w, int32_t m, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                               int32_t power_iters, const float *d_omega, void *d_w0, float *d_s, void *d_u,
                               void *d_v, void *d_ws, size_t ws_bytes, void *stream) {
  return decompose_band(d_w, m, N, K, rank, oversample, power_iters, 0, d_omega, d_w0, d_s, d_u, d_v, d_ws, ws_bytes,
                        stream);
}

size_t weightless_decompose_als_workspace_bytes(int32_t N, int32_t K, int32_t rank, int32_t oversample) {
  const size_t base = base_workspace_bytes(N, K, rank, oversample);
  return base ? base + als_extra_bytes(N, K) : 0;
}

wl_status weightless_decompose_als(const void *d_w, int32_t m, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                                   int32_t power_iters, int32_t sweeps, const float *d_omega, void *d_w0, float *d_s,
                                   void *d_u, void *d_v, void *d_ws, size_t ws_bytes, void *stream) {
  return decompose_band(d_w, m, N, K, rank, oversample, power_iters, sweeps, d_omega, d_w0, d_s, d_u, d_v, d_ws,
                        ws_bytes, stream);
}

}  // extern "C"
