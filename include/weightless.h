/*
 * weightless.h -- C ABI of the weightless linear on AMD Instinct MI355X (gfx950).
 *
 * The method (pages "Add a new model architecture", introduction, and
 * "Quality (Gemma 4 31B)", section "Kernel optimizations"): every dense
 * projection weight of a decoder layer is replaced by a theta bundle -- a
 * block W0 shared by a band of layers, a per-row scale s, and a rank-r delta
 * (U, V) -- and the projection of activations x is evaluated as
 *
 *     y = s (.) (W0 x) + U (V^T x)
 *
 * with the q/k/v (and gate/up) projections of one layer fused into a single
 * stacked call over their shared x.
 *
 * Conventions for every entry point
 *   - Row-major storage, tokens are rows: x [T, K], y [T, N] (N output rows of
 *     the projection become the columns of y), W0 [N, K], s [N], U [N, r],
 *     V [K, r].
 *   - bf16 = IEEE bfloat16 (raw 16-bit patterns); s is float32.  Arithmetic
 *     accumulates in float32; y is rounded to bf16, nearest-even.
 *   - Every function returns a wl_status (0 on success).  Argument errors are
 *     detected on the host and returned before anything is enqueued;
 *     wl_last_error() then describes the failure (thread-local string).
 *   - Device work is only enqueued on the given HIP stream (a hipStream_t
 *     passed as void*, NULL = the null stream); no entry point synchronizes
 *     unless its comment says so.  Device faults surface at the caller's next
 *     synchronization, as for any HIP launch.
 *   - The caller owns all device memory (arena, x, y, workspace).  The
 *     library never allocates device memory.
 */
#ifndef WEIGHTLESS_H
#define WEIGHTLESS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WL_OK = 0,
  WL_EINVAL = -1,   /* bad pointer, index, kind or duplicate/missing source */
  WL_ESHAPE = -2,   /* dimension not allowed (K % 8 != 0, rank > min(N, K), ...) */
  WL_EDTYPE = -3,   /* a source tensor is not in its required dtype */
  WL_ERANGE = -4,   /* layer or family out of range, or family absent */
  WL_ENOSPACE = -5, /* arena or workspace smaller than required */
  WL_EHIP = -6      /* a HIP runtime call failed (message has the HIP error) */
} wl_status;

/* The seven projection families of a decoder layer ("Add the weightless
 * fields" section: q_proj, k_proj, v_proj, o_proj, gate_proj, up_proj,
 * down_proj). */
typedef enum { WL_Q = 0, WL_K = 1, WL_V = 2, WL_O = 3, WL_GATE = 4, WL_UP = 5, WL_DOWN = 6 } wl_family;
#define WL_NUM_FAMILIES 7

/* Stacked calls over one shared x ("Kernel optimizations > GEMM path":
 * q/k/v batched into one call).  Output children are concatenated along N in
 * the order q, k, v (resp. gate, up). */
typedef enum { WL_STACK_QKV = 0, WL_STACK_GATE_UP = 1 } wl_stack;

typedef enum { WL_DTYPE_BF16 = 0, WL_DTYPE_F32 = 1 } wl_dtype;
typedef enum { WL_SRC_W0 = 0, WL_SRC_S = 1, WL_SRC_U = 2, WL_SRC_V = 3 } wl_src_kind;

#define WL_MAX_LAYER_TYPES 2

/* Shape of a theta bundle.
 *  num_layers L, num_bands G (G = the pages' shared_blocks, "Add the weightless
 *    fields"): layer l belongs to band floor(l * G / L) -- contiguous, balanced
 *    bands; 1 <= G <= L.  G = L gives one layer per band (passthrough).
 *  num_layer_types 1 (uniform attention) or 2 (mixed attention: e.g. 0 =
 *    sliding, 1 = full; "Decompose HF weights: the mixed-attention case").
 *  layer_type [L] with values < num_layer_types, or NULL for all type 0.
 *    The array is copied; the caller may free it after theta_bundle_load.
 *  out_dim/in_dim/rank [type][family]: N, K and r.  out_dim 0 means the family
 *    is absent on that type.  K % 8 == 0 is required; 0 <= r <= min(N, K).
 *  k_eq_v_type_mask: bit t set means layers of type t carry no v bundle and
 *    their v projection reuses k's (attention_k_eq_v).
 *  W0 grouping: attention families (q, k, v, o) have one W0 per
 *    (band, layer type, family); MLP families (gate, up, down) one W0 per
 *    (band, family) shared by both layer types, so their out/in dims must agree
 *    across types.  W0 exists only for (band, type) pairs that hold a layer.
 *  w0_format: WL_W0_BF16 (0; a zero-initialized spec) stores W0 as given;
 *    WL_W0_FP8 stores each W0 row as OCP E4M3 codes with one power-of-two
 *    scale q = 2^e per row (e the smallest integer with max|w| <= 448 * 2^e;
 *    code = E4M3(w / q), round to nearest even), coded by theta_bundle_load
 *    from bf16 device sources.  The bundle then stands for W0 = E4M3(code) * q
 *    (the quantized-shared-block variant, "Quality (Gemma 4 31B)" page,
 *    "Verdict"): decode reads one byte per W0 element; prefill and
 *    weightless_materialize expand the call's rows to bf16 in the workspace.
 *    WL_W0_MXFP4 stores W0 in the OCP microscaling format MXFP4: each row
 *    is cut into blocks of 32 elements (the row padded with zeros to a
 *    multiple of 128) sharing one E8M0 scale X = 2^(b - 127), with b = e +
 *    127 kept in [1, 254] and e = floor(log2(block max |w|)) - 2 (0 for an
 *    all-zero block); each element is the E2M1 code nearest to w / X (ties
 *    to the even mantissa, magnitudes clamped to 6), two codes per byte.
 *    Coded by theta_bundle_load from bf16 device sources; decode reads half
 *    a byte per W0 element plus one scale byte per 32, the GEMM paths expand
 *    to bf16 as for FP8. */
typedef enum { WL_W0_BF16 = 0, WL_W0_FP8 = 1, WL_W0_MXFP4 = 2 } wl_w0_format;
typedef struct {
  int32_t num_layers;
  int32_t num_bands;
  int32_t num_layer_types;
  const int8_t *layer_type;
  int32_t out_dim[WL_MAX_LAYER_TYPES][WL_NUM_FAMILIES];
  int32_t in_dim[WL_MAX_LAYER_TYPES][WL_NUM_FAMILIES];
  int32_t rank[WL_MAX_LAYER_TYPES][WL_NUM_FAMILIES];
  uint32_t k_eq_v_type_mask;
  int32_t w0_format;
} wl_bundle_spec;

/* One source tensor handed to theta_bundle_load.
 *  kind W0: index = band, layer_type = type (0 for MLP families), bf16 [N, K]
 *           (on the device for WL_W0_FP8 bundles)
 *  kind S:  index = layer, float32 [N]
 *  kind U:  index = layer, bf16 [N, r]
 *  kind V:  index = layer, bf16 [K, r]   (V, not V^T: y = U (V^T x))
 *  on_device != 0: ptr is device memory (copied on the stream);
 *  on_device == 0: ptr is host memory (copied before theta_bundle_load returns). */
typedef struct {
  int32_t kind;
  int32_t index;
  int32_t layer_type;
  int32_t family;
  int32_t dtype;
  int32_t on_device;
  const void *ptr;
} wl_src;

typedef struct wl_bundle wl_bundle; /* opaque; host metadata only */

/* Bytes of device arena that theta_bundle_load needs for this spec (0 if the
 * spec is invalid; wl_last_error() then says why).  The arena holds, 256-byte
 * aligned, each W0 once -- stacked groups [q;k;v] and [gate;up] with their
 * rows contiguous -- and per layer its s (float32), U (bf16, rows padded to a
 * multiple of 32 ranks) and V^T (bf16 [r, K], ranks padded to a multiple of
 * 32), plus 256 zero bytes used by the kernels for masking. */
size_t theta_bundle_arena_bytes(const wl_bundle_spec *spec);

/* Pack a theta bundle into the caller's device arena (d_arena, 256-byte
 * aligned, at least theta_bundle_arena_bytes(spec) bytes) on `stream`.
 * The ownership follows the pages' model: each shared block W0 is declared
 * once at model level and injected into every layer of its band ("Add a new
 * model architecture" page, "Swap in the weightless layers"), and the layers
 * hold only their s, U and V; pre-decomposed bundles are loaded as they are
 * ("Decompose HF weights: the uniform case", the theta-dict passthrough).
 * Every source the spec implies must appear exactly once in srcs[0..n_src);
 * any other source is an error.  The library never decomposes: sources are
 * already-decomposed bundles.  Nothing is synchronized: device sources may be
 * reused or freed once the stream has passed this point, host sources as soon
 * as the call returns (host V sources are transposed into host buffers owned
 * by the handle, so the handle must not be freed before the stream has passed
 * the load).
 * On success *out receives a handle that refers to the arena (not owning it). */
wl_status theta_bundle_load(const wl_bundle_spec *spec, const wl_src *srcs, size_t n_src,
                            void *d_arena, size_t arena_bytes, void *stream, wl_bundle **out);

/* Free the host handle (never the arena).  NULL is accepted.  Call it only
 * after the stream of its theta_bundle_load has passed the load. */
wl_status theta_bundle_free(wl_bundle *bundle);

/* Workspace bytes needed by any weightless_linear / weightless_stacked_linear
 * call on this bundle with T tokens (T <= 16: decode path; T > 16: prefill
 * path).  The workspace holds intermediate results of one call (fp32 K-slice
 * partials and z for decode; Z = X V and fp32 K-slice partials for prefill);
 * it needs no initialization and keeps nothing between calls.
 * 0 with wl_last_error() set on error. */
size_t weightless_workspace_bytes(const wl_bundle *bundle, int32_t T);

/* y = s (.) (W0 x) + U (V^T x) for one family of one layer: the forward of
 * a weightless projection ("Add a new model architecture" page,
 * introduction: shared block, per-row scale and low-rank delta in place of
 * the dense weight; "Quality (Gemma 4 31B)" page, "Kernel optimizations >
 * GEMM path": bf16 operands, fp32 accumulation).
 *  d_x bf16 [T, K], d_y bf16 [T, N] (must not alias d_x), T >= 0 (T = 0: no-op).
 *  T <= 16 runs the decode path (two launches: one streams [W0; V^T] x into
 *  fp32 K-slice partials of W0 x and z = V^T x, the other sums them, scales
 *  by s, adds U z and stores y), T > 16 the prefill MFMA GEMMs (Z = X V,
 *  then Y = (X W0^T) (.) s + Z U^T; GEMMs with few rows split K and add a
 *  summing launch: 2 to 4 launches).
 *  family WL_V on a K=V-tied layer type evaluates k's bundle.
 *  d_ws: workspace of at least weightless_workspace_bytes(bundle, T) bytes,
 *  256-byte aligned; concurrent calls need distinct workspaces. */
wl_status weightless_linear(const wl_bundle *bundle, int32_t layer, int32_t family,
                            const void *d_x, int32_t T, void *d_y,
                            void *d_ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * call as weightless_linear (same launches and results), with its workspace
 * taken from a fixed array of WL_NOALLOC_WORKSPACE_BYTES bytes of device
 * memory inside the library instead of a caller buffer.  Each GPU holds its
 * own array, reserved when the library is first used on that GPU and kept
 * until the process ends; its address is looked up once per device, on the
 * current device (the stream must belong to it).  Calls that need more
 * workspace than the array holds (weightless_workspace_bytes(bundle, T) >
 * WL_NOALLOC_WORKSPACE_BYTES, e.g. long prefill calls of big bundles or
 * prefill on an FP8 bundle) return WL_ENOSPACE before enqueuing anything.
 * Nothing is allocated and the array needs no initialization, but every call
 * on one GPU shares it: calls that may overlap on one GPU (on different
 * streams, or from several threads without ordering) race and must be
 * serialized by the caller. */
#define WL_NOALLOC_WORKSPACE_BYTES (64u << 20)
wl_status weightless_linear_noalloc(const wl_bundle *bundle, int32_t layer, int32_t family, const void *d_x,
                                    int32_t T, void *d_y, void *stream);

/* The stacked call ("Quality (Gemma 4 31B)" page, "Kernel optimizations >
 * GEMM path": the q, k and v projections of a layer batched into one call
 * over their shared input; K=V tying from "Decompose HF weights: the
 * mixed-attention case"): q|k|v (or gate|up) of one layer over one x: the same
 * launches as a single-family call, over all children's rows at once.  d_y bf16 [T, N_q + N_k + N_v] (resp.
 * [T, N_gate + N_up]).  On a K=V-tied layer type the v slot receives a copy of
 * k's output, so the output layout is the same on every layer. */
wl_status weightless_stacked_linear(const wl_bundle *bundle, int32_t layer, int32_t stack,
                                    const void *d_x, int32_t T, void *d_y,
                                    void *d_ws, size_t ws_bytes, void *stream);

/* Activation of the fused gate|up call (the model's hidden activation). */
typedef enum {
  WL_ACT_GELU_TANH = 0, /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
  WL_ACT_SILU = 1,      /* x / (1 + exp(-x)) */
  WL_ACT_GELU_ERF = 2   /* 0.5 x (1 + erf(x / sqrt(2))) */
} wl_act;

/* The gate|up stack with the MLP activation fused into its epilogue:
 * h = act(gate) (.) up, bf16 [T, N_gate] at d_h, where gate and up are the
 * two children of the stacked call, each kept in fp32 until the product is
 * rounded to bf16 once (so h is not act(bf16(gate)) * bf16(up)).  Requires
 * N_gate == N_up (else WL_ESHAPE); act outside wl_act gives WL_ERANGE.  The
 * same launches and workspace as weightless_stacked_linear(WL_STACK_GATE_UP);
 * d_h must not alias d_x.  It writes half the bytes of the stacked call's
 * y and saves the separate activation pass over it. */
wl_status weightless_gate_up_act(const wl_bundle *bundle, int32_t layer, int32_t act, const void *d_x, int32_t T,
                                 void *d_h, void *d_ws, size_t ws_bytes, void *stream);

/* Workspace bytes weightless_materialize needs for any family of this bundle
 * (the V rows of one family, K x padded rank bf16); 0 on error. */
size_t weightless_materialize_workspace_bytes(const wl_bundle *bundle);

/* The dense weight a bundle stands for: W_eff = diag(s) W0 + U V^T of one
 * family of one layer ("Override the graph build" page: the variant that
 * precomputes the effective weight outside the graph), written as bf16
 * [N, K] row-major to d_weff (16-byte aligned, must not overlap the arena).
 * Each element is one fp32 sum s_i W0[i][j] + sum_k U[i][k] V[j][k] rounded
 * to bf16 (nearest even).  family WL_V on a K=V-tied layer type gives k's
 * weight.  d_ws: at least weightless_materialize_workspace_bytes(bundle)
 * bytes, 256-byte aligned.  Two launches on `stream` (V^T -> V rows, then an
 * MFMA GEMM over the ranks with s W0 added in its epilogue). */
wl_status weightless_materialize(const wl_bundle *bundle, int32_t layer, int32_t family, void *d_weff,
                                 void *d_ws, size_t ws_bytes, void *stream);

/* ---- Decomposition ("Add a new model architecture" page, "Decompose HF
 * weights"; "Quality" page, "Why sharing fails: reconstruction error") ----
 * The analytic one-shot decomposition of one band of one family, on the GPU:
 *   W0 = bf16(mean of the band's m layers), the mean taken in fp64;
 *   per layer, s_i = <W_i, W0_i> / <W0_i, W0_i> (1 for a zero row of W0),
 *   computed in fp64 against the rounded W0 and stored fp32;
 *   U V^T = rank-r truncated SVD of R = W - diag(s) W0, split as
 *   U = P sqrt(S), V = Q sqrt(S), stored bf16.
 * The SVD is randomized subspace iteration (Halko, Martinsson and Tropp,
 * 2011): l = min(rank + oversample, N, K) sketch columns, power_iters rounds,
 * fp32 GPU products, Cholesky-QR orthonormalization (one pass between
 * products, three for the final basis; the l x l factorizations on the host
 * in fp64) and a Jacobi eigen-solve of the l x l matrix B B^T on the host.
 * Its delta is the exact truncated SVD's up to the sketch's accuracy: the
 * error approaches Eckart-Young's as power_iters grows and is exact when
 * rank(R) <= l (oversample 16 and 4 rounds stay within 1% on flat spectra).
 *
 * Workspace bytes for one call (fp32 residual, sketches and factors); 0 if
 * an argument is out of range. */
size_t weightless_decompose_workspace_bytes(int32_t N, int32_t K, int32_t rank, int32_t oversample);

/* d_w: bf16 [m][N][K], the band's layers in layer order (device).
 * d_omega: fp32 [K][l] test matrix, l = min(rank + oversample, N, K)
 *   (device; the caller draws it, e.g. standard normal; may be NULL if
 *   rank == 0).
 * Outputs (device): d_w0 bf16 [N][K]; d_s fp32 [m][N]; d_u bf16 [m][N][rank];
 *   d_v bf16 [m][K][rank] (the layouts theta_bundle_load takes; d_u, d_v may
 *   be NULL if rank == 0).  A zero residual gives U = V = 0.
 * d_ws: >= weightless_decompose_workspace_bytes(N, K, rank, oversample)
 *   bytes, 256-byte aligned.
 * Runs on `stream` and synchronizes it several times per layer (the small
 * host steps); returns when the outputs are written.  WL_EINVAL for NULL
 * pointers, bad counts or non-finite weights; WL_ESHAPE if rank > min(N, K). */
wl_status weightless_decompose(const void *d_w, int32_t m, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                               int32_t power_iters, const float *d_omega, void *d_w0, float *d_s, void *d_u,
                               void *d_v, void *d_ws, size_t ws_bytes, void *stream);

/* ---- ALS refinement of the decomposition ("Quality (Gemma 4 31B)" page,
 * "ALS optimization barely helps": alternating least squares, tried there as
 * an improvement over the mean W0; the page gives no steps) ----
 * weightless_decompose, then `sweeps` sweeps of block-coordinate least
 * squares on J = sum_l ||W_l - diag(s_l) W0 - U_l V_l^T||_F^2, each sweep:
 *   1. W0 = bf16(sum_l s_l (.) (W_l - U_l V_l^T) / sum_l s_l^2), row by row
 *      (fp32 sums in layer order; a row whose scales are all zero keeps W0);
 *   2. per layer, s_i = <(W - U V^T)_i, W0_i> / <W0_i, W0_i> in fp64 (1 for a
 *      zero W0 row), stored fp32;
 *   3. per layer, U V^T = the rank-r randomized truncated SVD of
 *      W - diag(s) W0, as in weightless_decompose (same d_omega).
 * U V^T in steps 1 and 2 is formed in fp32 from the stored bf16 U and V.
 * Each step minimizes J over its block (the SVD up to the sketch's accuracy),
 * so J does not grow from sweep to sweep beyond the rounding and the sketch
 * error.  sweeps == 0 gives weightless_decompose's outputs bit for bit.
 * Arguments, layouts and errors as weightless_decompose, plus: sweeps in
 * [0, 64] (WL_EINVAL otherwise); d_ws >= weightless_decompose_als_workspace_bytes
 * (N, K, rank, oversample) bytes (adds N x K + N fp32 sums). */
size_t weightless_decompose_als_workspace_bytes(int32_t N, int32_t K, int32_t rank, int32_t oversample);
wl_status weightless_decompose_als(const void *d_w, int32_t m, int32_t N, int32_t K, int32_t rank, int32_t oversample,
                                   int32_t power_iters, int32_t sweeps, const float *d_omega, void *d_w0, float *d_s,
                                   void *d_u, void *d_v, void *d_ws, size_t ws_bytes, void *stream);

/* Output width N of a single-family call, or of a stacked call (stack >= 0
 * with family < 0); 0 on error.  Host-only. */
int32_t weightless_out_dim(const wl_bundle *bundle, int32_t layer, int32_t family, int32_t stack);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *wl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WEIGHTLESS_H */
