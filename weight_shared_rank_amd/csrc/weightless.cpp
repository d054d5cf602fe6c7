// Host side of the weightless linear library: theta-bundle spec validation,
// arena layout, bundle loading and call dispatch (include/weightless.h).
//
// Arena layout (all offsets 256-byte aligned), following the pages' ownership
// model -- W0 declared once per band at model level and injected into every
// layer of the band ("Add a new model architecture" page, "Swap in the
// weightless layers"), grouped per (band, layer type, family) for attention
// and per (band, family) for the MLP ("Decompose HF weights: the
// mixed-attention case"):
//
//   for each band b, layer-type key t, group g in {QKV, O, GATE_UP, DOWN}
//   that some layer of the band uses:
//       W0 group block [sum of child N, K] bf16 -- children's rows
//       concatenated (q;k;v, gate;up), so a stacked call streams one block
//   for each layer l, group g present on l's type:
//       s   [sum N]          float32
//       V^T [sum rpad, K]    bf16   (child ranks padded to a multiple of 32
//                                    with zero rows)
//       U   [N, rpad]        bf16, one block per child (zero pad columns)
//
//   a 256-byte block of zeros (read by the prefill GEMM in place of rows or
//   k columns outside an operand)
//
// A stacked call therefore sees contiguous W0 rows, contiguous s, contiguous
// V^T rows and one U block per child; a single-family call sees a row slice.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "weightless.h"

namespace {

constexpr int kGroups = 4;
enum { G_QKV = 0, G_O = 1, G_GATEUP = 2, G_DOWN = 3 };
constexpr int kGroupOf[WL_NUM_FAMILIES] = {G_QKV, G_QKV, G_QKV, G_O, G_GATEUP, G_GATEUP, G_DOWN};
constexpr int kGroupFams[kGroups][3] = {{WL_Q, WL_K, WL_V}, {WL_O, -1, -1}, {WL_GATE, WL_UP, -1}, {WL_DOWN, -1, -1}};
constexpr int kGroupNFam[kGroups] = {3, 1, 2, 1};
constexpr int32_t kMaxDim = 1 << 20;

inline bool is_mlp_group(int g) { return g >= G_GATEUP; }
inline bool is_mlp_family(int f) { return f >= WL_GATE; }
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

thread_local std::string g_err;

wl_status fail(wl_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

wl_status hip_fail(hipError_t e, const char *what) {
  return fail(WL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

struct GroupShape {
  bool any = false;
  bool tied = false;  // QKV group on a K=V-tied type: the v slot copies k
  int K = 0;
  int Kp = 0;         // FP8 W0 row stride in bytes (K rounded up to 16)
  int Kq = 0;         // MXFP4 W0 elements per row (K rounded up to 128)
  int nchild = 0;
  int fam[3] = {-1, -1, -1};
  int N[3] = {0, 0, 0};
  int r[3] = {0, 0, 0};
  int rpad[3] = {0, 0, 0};
  int row_start[3] = {0, 0, 0};
  int zoff[3] = {0, 0, 0};
  int Ntot = 0;
  int Rtot = 0;
  int child_of_fam[WL_NUM_FAMILIES] = {-1, -1, -1, -1, -1, -1, -1};
};

struct LayerOff {
  int64_t s[kGroups];
  int64_t vt[kGroups];
  int64_t u[kGroups][3];
};

struct Layout {
  int L = 0, G = 0, NT = 0;
  std::vector<int8_t> ltype;
  uint32_t tied_mask = 0;
  GroupShape gs[WL_MAX_LAYER_TYPES][kGroups];
  std::vector<int64_t> w0;  // [(band * NT + tkey) * kGroups + g], -1 if absent
  std::vector<int64_t> w0q; // FP8: per-row scales of that W0 block; MXFP4: its block scales
  bool fp8 = false;
  bool mxfp4 = false;
  bool coded() const { return fp8 || mxfp4; }
  std::vector<LayerOff> lay;
  size_t bytes = 0;
  size_t zero_off = 0;  // 256 zero bytes
  int Rmax = 0;  // largest sum of padded ranks of a group
  int Nmax = 0;  // largest sum of rows of a group

  int band(int l) const { return static_cast<int>((static_cast<int64_t>(l) * G) / L); }
  int64_t &w0_at(int b, int t, int g) { return w0[(static_cast<size_t>(b) * NT + t) * kGroups + g]; }
  int64_t w0_at(int b, int t, int g) const { return w0[(static_cast<size_t>(b) * NT + t) * kGroups + g]; }
  int64_t &w0q_at(int b, int t, int g) { return w0q[(static_cast<size_t>(b) * NT + t) * kGroups + g]; }
  int64_t w0q_at(int b, int t, int g) const { return w0q[(static_cast<size_t>(b) * NT + t) * kGroups + g]; }
  size_t w0_row_bytes(const GroupShape &gs) const {
    return fp8 ? static_cast<size_t>(gs.Kp) : mxfp4 ? static_cast<size_t>(gs.Kq) / 2 : static_cast<size_t>(gs.K) * 2;
  }
  // bytes per row of the scale region after a coded W0 block
  size_t w0_scale_row_bytes(const GroupShape &gs) const { return fp8 ? 4 : static_cast<size_t>(gs.Kq) / 32; }
};

bool tied(const Layout &lo, int t) { return (lo.tied_mask >> t) & 1u; }

// Validate the spec and compute the arena layout.
wl_status make_layout(const wl_bundle_spec *spec, Layout &lo) {
  if (!spec) return fail(WL_EINVAL, "spec is NULL");
  const int L = spec->num_layers, G = spec->num_bands, NT = spec->num_layer_types;
  if (L < 1 || L > kMaxDim) return fail(WL_EINVAL, "num_layers %d out of range", L);
  if (G < 1 || G > L) return fail(WL_EINVAL, "num_bands %d must be in [1, num_layers=%d]", G, L);
  if (NT < 1 || NT > WL_MAX_LAYER_TYPES) return fail(WL_EINVAL, "num_layer_types %d must be 1 or 2", NT);
  if (spec->k_eq_v_type_mask >> NT) return fail(WL_EINVAL, "k_eq_v_type_mask 0x%x names a layer type >= %d", spec->k_eq_v_type_mask, NT);
  if (spec->w0_format != WL_W0_BF16 && spec->w0_format != WL_W0_FP8 && spec->w0_format != WL_W0_MXFP4)
    return fail(WL_EINVAL, "w0_format %d invalid", spec->w0_format);
  lo.fp8 = spec->w0_format == WL_W0_FP8;
  lo.mxfp4 = spec->w0_format == WL_W0_MXFP4;
  lo.L = L;
  lo.G = G;
  lo.NT = NT;
  lo.tied_mask = spec->k_eq_v_type_mask;
  lo.ltype.assign(L, 0);
  if (spec->layer_type) {
    for (int l = 0; l < L; ++l) {
      if (spec->layer_type[l] < 0 || spec->layer_type[l] >= NT)
        return fail(WL_EINVAL, "layer_type[%d] = %d out of range", l, spec->layer_type[l]);
      lo.ltype[l] = spec->layer_type[l];
    }
  }
  for (int t = 0; t < NT; ++t) {
    for (int f = 0; f < WL_NUM_FAMILIES; ++f) {
      if (f == WL_V && tied(lo, t)) continue;
      const int N = spec->out_dim[t][f], K = spec->in_dim[t][f], r = spec->rank[t][f];
      if (N < 0 || N > kMaxDim) return fail(WL_ESHAPE, "out_dim[%d][%d] = %d out of range", t, f, N);
      if (N == 0) continue;
      if (K <= 0 || K > kMaxDim) return fail(WL_ESHAPE, "in_dim[%d][%d] = %d out of range", t, f, K);
      if (K % 8) return fail(WL_ESHAPE, "in_dim[%d][%d] = %d is not a multiple of 8", t, f, K);
      if (r < 0 || r > N || r > K) return fail(WL_ESHAPE, "rank[%d][%d] = %d outside [0, min(N=%d, K=%d)]", t, f, r, N, K);
    }
    if (tied(lo, t) && spec->out_dim[t][WL_K] == 0)
      return fail(WL_ESHAPE, "layer type %d ties v to k but has no k", t);
  }
  if (NT == 2) {
    for (int f = WL_GATE; f <= WL_DOWN; ++f)
      if (spec->out_dim[0][f] != spec->out_dim[1][f] || (spec->out_dim[0][f] && spec->in_dim[0][f] != spec->in_dim[1][f]))
        return fail(WL_ESHAPE, "MLP family %d shares W0 across layer types but its shape differs between them", f);
  }
  // Group shapes per layer type.
  lo.Rmax = 0;
  lo.Nmax = 0;
  for (int t = 0; t < NT; ++t) {
    for (int g = 0; g < kGroups; ++g) {
      GroupShape &gs = lo.gs[t][g];
      gs = GroupShape();
      for (int i = 0; i < kGroupNFam[g]; ++i) {
        const int f = kGroupFams[g][i];
        if (f == WL_V && tied(lo, t)) {
          gs.tied = true;
          continue;
        }
        const int N = spec->out_dim[t][f];
        if (N == 0) continue;
        const int K = spec->in_dim[t][f];
        if (gs.nchild > 0 && K != gs.K)
          return fail(WL_ESHAPE, "families of one stacked group need one in_dim (type %d family %d: %d vs %d)", t, f, K, gs.K);
        const int c = gs.nchild++;
        gs.K = K;
        gs.Kp = (K + 15) & ~15;
        gs.Kq = (K + 127) & ~127;
        gs.fam[c] = f;
        gs.N[c] = N;
        gs.r[c] = spec->rank[t][f];
        gs.rpad[c] = (gs.r[c] + 31) & ~31;
        gs.row_start[c] = gs.Ntot;
        gs.zoff[c] = gs.Rtot;
        gs.Ntot += N;
        gs.Rtot += gs.rpad[c];
        gs.child_of_fam[f] = c;
        gs.any = true;
      }
      if (!gs.any) gs.tied = false;
      if (gs.Rtot > lo.Rmax) lo.Rmax = gs.Rtot;
      if (gs.Ntot > lo.Nmax) lo.Nmax = gs.Ntot;
    }
  }
  // W0 regions: one per (band, type key, group) used by some layer.
  size_t off = 0;
  lo.w0.assign(static_cast<size_t>(G) * NT * kGroups, -1);
  lo.w0q.assign(static_cast<size_t>(G) * NT * kGroups, -1);
  for (int b = 0; b < G; ++b) {
    for (int t = 0; t < NT; ++t) {
      for (int g = 0; g < kGroups; ++g) {
        if (is_mlp_group(g) && t != 0) continue;
        bool used = false;
        for (int l = 0; l < L && !used; ++l)
          if (lo.band(l) == b && (is_mlp_group(g) || lo.ltype[l] == t) && lo.gs[lo.ltype[l]][g].any) used = true;
        if (!used) continue;
        const GroupShape &gs = lo.gs[t][g];
        lo.w0_at(b, t, g) = static_cast<int64_t>(off);
        off = align256(off + static_cast<size_t>(gs.Ntot) * lo.w0_row_bytes(gs));
        if (lo.coded()) {
          lo.w0q_at(b, t, g) = static_cast<int64_t>(off);
          off = align256(off + static_cast<size_t>(gs.Ntot) * lo.w0_scale_row_bytes(gs));
        }
      }
    }
  }
  lo.lay.resize(L);
  for (int l = 0; l < L; ++l) {
    LayerOff &lf = lo.lay[l];
    const int t = lo.ltype[l];
    for (int g = 0; g < kGroups; ++g) {
      lf.s[g] = lf.vt[g] = -1;
      for (int c = 0; c < 3; ++c) lf.u[g][c] = -1;
      const GroupShape &gs = lo.gs[t][g];
      if (!gs.any) continue;
      lf.s[g] = static_cast<int64_t>(off);
      off = align256(off + static_cast<size_t>(gs.Ntot) * 4);
      lf.vt[g] = static_cast<int64_t>(off);
      off = align256(off + static_cast<size_t>(gs.Rtot) * gs.K * 2);
      for (int c = 0; c < gs.nchild; ++c) {
        lf.u[g][c] = static_cast<int64_t>(off);
        off = align256(off + static_cast<size_t>(gs.N[c]) * gs.rpad[c] * 2);
      }
    }
  }
  lo.zero_off = off;
  off += 256;
  lo.bytes = off;
  return WL_OK;
}

// Workspace.  Decode (T <= 16): the stream launch's fp32 partials,
// p_part [kDecodeMaxSlices][T][Nmax] (fp32), then z: a bf16 pair or two fp32
// slice partials, [2][T][Rmax] of 4-byte slots.
// Prefill (T > 16): Z = X V as bf16 [T][Rmax].
size_t ws_p_part_bytes(const Layout &lo, int32_t T) {
  return align256(static_cast<size_t>(wl::kDecodeMaxSlices) * T * lo.Nmax * 4);
}

// Prefill (T > 16): Z [T][Rmax] bf16, then the fp32 K-split partials of the
// largest call shape of the bundle.
size_t ws_prefill_z_bytes(const Layout &lo, int32_t T) { return align256(static_cast<size_t>(T) * lo.Rmax * 2); }

size_t ws_prefill_partial_bytes(const Layout &lo, int32_t T) {
  size_t n = 0;
  for (int t = 0; t < lo.NT; ++t)
    for (int g = 0; g < kGroups; ++g) {
      const GroupShape &gs = lo.gs[t][g];
      if (!gs.any) continue;
      // the stacked call and every single-family call of the group
      int rmax = 0;
      for (int c = 0; c < gs.nchild; ++c) {
        rmax = std::max(rmax, gs.rpad[c]);
        n = std::max(n, wl::prefill_partial_bytes(gs.N[c], gs.rpad[c], gs.rpad[c], gs.K, T));
      }
      n = std::max(n, wl::prefill_partial_bytes(gs.Ntot, gs.Rtot, rmax, gs.K, T));
    }
  return align256(n);
}

// FP8 and MXFP4 bundles: the bf16 expansion of the largest W0 row block a
// call reads (prefill and materialization run the bf16 GEMM on it).
size_t ws_w0_expand_bytes(const Layout &lo) {
  if (!lo.coded()) return 0;
  size_t n = 0;
  for (int t = 0; t < lo.NT; ++t)
    for (int g = 0; g < kGroups; ++g) {
      const GroupShape &gs = lo.gs[t][g];
      if (gs.any) n = std::max(n, static_cast<size_t>(gs.Ntot) * gs.K * 2);
    }
  return align256(n);
}

size_t ws_bytes_for(const Layout &lo, int32_t T) {
  size_t n;
  if (T <= wl::kDecodeMaxT)  // z: a bf16 pair or two fp32 slices, [2][T][Rmax]
    n = ws_p_part_bytes(lo, T) + align256(static_cast<size_t>(2) * T * lo.Rmax * 4);
  else
    n = ws_prefill_z_bytes(lo, T) + ws_prefill_partial_bytes(lo, T) + ws_w0_expand_bytes(lo);
  return n < 256 ? 256 : n;
}

}  // namespace

struct wl_bundle {
  Layout lo;
  uint8_t *arena = nullptr;
  size_t arena_bytes = 0;
  // V^T of host-resident V sources, transposed on the host; the load's
  // copies read them on the stream, so they live as long as the handle
  std::vector<std::vector<uint16_t>> host_vt;
};

namespace {

struct Resolved {
  wl::CallDesc c;
  int out_dim;
};

// Fill a CallDesc for (layer, family) or (layer, stack).
wl_status resolve(const wl_bundle *h, int32_t layer, int32_t family, int32_t stack, Resolved &rv) {
  if (!h) return fail(WL_EINVAL, "bundle is NULL");
  const Layout &lo = h->lo;
  if (layer < 0 || layer >= lo.L) return fail(WL_ERANGE, "layer %d outside [0, %d)", layer, lo.L);
  const int t = lo.ltype[layer];
  const int b = lo.band(layer);
  int g;
  int first = 0, last = 0;  // children range [first, last)
  const bool single = stack < 0;
  if (single) {
    if (family < 0 || family >= WL_NUM_FAMILIES) return fail(WL_ERANGE, "family %d out of range", family);
    int f = family;
    if (f == WL_V && tied(lo, t)) f = WL_K;
    g = kGroupOf[f];
    const int c = lo.gs[t][g].child_of_fam[f];
    if (c < 0) return fail(WL_ERANGE, "family %d is absent on layer %d (type %d)", family, layer, t);
    first = c;
    last = c + 1;
  } else {
    if (stack != WL_STACK_QKV && stack != WL_STACK_GATE_UP) return fail(WL_ERANGE, "stack %d out of range", stack);
    g = stack == WL_STACK_QKV ? G_QKV : G_GATEUP;
    const GroupShape &gs = lo.gs[t][g];
    const int need = stack == WL_STACK_QKV ? (gs.tied ? 2 : 3) : 2;
    if (gs.nchild != need)
      return fail(WL_ERANGE, "stacked call %d needs all of its families on layer %d (type %d has %d of %d)", stack, layer, t, gs.nchild, need);
    first = 0;
    last = gs.nchild;
  }
  const GroupShape &gs = lo.gs[t][g];
  const int tkey = is_mlp_group(g) ? 0 : t;
  const int64_t w0off = lo.w0_at(b, tkey, g);
  const LayerOff &lf = lo.lay[layer];
  uint8_t *A = h->arena;
  wl::CallDesc &c = rv.c;
  std::memset(&c, 0, sizeof c);
  const int rs0 = gs.row_start[first];
  const int z0 = gs.zoff[first];
  c.K = gs.K;
  if (lo.fp8) {
    c.W0 = nullptr;
    c.W0f8 = A + w0off + static_cast<size_t>(rs0) * gs.Kp;
    c.q = reinterpret_cast<const float *>(A + lo.w0q_at(b, tkey, g)) + rs0;
    c.ldw0 = gs.Kp;
  } else if (lo.mxfp4) {
    c.W0 = nullptr;
    c.ldw0 = gs.Kq / 2;
    c.ldsc = gs.Kq / 32;
    c.W0f4 = A + w0off + static_cast<size_t>(rs0) * c.ldw0;
    c.sc4 = A + lo.w0q_at(b, tkey, g) + static_cast<size_t>(rs0) * c.ldsc;
  } else {
    c.W0 = reinterpret_cast<const uint16_t *>(A + w0off) + static_cast<size_t>(rs0) * gs.K;
  }
  c.s = reinterpret_cast<const float *>(A + lf.s[g]) + rs0;
  c.Vt = reinterpret_cast<const uint16_t *>(A + lf.vt[g]) + static_cast<size_t>(z0) * gs.K;
  c.nchild = last - first;
  int ycol = 0;
  c.Ntot = 0;
  c.Rz = 0;
  for (int i = first; i < last; ++i) {
    wl::ChildDesc &ch = c.ch[i - first];
    ch.U = reinterpret_cast<const uint16_t *>(A + lf.u[g][i]);
    ch.row_start = gs.row_start[i] - rs0;
    ch.N = gs.N[i];
    ch.rpad = gs.rpad[i];
    ch.zoff = gs.zoff[i] - z0;
    ch.y_off = ycol;
    ycol += gs.N[i];
    ch.dup_off = -1;
    c.Ntot += gs.N[i];
    c.Rz += gs.rpad[i];
  }
  if (!single && gs.tied) {
    // q | k | k: the k child also writes the v slot right after itself.
    wl::ChildDesc &kch = c.ch[gs.child_of_fam[WL_K]];
    kch.dup_off = ycol;
    ycol += kch.N;
  }
  rv.out_dim = ycol;
  return WL_OK;
}

// act >= 0: the gate|up stack with the activation fused; d_y then receives
// h = act(gate) * up, [T, N_gate].
wl_status run_call(const wl_bundle *h, int32_t layer, int32_t family, int32_t stack, const void *d_x,
                   int32_t T, void *d_y, void *d_ws, size_t ws_bytes, void *stream, int32_t act = -1) {
  Resolved rv;
  wl_status st = resolve(h, layer, family, stack, rv);
  if (st != WL_OK) return st;
  if (act >= 0) {
    if (rv.c.nchild != 2 || rv.c.ch[0].N != rv.c.ch[1].N)
      return fail(WL_ESHAPE, "gate and up of layer %d must have equal out_dim", layer);
    rv.out_dim = rv.c.ch[0].N;
  }
  if (T < 0) return fail(WL_EINVAL, "T = %d is negative", T);
  if (T > kMaxDim) return fail(WL_ESHAPE, "T = %d too large", T);
  if (T == 0) return WL_OK;
  if (!d_x || !d_y || !d_ws) return fail(WL_EINVAL, "x, y and workspace must be non-NULL");
  if (reinterpret_cast<uintptr_t>(d_x) % 16) return fail(WL_EINVAL, "x must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(d_y) % 2) return fail(WL_EINVAL, "y must be 2-byte aligned");
  if (reinterpret_cast<uintptr_t>(d_ws) % 256) return fail(WL_EINVAL, "workspace must be 256-byte aligned");
  const size_t need = ws_bytes_for(h->lo, T);
  if (ws_bytes < need) return fail(WL_ENOSPACE, "workspace has %zu bytes, call needs %zu", ws_bytes, need);
  const uint8_t *xb = static_cast<const uint8_t *>(d_x);
  const uint8_t *yb = static_cast<const uint8_t *>(d_y);
  const size_t xbytes = static_cast<size_t>(T) * rv.c.K * 2, ybytes = static_cast<size_t>(T) * rv.out_dim * 2;
  if (xb < yb + ybytes && yb < xb + xbytes) return fail(WL_EINVAL, "y must not overlap x");
  rv.c.x = static_cast<const uint16_t *>(d_x);
  rv.c.y = static_cast<uint16_t *>(d_y);
  rv.c.T = T;
  rv.c.ldy = rv.out_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = static_cast<uint8_t *>(d_ws);
  hipError_t e;
  uint16_t *hout = act >= 0 ? static_cast<uint16_t *>(d_y) : nullptr;
  if (T <= wl::kDecodeMaxT)
    e = wl::launch_decode(rv.c, reinterpret_cast<float *>(ws), ws + ws_p_part_bytes(h->lo, T), s, act, hout,
                          rv.out_dim);
  else {
    // internal guard: this call's split partials fit the region sized for
    // the largest call shape of the bundle
    int rmax = 0;
    for (int c = 0; c < rv.c.nchild; ++c) rmax = std::max(rmax, static_cast<int>(rv.c.ch[c].rpad));
    if (wl::prefill_partial_bytes(rv.c.Ntot, rv.c.Rz, rmax, rv.c.K, T) > ws_prefill_partial_bytes(h->lo, T))
      return fail(WL_ENOSPACE, "internal: prefill partials of this call exceed the planned workspace");
    if (h->lo.coded()) {
      // FP8 / MXFP4 bundle: expand this call's W0 rows to bf16 for the GEMM
      uint16_t *w0 = reinterpret_cast<uint16_t *>(ws + ws_prefill_z_bytes(h->lo, T) + ws_prefill_partial_bytes(h->lo, T));
      e = h->lo.fp8 ? wl::launch_dequantize_rows(rv.c.W0f8, rv.c.ldw0, rv.c.q, rv.c.Ntot, rv.c.K, w0, s)
                    : wl::launch_dequantize_mxfp4(rv.c.W0f4, 2 * rv.c.ldw0, rv.c.sc4, rv.c.Ntot, rv.c.K, w0, s);
      if (e != hipSuccess) return hip_fail(e, "W0 expand launch");
      rv.c.W0 = w0;
    }
    e = wl::launch_prefill(rv.c, reinterpret_cast<uint16_t *>(ws),
                           reinterpret_cast<float *>(ws + ws_prefill_z_bytes(h->lo, T)),
                           reinterpret_cast<const uint16_t *>(h->arena + h->lo.zero_off), s, act, hout,
                           rv.out_dim);
  }
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return WL_OK;
}

// Fixed device workspace of weightless_linear_noalloc, for callers that
// cannot allocate.  Each device holds its own copy of the array for the life
// of the process; host code uses only the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
__device__ __align__(256) uint8_t scratch[WL_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array, looked up once per device.
wl_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(WL_EINVAL, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(WL_EHIP, "hipGetSymbolAddress(scratch) returned NULL on device %d", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WL_OK;
}

}  // namespace

namespace wl {
void set_last_error(const char *msg) { g_err = msg ? msg : ""; }
}  // namespace wl

extern "C" {

const char *wl_last_error(void) { return g_err.c_str(); }

size_t theta_bundle_arena_bytes(const wl_bundle_spec *spec) {
  Layout lo;
  if (make_layout(spec, lo) != WL_OK) return 0;
  g_err.clear();
  return lo.bytes;
}

wl_status theta_bundle_load(const wl_bundle_spec *spec, const wl_src *srcs, size_t n_src, void *d_arena,
                            size_t arena_bytes, void *stream, wl_bundle **out) {
  if (!out) return fail(WL_EINVAL, "out is NULL");
  *out = nullptr;
  Layout lo;
  wl_status st = make_layout(spec, lo);
  if (st != WL_OK) return st;
  if (!d_arena) return fail(WL_EINVAL, "arena is NULL");
  if (reinterpret_cast<uintptr_t>(d_arena) % 256) return fail(WL_EINVAL, "arena must be 256-byte aligned");
  if (arena_bytes < lo.bytes) return fail(WL_ENOSPACE, "arena has %zu bytes, bundle needs %zu", arena_bytes, lo.bytes);
  if (n_src && !srcs) return fail(WL_EINVAL, "srcs is NULL");

  // Expected sources.
  using Key = std::array<int, 4>;  // kind, index, type key, family
  std::map<Key, int> expect;       // -> index in srcs, or -1 while missing
  for (int b = 0; b < lo.G; ++b)
    for (int t = 0; t < lo.NT; ++t)
      for (int g = 0; g < kGroups; ++g) {
        if (lo.w0_at(b, t, g) < 0) continue;
        const GroupShape &gs = lo.gs[t][g];
        for (int c = 0; c < gs.nchild; ++c) expect[Key{WL_SRC_W0, b, t, gs.fam[c]}] = -1;
      }
  for (int l = 0; l < lo.L; ++l) {
    const int t = lo.ltype[l];
    for (int g = 0; g < kGroups; ++g) {
      const GroupShape &gs = lo.gs[t][g];
      for (int c = 0; c < gs.nchild; ++c) {
        expect[Key{WL_SRC_S, l, 0, gs.fam[c]}] = -1;
        if (gs.r[c] > 0) {
          expect[Key{WL_SRC_U, l, 0, gs.fam[c]}] = -1;
          expect[Key{WL_SRC_V, l, 0, gs.fam[c]}] = -1;
        }
      }
    }
  }
  for (size_t i = 0; i < n_src; ++i) {
    const wl_src &s = srcs[i];
    if (s.kind < WL_SRC_W0 || s.kind > WL_SRC_V) return fail(WL_EINVAL, "source %zu: kind %d invalid", i, s.kind);
    if (s.family < 0 || s.family >= WL_NUM_FAMILIES) return fail(WL_EINVAL, "source %zu: family %d invalid", i, s.family);
    if (!s.ptr) return fail(WL_EINVAL, "source %zu: ptr is NULL", i);
    const int want_dtype = s.kind == WL_SRC_S ? WL_DTYPE_F32 : WL_DTYPE_BF16;
    if (s.dtype != want_dtype)
      return fail(WL_EDTYPE, "source %zu (kind %d): dtype %d, required %d", i, s.kind, s.dtype, want_dtype);
    int tkey = 0;
    if (s.kind == WL_SRC_W0 && !is_mlp_family(s.family)) tkey = s.layer_type;
    const Key k{s.kind, s.index, tkey, s.family};
    auto it = expect.find(k);
    if (it == expect.end())
      return fail(WL_EINVAL, "source %zu (kind %d, index %d, type %d, family %d) is not part of this bundle", i, s.kind,
                  s.index, s.layer_type, s.family);
    if (it->second >= 0) return fail(WL_EINVAL, "source %zu duplicates source %d", i, it->second);
    if (s.kind == WL_SRC_W0 && lo.coded() && !s.on_device)
      return fail(WL_EINVAL, "source %zu: an FP8 or MXFP4 bundle codes W0 on the device; pass a device tensor", i);
    it->second = static_cast<int>(i);
  }
  for (const auto &kv : expect)
    if (kv.second < 0)
      return fail(WL_EINVAL, "missing source: kind %d, index %d, type %d, family %d", kv.first[0], kv.first[1],
                  kv.first[2], kv.first[3]);

  hipStream_t strm = static_cast<hipStream_t>(stream);
  uint8_t *A = static_cast<uint8_t *>(d_arena);
  hipError_t e = wl::launch_fill_zero(A, lo.bytes, strm);
  if (e != hipSuccess) return hip_fail(e, "arena fill");
  std::unique_ptr<wl_bundle> h(new wl_bundle);
  for (const auto &kv : expect) {
    const wl_src &s = srcs[kv.second];
    const hipMemcpyKind kind = s.on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
    if (s.kind == WL_SRC_W0) {
      const int t = kv.first[2];
      const int g = kGroupOf[s.family];
      const GroupShape &gs = lo.gs[t][g];
      const int c = gs.child_of_fam[s.family];
      uint8_t *dst = A + lo.w0_at(s.index, t, g) + static_cast<size_t>(gs.row_start[c]) * lo.w0_row_bytes(gs);
      if (lo.fp8) {
        float *q = reinterpret_cast<float *>(A + lo.w0q_at(s.index, t, g)) + gs.row_start[c];
        e = wl::launch_quantize_rows(static_cast<const uint16_t *>(s.ptr), gs.N[c], gs.K, dst, gs.Kp, q, strm);
        if (e != hipSuccess) return hip_fail(e, "W0 quantize");
        continue;
      }
      if (lo.mxfp4) {
        uint8_t *sc = A + lo.w0q_at(s.index, t, g) + static_cast<size_t>(gs.row_start[c]) * lo.w0_scale_row_bytes(gs);
        e = wl::launch_quantize_mxfp4(static_cast<const uint16_t *>(s.ptr), gs.N[c], gs.K, dst, gs.Kq, sc, strm);
        if (e != hipSuccess) return hip_fail(e, "W0 quantize");
        continue;
      }
      e = hipMemcpyAsync(dst, s.ptr, static_cast<size_t>(gs.N[c]) * gs.K * 2, kind, strm);
      if (e != hipSuccess) return hip_fail(e, "W0 copy");
      continue;
    }
    const int l = s.index;
    const int t = lo.ltype[l];
    const int g = kGroupOf[s.family];
    const GroupShape &gs = lo.gs[t][g];
    const int c = gs.child_of_fam[s.family];
    const LayerOff &lf = lo.lay[l];
    const int N = gs.N[c], K = gs.K, r = gs.r[c];
    if (s.kind == WL_SRC_S) {
      e = hipMemcpyAsync(A + lf.s[g] + static_cast<size_t>(gs.row_start[c]) * 4, s.ptr, static_cast<size_t>(N) * 4, kind, strm);
    } else if (s.kind == WL_SRC_U) {
      uint8_t *dst = A + lf.u[g][c];
      if (r == gs.rpad[c])
        e = hipMemcpyAsync(dst, s.ptr, static_cast<size_t>(N) * r * 2, kind, strm);
      else
        e = hipMemcpy2DAsync(dst, static_cast<size_t>(gs.rpad[c]) * 2, s.ptr, static_cast<size_t>(r) * 2,
                             static_cast<size_t>(r) * 2, N, kind, strm);
    } else {  // V [K, r] -> V^T rows zoff.. of the group block
      uint16_t *dst = reinterpret_cast<uint16_t *>(A + lf.vt[g]) + static_cast<size_t>(gs.zoff[c]) * K;
      if (s.on_device) {
        e = wl::launch_transpose_v(static_cast<const uint16_t *>(s.ptr), K, r, dst, strm);
      } else {
        const uint16_t *V = static_cast<const uint16_t *>(s.ptr);
        h->host_vt.emplace_back(static_cast<size_t>(r) * K);
        std::vector<uint16_t> &vt = h->host_vt.back();
        for (int k = 0; k < K; ++k)
          for (int j = 0; j < r; ++j) vt[static_cast<size_t>(j) * K + k] = V[static_cast<size_t>(k) * r + j];
        e = hipMemcpyAsync(dst, vt.data(), vt.size() * 2, hipMemcpyHostToDevice, strm);
      }
    }
    if (e != hipSuccess) return hip_fail(e, "bundle copy");
  }
  h->lo = std::move(lo);
  h->arena = A;
  h->arena_bytes = arena_bytes;
  *out = h.release();
  g_err.clear();
  return WL_OK;
}

wl_status theta_bundle_free(wl_bundle *bundle) {
  delete bundle;
  return WL_OK;
}

size_t weightless_workspace_bytes(const wl_bundle *bundle, int32_t T) {
  if (!bundle) {
    fail(WL_EINVAL, "bundle is NULL");
    return 0;
  }
  if (T < 0) {
    fail(WL_EINVAL, "T = %d is negative", T);
    return 0;
  }
  return ws_bytes_for(bundle->lo, T);
}

wl_status weightless_linear(const wl_bundle *bundle, int32_t layer, int32_t family, const void *d_x, int32_t T,
                            void *d_y, void *d_ws, size_t ws_bytes, void *stream) {
  return run_call(bundle, layer, family, -1, d_x, T, d_y, d_ws, ws_bytes, stream);
}

wl_status weightless_linear_noalloc(const wl_bundle *bundle, int32_t layer, int32_t family, const void *d_x,
                                    int32_t T, void *d_y, void *stream) {
  if (!bundle) return fail(WL_EINVAL, "bundle is NULL");
  if (T < 0) return fail(WL_EINVAL, "T = %d is negative", T);
  if (T > kMaxDim) return fail(WL_ESHAPE, "T = %d too large", T);
  const size_t need = ws_bytes_for(bundle->lo, T);
  if (need > WL_NOALLOC_WORKSPACE_BYTES)
    return fail(WL_ENOSPACE, "this call needs %zu bytes of workspace; the fixed workspace of "
                "weightless_linear_noalloc holds %zu (use weightless_linear with a caller workspace)",
                need, static_cast<size_t>(WL_NOALLOC_WORKSPACE_BYTES));
  void *ws = nullptr;
  const wl_status st = scratch_of_current_device(&ws);
  if (st != WL_OK) return st;
  return run_call(bundle, layer, family, -1, d_x, T, d_y, ws, WL_NOALLOC_WORKSPACE_BYTES, stream);
}

wl_status weightless_stacked_linear(const wl_bundle *bundle, int32_t layer, int32_t stack, const void *d_x, int32_t T,
                                    void *d_y, void *d_ws, size_t ws_bytes, void *stream) {
  if (stack < 0) return fail(WL_ERANGE, "stack %d out of range", stack);
  return run_call(bundle, layer, -1, stack, d_x, T, d_y, d_ws, ws_bytes, stream);
}

wl_status weightless_gate_up_act(const wl_bundle *bundle, int32_t layer, int32_t act, const void *d_x, int32_t T,
                                 void *d_h, void *d_ws, size_t ws_bytes, void *stream) {
  if (act < WL_ACT_GELU_TANH || act > WL_ACT_GELU_ERF) return fail(WL_ERANGE, "activation %d out of range", act);
  return run_call(bundle, layer, -1, WL_STACK_GATE_UP, d_x, T, d_h, d_ws, ws_bytes, stream, act);
}

size_t weightless_materialize_workspace_bytes(const wl_bundle *bundle) {
  if (!bundle) {
    fail(WL_EINVAL, "bundle is NULL");
    return 0;
  }
  size_t n = 256;
  const Layout &lo = bundle->lo;
  for (int t = 0; t < lo.NT; ++t)
    for (int g = 0; g < kGroups; ++g) {
      const GroupShape &gs = lo.gs[t][g];
      for (int c = 0; c < gs.nchild; ++c)
        n = std::max(n, align256(static_cast<size_t>(gs.K) * gs.rpad[c] * 2));
    }
  return n + ws_w0_expand_bytes(lo);
}

wl_status weightless_materialize(const wl_bundle *bundle, int32_t layer, int32_t family, void *d_weff, void *d_ws,
                                 size_t ws_bytes, void *stream) {
  Resolved rv;
  wl_status st = resolve(bundle, layer, family, -1, rv);
  if (st != WL_OK) return st;
  if (!d_weff || !d_ws) return fail(WL_EINVAL, "w_eff and workspace must be non-NULL");
  if (reinterpret_cast<uintptr_t>(d_weff) % 16) return fail(WL_EINVAL, "w_eff must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(d_ws) % 256) return fail(WL_EINVAL, "workspace must be 256-byte aligned");
  const size_t need = weightless_materialize_workspace_bytes(bundle);
  if (ws_bytes < need) return fail(WL_ENOSPACE, "workspace has %zu bytes, materialize needs %zu", ws_bytes, need);
  const wl::CallDesc &c = rv.c;
  const wl::ChildDesc &ch = c.ch[0];
  const uint8_t *wb = static_cast<const uint8_t *>(d_weff);
  const size_t wbytes = static_cast<size_t>(c.Ntot) * c.K * 2;
  if (wb < bundle->arena + bundle->arena_bytes && bundle->arena < wb + wbytes)
    return fail(WL_EINVAL, "w_eff must not overlap the bundle arena");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t *vrows = static_cast<uint16_t *>(d_ws);
  // V^T [rpad][K] -> V rows [K][rpad] (ranks contiguous), the GEMM's A operand
  hipError_t e = wl::launch_transpose_v(c.Vt, ch.rpad, c.K, vrows, s);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  const uint16_t *w0 = c.W0;
  if (bundle->lo.coded()) {
    uint16_t *buf = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(d_ws) + need - ws_w0_expand_bytes(bundle->lo));
    e = bundle->lo.fp8 ? wl::launch_dequantize_rows(c.W0f8, c.ldw0, c.q, c.Ntot, c.K, buf, s)
                       : wl::launch_dequantize_mxfp4(c.W0f4, 2 * c.ldw0, c.sc4, c.Ntot, c.K, buf, s);
    if (e != hipSuccess) return hip_fail(e, "W0 expand launch");
    w0 = buf;
  }
  e = wl::launch_materialize(vrows, ch.U, c.Ntot, c.K, ch.rpad, c.s, w0, static_cast<uint16_t *>(d_weff),
                             reinterpret_cast<const uint16_t *>(bundle->arena + bundle->lo.zero_off), s);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return WL_OK;
}

int32_t weightless_out_dim(const wl_bundle *bundle, int32_t layer, int32_t family, int32_t stack) {
  Resolved rv;
  if (resolve(bundle, layer, stack >= 0 ? -1 : family, stack >= 0 ? stack : -1, rv) != WL_OK) return 0;
  return rv.out_dim;
}

}  // extern "C"
