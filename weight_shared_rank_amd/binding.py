"""ctypes binding of the C ABI in include/weightless.h.

Argument marshalling only: every step of the weightless linear runs in the
HIP library.  torch supplies device memory (arena, workspace, x, y) and the
current HIP stream.  There is no fallback: if libweightless.so is missing or
fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "libweightless.so")

FAMILIES = ("q", "k", "v", "o", "gate", "up", "down")
FAMILY = {f: i for i, f in enumerate(FAMILIES)}
STACKS = {"qkv": 0, "gate_up": 1}
ACTS = {"gelu_tanh": 0, "silu": 1, "gelu": 2}
W0_FORMATS = {"bf16": 0, "fp8": 1, "mxfp4": 2}
WL_DTYPE_BF16, WL_DTYPE_F32 = 0, 1
WL_SRC_W0, WL_SRC_S, WL_SRC_U, WL_SRC_V = 0, 1, 2, 3
SRC_KIND = {"w0": WL_SRC_W0, "s": WL_SRC_S, "u": WL_SRC_U, "v": WL_SRC_V}
STATUS = {0: "WL_OK", -1: "WL_EINVAL", -2: "WL_ESHAPE", -3: "WL_EDTYPE", -4: "WL_ERANGE",
          -5: "WL_ENOSPACE", -6: "WL_EHIP"}
MAX_TYPES = 2
DECODE_MAX_T = 16
NOALLOC_WORKSPACE_BYTES = 64 << 20    # WL_NOALLOC_WORKSPACE_BYTES

# every symbol include/weightless.h declares
EXPORTS = ("theta_bundle_arena_bytes", "theta_bundle_load", "theta_bundle_free",
           "weightless_workspace_bytes",
           "weightless_linear", "weightless_linear_noalloc", "weightless_stacked_linear", "weightless_out_dim", "wl_last_error",
           "weightless_materialize_workspace_bytes", "weightless_materialize", "weightless_gate_up_act",
           "weightless_decompose_workspace_bytes", "weightless_decompose",
           "weightless_decompose_als_workspace_bytes", "weightless_decompose_als")


class WlBundleSpec(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_bands", ctypes.c_int32),
                ("num_layer_types", ctypes.c_int32), ("layer_type", ctypes.POINTER(ctypes.c_int8)),
                ("out_dim", (ctypes.c_int32 * 7) * MAX_TYPES), ("in_dim", (ctypes.c_int32 * 7) * MAX_TYPES),
                ("rank", (ctypes.c_int32 * 7) * MAX_TYPES), ("k_eq_v_type_mask", ctypes.c_uint32),
                ("w0_format", ctypes.c_int32)]


class WlSrc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("index", ctypes.c_int32), ("layer_type", ctypes.c_int32),
                ("family", ctypes.c_int32), ("dtype", ctypes.c_int32), ("on_device", ctypes.c_int32),
                ("ptr", ctypes.c_void_p)]


class WlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """Load libweightless.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise RuntimeError(f"{LIBPATH} is not built; run `python -m weight_shared_rank_amd.build`")
    # torch's HIP runtime must be the process's only one: loaded first, it
    # satisfies the library's libamdhip64 dependency.  Loaded the other way
    # round, the library pulls in the system runtime beside torch's, and that
    # second runtime finds no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIBPATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "theta_bundle_arena_bytes": (sz, [ctypes.POINTER(WlBundleSpec)]),
        "theta_bundle_load": (i32, [ctypes.POINTER(WlBundleSpec), ctypes.POINTER(WlSrc), sz, vp, sz, vp,
                                    ctypes.POINTER(vp)]),
        "theta_bundle_free": (i32, [vp]),
        "weightless_workspace_bytes": (sz, [vp, i32]),
        "weightless_linear": (i32, [vp, i32, i32, vp, i32, vp, vp, sz, vp]),
        "weightless_linear_noalloc": (i32, [vp, i32, i32, vp, i32, vp, vp]),
        "weightless_stacked_linear": (i32, [vp, i32, i32, vp, i32, vp, vp, sz, vp]),
        "weightless_out_dim": (i32, [vp, i32, i32, i32]),
        "wl_last_error": (ctypes.c_char_p, []),
        "weightless_materialize_workspace_bytes": (sz, [vp]),
        "weightless_materialize": (i32, [vp, i32, i32, vp, vp, sz, vp]),
        "weightless_gate_up_act": (i32, [vp, i32, i32, vp, i32, vp, vp, sz, vp]),
        "weightless_decompose_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "weightless_decompose": (i32, [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "weightless_decompose_als_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "weightless_decompose_als": (i32, [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().wl_last_error().decode()


def _check(st: int):
    if st != 0:
        raise WlError(st, last_error())


def make_spec(num_layers: int, num_bands: int, dims: Dict[Tuple[int, str], Tuple[int, int]],
              ranks: Dict[Tuple[int, str], int], layer_types: Optional[Sequence[int]] = None,
              k_eq_v_types: Iterable[int] = (), w0_format: str = "bf16") -> WlBundleSpec:
    """Spec from Python dicts: dims[(type, family)] = (N, K), ranks[(type, family)] = r;
    w0_format "bf16" or "fp8" (E4M3 codes with a power-of-two scale per W0 row)."""
    sp = WlBundleSpec()
    sp.num_layers = num_layers
    sp.num_bands = num_bands
    nt = (max(layer_types) + 1) if layer_types else 1
    nt = max(nt, max([t for t, _ in dims] + [0]) + 1)
    sp.num_layer_types = nt
    if layer_types is not None:
        arr = (ctypes.c_int8 * len(layer_types))(*layer_types)
        sp.layer_type = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int8))
        sp._keep = arr  # keep the array alive with the struct
    for (t, f), (n, k) in dims.items():
        sp.out_dim[t][FAMILY[f]] = n
        sp.in_dim[t][FAMILY[f]] = k
        sp.rank[t][FAMILY[f]] = ranks.get((t, f), 0)
    mask = 0
    for t in k_eq_v_types:
        mask |= 1 << t
    sp.k_eq_v_type_mask = mask
    sp.w0_format = W0_FORMATS[w0_format]
    return sp


def _stream_ptr(stream) -> ctypes.c_void_p:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def theta_bundle_arena_bytes(spec: WlBundleSpec) -> int:
    n = lib().theta_bundle_arena_bytes(ctypes.byref(spec))
    if n == 0:
        raise WlError(-1, last_error())
    return n


class ThetaBundle:
    """A theta bundle resident in a torch-allocated device arena."""

    def __init__(self, spec: WlBundleSpec, sources, device="cuda", stream=None, arena=None):
        """sources: iterable of (kind, index, layer_type, family, tensor) with
        kind in {"w0", "s", "u", "v"}; tensors may live on the host or the
        device (bf16 for w0/u/v, float32 for s, contiguous)."""
        import torch
        self.spec = spec
        need = theta_bundle_arena_bytes(spec)
        self.arena = arena if arena is not None else torch.empty(need, dtype=torch.uint8, device=device)
        if self.arena.numel() < need:
            raise WlError(-5, f"arena has {self.arena.numel()} bytes, bundle needs {need}")
        keep = []
        srcs = (WlSrc * max(1, len(sources)))()
        for i, (kind, index, ltype, fam, t) in enumerate(sources):
            if not t.is_contiguous():
                t = t.contiguous()
            keep.append(t)
            srcs[i].kind = SRC_KIND[kind]
            srcs[i].index = index
            srcs[i].layer_type = ltype
            srcs[i].family = FAMILY[fam]
            srcs[i].dtype = WL_DTYPE_F32 if t.dtype == torch.float32 else (WL_DTYPE_BF16 if t.dtype == torch.bfloat16 else 99)
            srcs[i].on_device = 1 if t.is_cuda else 0
            srcs[i].ptr = t.data_ptr()
        h = ctypes.c_void_p()
        _check(lib().theta_bundle_load(ctypes.byref(spec), srcs, len(sources), self.arena.data_ptr(),
                                       self.arena.numel(), _stream_ptr(stream), ctypes.byref(h)))
        self.handle = h
        self._keep_until_sync = keep
        # the load is asynchronous: the handle (which owns the host-side V^T
        # copies) is freed only once the stream has passed this event
        self._loaded = torch.cuda.Event()
        self._loaded.record(stream if stream is not None else torch.cuda.current_stream())
        self._ws = {}

    def close(self):
        if getattr(self, "handle", None):
            self._loaded.synchronize()
            lib().theta_bundle_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def out_dim(self, layer: int, family: Optional[str] = None, stack: Optional[str] = None) -> int:
        n = lib().weightless_out_dim(self.handle, layer, FAMILY[family] if family else -1,
                                     STACKS[stack] if stack else -1)
        if n == 0:
            raise WlError(-4, last_error())
        return n

    def workspace_bytes(self, T: int) -> int:
        n = lib().weightless_workspace_bytes(self.handle, T)
        if n == 0:
            raise WlError(-1, last_error())
        return n

    def workspace(self, T: int, stream=None):
        """A workspace large enough for T tokens."""
        import torch
        return torch.empty(self.workspace_bytes(T), dtype=torch.uint8, device=self.arena.device)

    def _ws_for(self, T, stream):
        need = self.workspace_bytes(T)
        key = "prefill" if T > DECODE_MAX_T else "decode"
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            ws = self.workspace(T, stream)
            self._ws[key] = ws
        return ws

    def _call(self, fn, layer, code, x, y, ws, stream, width):
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, width), dtype=torch.bfloat16, device=x.device)
        if ws is None:
            ws = self._ws_for(T, stream)
        _check(fn(self.handle, layer, code, x.data_ptr(), T, y.data_ptr(), ws.data_ptr(), ws.numel(),
                  _stream_ptr(stream)))
        return y

    def linear(self, layer: int, family: str, x, y=None, ws=None, stream=None):
        """y = s*(W0 x) + U (V^T x) for one family; x bf16 [T, K] on the device."""
        return self._call(lib().weightless_linear, layer, FAMILY[family], x, y, ws, stream,
                          self.out_dim(layer, family=family))

    def linear_noalloc(self, layer: int, family: str, x, y=None, stream=None):
        """weightless_linear on the library's fixed device workspace (no
        caller workspace); y is allocated here only if not given."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.out_dim(layer, family=family)), dtype=torch.bfloat16, device=x.device)
        _check(lib().weightless_linear_noalloc(self.handle, layer, FAMILY[family], x.data_ptr(), T, y.data_ptr(),
                                               _stream_ptr(stream)))
        return y

    def stacked(self, layer: int, stack: str, x, y=None, ws=None, stream=None):
        """The stacked q|k|v or gate|up call over one x."""
        return self._call(lib().weightless_stacked_linear, layer, STACKS[stack], x, y, ws, stream,
                          self.out_dim(layer, stack=stack))

    def gate_up_act(self, layer: int, act: str, x, h=None, ws=None, stream=None):
        """h = act(gate) * up of one layer's gate|up stack, bf16 [T, N_gate]."""
        return self._call(lambda hd, l, code, *rest: lib().weightless_gate_up_act(hd, l, ACTS[act], *rest),
                          layer, 0, x, h, ws, stream, self.out_dim(layer, family="gate"))

    def in_dim(self, layer: int, family: str) -> int:
        """K of one family of one layer (from the spec)."""
        t = self.spec.layer_type[layer] if self.spec.layer_type else 0
        f = FAMILY[family]
        if family == "v" and (self.spec.k_eq_v_type_mask >> t) & 1:
            f = FAMILY["k"]
        return self.spec.in_dim[t][f]

    def materialize(self, layer: int, family: str, out=None, ws=None, stream=None):
        """W_eff = diag(s) W0 + U V^T of one family, bf16 [N, K] on the device."""
        import torch
        n, k = self.out_dim(layer, family=family), self.in_dim(layer, family)
        if out is None:
            out = torch.empty((n, k), dtype=torch.bfloat16, device=self.arena.device)
        if ws is None:
            need = lib().weightless_materialize_workspace_bytes(self.handle)
            if need == 0:
                raise WlError(-1, last_error())
            ws = torch.empty(need, dtype=torch.uint8, device=self.arena.device)
        _check(lib().weightless_materialize(self.handle, layer, FAMILY[family], out.data_ptr(), ws.data_ptr(),
                                            ws.numel(), _stream_ptr(stream)))
        return out


def sketch_columns(N: int, K: int, rank: int, oversample: int) -> int:
    """Columns l of the test matrix weightless_decompose takes: min(rank + oversample, N, K)."""
    return min(rank + oversample, N, K)


def decompose(w, rank: int, omega=None, oversample: int = 16, power_iters: int = 4, stream=None,
              als_sweeps: int = None):
    """Decompose one band of one family on the GPU.

    w: bf16 [m, N, K] device tensor (the band's layers in layer order);
    omega: fp32 [K, l] device test matrix, l = sketch_columns(N, K, rank, oversample)
    (required when rank > 0).  als_sweeps: None calls weightless_decompose;
    an integer calls weightless_decompose_als with that many ALS sweeps.
    Returns (W0 bf16 [N, K], s fp32 [m, N], U bf16 [m, N, rank], V bf16
    [m, K, rank]), the layouts theta_bundle_load takes."""
    import torch
    if w.dim() != 3 or w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous():
        raise WlError(-1, "w must be a contiguous bf16 [m, N, K] device tensor")
    m, n, k = w.shape
    dev = w.device
    l = sketch_columns(n, k, rank, oversample)
    if rank > 0:
        if omega is None or tuple(omega.shape) != (k, l) or omega.dtype != torch.float32 \
                or not omega.is_contiguous() or omega.device != dev:
            raise WlError(-1, f"omega must be a contiguous fp32 [{k}, {l}] tensor on {dev}")
    als = als_sweeps is not None
    need = (lib().weightless_decompose_als_workspace_bytes if als else lib().weightless_decompose_workspace_bytes)(
        n, k, rank, oversample)
    if need == 0:
        raise WlError(-1, "decomposition workspace size: arguments out of range")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    w0 = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
    s = torch.empty((m, n), dtype=torch.float32, device=dev)
    u = torch.empty((m, n, rank), dtype=torch.bfloat16, device=dev)
    v = torch.empty((m, k, rank), dtype=torch.bfloat16, device=dev)
    lead = (w.data_ptr(), m, n, k, rank, oversample, power_iters) + ((als_sweeps,) if als else ())
    fn = lib().weightless_decompose_als if als else lib().weightless_decompose
    _check(fn(*lead, omega.data_ptr() if rank > 0 else None, w0.data_ptr(), s.data_ptr(),
              u.data_ptr() if rank > 0 else None, v.data_ptr() if rank > 0 else None,
              ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    return w0, s, u, v
