"""The oracle's view of a synthetic workload: fp64 bundle parameters and the
expected output of each call.  Test infrastructure: only the tests, the smoke
check and the benchmark's CPU baseline use it; the HIP library never does.

Which bundle a call uses is decided here, from the workload's shape alone
(its layer count, band count, layer types and K=V-tied types), never from the
input generator:

  * bands: layer l sits in band floor(l G / L) (``decompose.band_of``:
    contiguous, balanced bands; "Quality (Gemma 4 31B)" page, "Decomposition
    quality": 5 bands of 12 layers over 60);
  * shared blocks: the attention families (q, k, v, o) keep one W0 per
    (band, layer type, family); the MLP families (gate, up, down) keep one W0
    per (band, family), shared by every layer type of the band ("Add a new
    model architecture" page, "Decompose HF weights: the mixed-attention
    case");
  * K=V tying: on a tied layer type v has no bundle and its output is k's
    output ("Decompose HF weights: the mixed-attention case",
    attention_k_eq_v).

Directly drawn workloads take W0 under that key from the generator and s, U, V
per layer.  Decomposed workloads run ``decompose.decompose_band`` over the
member layers of the W0 group (all layers of the band for an MLP family; the
band's layers of one type for an attention family).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import forward, quant
from .decompose import band_of, decompose_band

ATTENTION_FAMILIES = ("q", "k", "v", "o")
_CALLS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


def to64(t):
    """Exact upcast of a bf16/fp32 torch tensor to a float64 numpy array."""
    return t.detach().to("cpu").float().double().numpy()


def w0_key(band, ltype, fam):
    """The W0 group of a family of a layer type in a band: (band, type key,
    family), the type key being the layer type for attention families and 0
    (one block for every type) for MLP families."""
    return (band, ltype if fam in ATTENTION_FAMILIES else 0, fam)


class OracleWorkload:
    def __init__(self, wl, device="cpu", cache_w0=4, w0_format="bf16"):
        """w0_format "fp8": the bundle stands for W0 coded per row in E4M3
        with a power-of-two scale; "mxfp4": W0 coded in E2M1 with one E8M0
        scale per 32 elements (oracle.quant); every W0 the oracle uses is
        that dequantized block."""
        self.wl = wl
        self.device = device
        self._dec = {}
        self._w0 = {}
        self._cache_w0 = cache_w0
        self.w0_format = w0_format

    # ---- resolution ------------------------------------------------------
    def band(self, layer):
        return band_of(layer, self.wl.num_layers, self.wl.num_bands)

    def tied(self, layer, fam):
        """v of a layer whose type ties v to k."""
        return fam == "v" and self.wl.layer_types[layer] in self.wl.k_eq_v_types

    def group_members(self, band, ltype, fam):
        """Layers whose ``fam`` bundle uses the W0 of (band, ltype): those
        with the same W0 key (every layer of the band for an MLP family, the
        band's layers of type ltype for an attention family)."""
        wl = self.wl
        key = w0_key(band, ltype, fam)
        return [l for l in range(wl.num_layers) if w0_key(self.band(l), wl.layer_types[l], fam) == key]

    # ---- parameters ------------------------------------------------------
    def w0(self, band, ltype, fam):
        """Directly drawn workloads: the shared block of (band, ltype, fam)."""
        key = w0_key(band, ltype, fam)
        if key not in self._w0:
            if len(self._w0) >= self._cache_w0:
                self._w0.pop(next(iter(self._w0)))
            w = to64(self.wl.w0(key[0], key[1], fam, self.device))
            if self.w0_format == "fp8":
                w = quant.dequantize(*quant.quantize_rows(w))
            elif self.w0_format == "mxfp4":
                w = quant.dequantize_mxfp4(*quant.quantize_mxfp4(w), w.shape[1])
            self._w0[key] = w
        return self._w0[key]

    def _decompose_group(self, key):
        band, key_type, fam = key
        members = self.group_members(band, key_type, fam)
        Ws = [to64(self.wl.layer_weight(l, fam, self.device)) for l in members]
        W0, res = decompose_band(Ws, self.wl.rank, store=True)
        return W0, dict(zip(members, res))

    def prefetch_decompositions(self, keys, workers=8):
        """Decompose several (band, layer type, family) groups concurrently.
        Each decomposition is the same sequential computation as
        ``decomposed_band``; only the scheduling is parallel (LAPACK releases
        the GIL; each thread's BLAS is limited to one core)."""
        todo = sorted({w0_key(*k) for k in keys} - set(self._dec))
        if not todo:
            return
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except Exception:  # pragma: no cover
            limiter = None
        try:
            with ThreadPoolExecutor(workers) as ex:
                for key, val in zip(todo, ex.map(self._decompose_group, todo)):
                    self._dec[key] = val
        finally:
            if limiter is not None:
                limiter.restore_original_limits()

    def decomposed_band(self, band, ltype, fam):
        """Decomposed workloads: (W0, {layer: {"s", "U", "V", ...}}) of the W0
        group that (band, ltype, fam) belongs to."""
        key = w0_key(band, ltype, fam)
        if key not in self._dec:
            self._dec[key] = self._decompose_group(key)
        return self._dec[key]

    def params(self, layer, fam):
        """(W0, s, U, V) as fp64 arrays for one layer and family (k's bundle
        for v on a tied layer type)."""
        wl = self.wl
        if self.tied(layer, fam):
            fam = "k"
        lt = wl.layer_types[layer]
        band = self.band(layer)
        if wl.decomposed:
            W0, per = self.decomposed_band(band, lt, fam)
            m = per[layer]
            return W0, m["s"], m["U"], m["V"]
        return (self.w0(band, lt, fam), to64(wl.s(layer, fam, self.device)),
                to64(wl.u(layer, fam, self.device)), to64(wl.v(layer, fam, self.device)))

    def families_of(self, layer, call):
        """The families a call evaluates on this layer, in output order (a
        tied v stays: its slot repeats k)."""
        fams = _CALLS.get(call, (call,))
        lt = self.wl.layer_types[layer]
        return [f for f in fams if (lt, f) in self.wl.dims or self.tied(layer, f)]

    def call(self, layer, call, x):
        """Expected fp64 output of a single-family or stacked call."""
        x = np.asarray(x, np.float64)
        fams = self.families_of(layer, call)
        if len(fams) == 1:
            return forward.factored(x, *self.params(layer, fams[0]))
        children = ["dup" if self.tied(layer, f) else self.params(layer, f) for f in fams]
        return forward.stacked(x, children)

    def gate_up_act(self, layer, x, name):
        """Expected fp64 h = act(gate) * up of one layer's gate|up stack."""
        return forward.gate_up_act(np.asarray(x, np.float64), self.params(layer, "gate"),
                                   self.params(layer, "up"), name)
