"""The oracle's view of a synthetic workload: fp64 bundle parameters and the
expected output of each call.

Directly drawn workloads take W0 per (band, layer type, family) -- MLP families
share one block across layer types, as the mixed-attention adapter groups them
("Decompose HF weights: the mixed-attention case") -- and s, U, V per layer.
Decomposed workloads run ``decompose.decompose_band`` on the seeded per-layer
weights of the band (and layer type) the layer belongs to.  With K=V tying,
v has no bundle and its output is k's.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import forward, quant
from .decompose import band_members, decompose_band

_CALLS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


def to64(t):
    """Exact upcast of a bf16/fp32 torch tensor to a float64 numpy array."""
    return t.detach().to("cpu").float().double().numpy()


class OracleWorkload:
    def __init__(self, wl, device="cpu", cache_w0=4, w0_format="bf16"):
        """w0_format "fp8": the bundle stands for W0 coded per row in E4M3
        with a power-of-two scale (oracle.quant); every W0 the oracle uses is
        that dequantized block."""
        self.wl = wl
        self.device = device
        self._dec = {}
        self._w0 = {}
        self._cache_w0 = cache_w0
        self.w0_format = w0_format

    def w0(self, band, ltype, fam):
        key = (band, ltype if fam in ("q", "k", "v", "o") else 0, fam)
        if key not in self._w0:
            if len(self._w0) >= self._cache_w0:
                self._w0.pop(next(iter(self._w0)))
            w = to64(self.wl.w0(band, ltype, fam, self.device))
            if self.w0_format == "fp8":
                w = quant.dequantize(*quant.quantize_rows(w))
            self._w0[key] = w
        return self._w0[key]

    def prefetch_decompositions(self, keys, workers=8):
        """Decompose several (band, layer type, family) groups concurrently.
        Each decomposition is the same sequential computation as
        ``decomposed_band``; only the scheduling is parallel (LAPACK releases
        the GIL; each thread's BLAS is limited to one core)."""
        todo = [k for k in keys if k not in self._dec]
        if not todo:
            return
        wl = self.wl
        inputs = {}
        for (b, t, f) in todo:
            members = [l for l in band_members(b, wl.num_layers, wl.num_bands) if wl.layer_types[l] == t]
            inputs[(b, t, f)] = (members, [to64(wl.layer_weight(l, f, self.device)) for l in members])

        def work(key):
            members, Ws = inputs[key]
            W0, res = decompose_band(Ws, wl.rank, store=True)
            return key, (W0, dict(zip(members, res)))

        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except Exception:  # pragma: no cover
            limiter = None
        try:
            with ThreadPoolExecutor(workers) as ex:
                for key, val in ex.map(work, todo):
                    self._dec[key] = val
        finally:
            if limiter is not None:
                limiter.restore_original_limits()

    def _tied(self, layer, fam):
        return fam == "v" and self.wl.layer_types[layer] in self.wl.k_eq_v_types

    def decomposed_band(self, band, ltype, fam):
        key = (band, ltype, fam)
        if key not in self._dec:
            wl = self.wl
            members = [l for l in band_members(band, wl.num_layers, wl.num_bands)
                       if wl.layer_types[l] == ltype]
            Ws = [to64(wl.layer_weight(l, fam, self.device)) for l in members]
            W0, res = decompose_band(Ws, wl.rank, store=True)
            self._dec[key] = (W0, dict(zip(members, res)))
        return self._dec[key]

    def params(self, layer, fam):
        """(W0, s, U, V) as fp64 arrays for one layer and family."""
        wl = self.wl
        if self._tied(layer, fam):
            fam = "k"
        lt = wl.layer_types[layer]
        if wl.decomposed:
            W0, per = self.decomposed_band(wl.band(layer), lt, fam)
            m = per[layer]
            return W0, m["s"], m["U"], m["V"]
        return (self.w0(wl.band(layer), lt, fam), to64(wl.s(layer, fam, self.device)),
                to64(wl.u(layer, fam, self.device)), to64(wl.v(layer, fam, self.device)))

    def families_of(self, layer, call):
        fams = _CALLS.get(call, (call,))
        lt = self.wl.layer_types[layer]
        return [f for f in fams if (lt, f) in self.wl.dims or self._tied(layer, f)]

    def call(self, layer, call, x):
        """Expected fp64 output of a single-family or stacked call."""
        x = np.asarray(x, np.float64)
        children = []
        for f in self.families_of(layer, call):
            children.append("dup" if self._tied(layer, f) else self.params(layer, f))
        return forward.stacked(x, children)

    def gate_up_act(self, layer, x, name):
        """Expected fp64 h = act(gate) * up of one layer's gate|up stack."""
        return forward.gate_up_act(np.asarray(x, np.float64), self.params(layer, "gate"),
                                   self.params(layer, "up"), name)
