"""The oracle's view of a synthetic workload: fp64 bundle parameters and the
expected output of each call.

Directly drawn workloads take W0 per (band, layer type, family) -- MLP families
share one block across layer types, as the mixed-attention adapter groups them
("Decompose HF weights: the mixed-attention case") -- and s, U, V per layer.
Decomposed workloads run ``decompose.decompose_band`` on the seeded per-layer
weights of the band (and layer type) the layer belongs to.  With K=V tying,
v has no bundle and its output is k's.
"""
import numpy as np

from . import forward
from .decompose import band_members, decompose_band

_CALLS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


def to64(t):
    """Exact upcast of a bf16/fp32 torch tensor to a float64 numpy array."""
    return t.detach().to("cpu").float().double().numpy()


class OracleWorkload:
    def __init__(self, wl, device="cpu"):
        self.wl = wl
        self.device = device
        self._dec = {}

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
        return (to64(wl.w0(wl.band(layer), lt, fam, self.device)), to64(wl.s(layer, fam, self.device)),
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
