"""Deliver a synthetic workload's theta bundle to the GPU library.

Maps a ``synth.Workload`` to a bundle spec and a list of source tensors.  It
only arranges tensors the generator draws (or tensors the caller passes in);
it computes nothing of the method.
"""
from __future__ import annotations

from typing import Callable, Optional

from weight_shared_rank_amd import binding


def band_of_layer(layer: int, num_layers: int, num_bands: int) -> int:
    """The library's band of a layer, floor(l G / L) (the rule its header
    states), used here only to list the W0 sources a bundle must be given."""
    return (layer * num_bands) // num_layers


def spec_of(wl, w0_format="bf16") -> binding.WlBundleSpec:
    ranks = {key: min(wl.rank, *wl.dims[key]) for key in wl.dims}
    return binding.make_spec(wl.num_layers, wl.num_bands, dict(wl.dims), ranks,
                             list(wl.layer_types), wl.k_eq_v_types, w0_format=w0_format)


def sources_of(wl, device="cuda", tensors: Optional[Callable] = None, layers=None):
    """Source list for ThetaBundle.  ``tensors(kind, index, ltype, fam)`` may
    supply the tensors (decomposed workloads); by default they are drawn from
    the workload's seeded streams on ``device``."""
    if tensors is None:
        def tensors(kind, index, ltype, fam):
            if kind == "w0":
                return wl.w0(index, ltype, fam, device)
            return getattr(wl, kind)(index, fam, device)
    srcs = []
    for b in range(wl.num_bands):
        for t in range(wl.num_layer_types):
            members = [l for l in range(wl.num_layers) if band_of_layer(l, wl.num_layers, wl.num_bands) == b]
            for fam in wl.families(t):
                if not wl.has(t, fam):
                    continue
                mlp = fam in ("gate", "up", "down")
                if mlp and t != 0:
                    continue
                if not any(mlp or wl.layer_types[l] == t for l in members):
                    continue
                srcs.append(("w0", b, t if not mlp else 0, fam, tensors("w0", b, t, fam)))
    for l in range(wl.num_layers):
        t = wl.layer_types[l]
        for fam in wl.families(t):
            if not wl.has(t, fam):
                continue
            srcs.append(("s", l, 0, fam, tensors("s", l, t, fam)))
            if wl.clamped_rank(t, fam) > 0:
                srcs.append(("u", l, 0, fam, tensors("u", l, t, fam)))
                srcs.append(("v", l, 0, fam, tensors("v", l, t, fam)))
    return srcs


def load(wl, device="cuda", tensors=None, stream=None, w0_format="bf16") -> binding.ThetaBundle:
    return binding.ThetaBundle(spec_of(wl, w0_format), sources_of(wl, device, tensors), device=device,
                               stream=stream)
