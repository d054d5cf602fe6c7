"""Seeded synthetic workloads for the weightless linear.

This module only draws random tensors and describes workload shapes.  It holds
none of the method's arithmetic (no band means, no scaling, no products): both
the GPU path and the CPU oracle take their inputs from here, and nothing else
is shared between them.

Shapes follow the two model families the pages measure on ("Quality" page for
Gemma 3 1B and "Quality (Gemma 4 31B)" page, section "Architecture and weight
shapes"; the theta-bundle section of the "Compression" page gives the Gemma 3
1B dimensions: 26 layers, hidden 1152, head_dim 256, intermediate 4096).  The
real checkpoints are not available, so every tensor is drawn from a seeded
normal distribution with the variance a trained weight of that fan-in would
roughly have.

Seeding: every tensor has its own stream, keyed by
(root seed, tensor kind, layer-or-band, layer type, family), so any single
tensor can be regenerated without drawing the others.  Draws are fp32 normals
from torch's generator on the requested device (Philox on a GPU, mt19937 on
the CPU), then rounded to bfloat16 (round-to-nearest-even) where the tensor is
stored as bf16.  The same device and seed always give the same bytes.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import torch

FAMILIES = ("q", "k", "v", "o", "gate", "up", "down")
FAM_ID = {f: i for i, f in enumerate(FAMILIES)}
ATTN_FAMILIES = ("q", "k", "v", "o")
MLP_FAMILIES = ("gate", "up", "down")

# Calls a decoder layer makes, in order: (call name, families in output order).
CALLS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))

_KIND = {"w0": 1, "s": 2, "u": 3, "v": 4, "x": 5, "layer_w": 6, "band_w": 7, "sketch": 8}


def _seed(root: int, kind: str, index: int, ltype: int, fam: int, extra: int = 0) -> int:
    """63-bit seed from the tensor's key (sha256 of the key tuple)."""
    key = f"{root}/{_KIND[kind]}/{index}/{ltype}/{fam}/{extra}".encode()
    return int.from_bytes(hashlib.sha256(key).digest()[:8], "little") & ((1 << 63) - 1)


def _normal(shape, seed: int, mean: float, std: float, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: model shape, sharing setting and token count."""

    cid: int
    name: str
    num_layers: int
    num_bands: int
    rank: int
    tokens: Tuple[int, ...]
    # dims[(layer_type, family)] = (out_dim N, in_dim K); a missing key means absent.
    dims: Dict[Tuple[int, str], Tuple[int, int]]
    layer_types: Tuple[int, ...]
    k_eq_v_types: Tuple[int, ...] = ()
    x_std: float = 1.0
    # True: s/U/V and W0 come from decomposing seeded layer weights (the oracle
    # does that); False: the bundle is drawn directly.
    decomposed: bool = False

    @property
    def root(self) -> int:
        return 1000 + self.cid

    @property
    def num_layer_types(self) -> int:
        return max(self.layer_types) + 1

    def families(self, ltype: int):
        return [f for f in FAMILIES if (ltype, f) in self.dims]

    def has(self, ltype: int, fam: str) -> bool:
        if fam == "v" and ltype in self.k_eq_v_types:
            return False
        return (ltype, fam) in self.dims

    def shape(self, ltype: int, fam: str) -> Tuple[int, int]:
        if fam == "v" and ltype in self.k_eq_v_types:
            fam = "k"
        return self.dims[(ltype, fam)]

    def clamped_rank(self, ltype: int, fam: str) -> int:
        n, k = self.shape(ltype, fam)
        return min(self.rank, n, k)

    # ---- tensors -------------------------------------------------------
    def w0(self, index: int, key_type: int, fam: str, device="cpu") -> torch.Tensor:
        """A directly drawn shared block, N(0, 1/in) in bf16, with the shape
        of ``fam`` on layer type ``key_type``; its stream is keyed by
        (index, key_type, family) exactly as given.  Which blocks a bundle
        holds, and which layers use each, is the caller's business."""
        n, k = self.shape(key_type, fam)
        return _normal((n, k), _seed(self.root, "w0", index, key_type, FAM_ID[fam]),
                       0.0, 1.0 / math.sqrt(k), device).to(torch.bfloat16)

    def s(self, layer: int, fam: str, device="cpu") -> torch.Tensor:
        n, _ = self.shape(self.layer_types[layer], fam)
        return _normal((n,), _seed(self.root, "s", layer, 0, FAM_ID[fam]), 1.0, 0.05, device)

    def u(self, layer: int, fam: str, device="cpu") -> torch.Tensor:
        lt = self.layer_types[layer]
        n, _ = self.shape(lt, fam)
        r = self.clamped_rank(lt, fam)
        return _normal((n, r), _seed(self.root, "u", layer, 0, FAM_ID[fam]), 0.0, 0.02,
                       device).to(torch.bfloat16)

    def v(self, layer: int, fam: str, device="cpu") -> torch.Tensor:
        lt = self.layer_types[layer]
        _, k = self.shape(lt, fam)
        r = self.clamped_rank(lt, fam)
        return _normal((k, r), _seed(self.root, "v", layer, 0, FAM_ID[fam]), 0.0, 0.02,
                       device).to(torch.bfloat16)

    def layer_weight(self, layer: int, fam: str, device="cpu") -> torch.Tensor:
        """A dense per-layer projection weight, N(0, 1/in) in bf16; the input
        of the decomposition for decomposed workloads."""
        n, k = self.shape(self.layer_types[layer], fam)
        return _normal((n, k), _seed(self.root, "layer_w", layer, 0, FAM_ID[fam]),
                       0.0, 1.0 / math.sqrt(k), device).to(torch.bfloat16)

    def x(self, layer: int, call: str, T: int, device="cpu", salt: int = 0) -> torch.Tensor:
        """Activations for one call: [T, K] bf16."""
        fams = dict(CALLS)[call] if call in dict(CALLS) else (call,)
        lt = self.layer_types[layer]
        _, k = self.shape(lt, fams[0])
        call_id = [c for c, _ in CALLS].index(call) if call in dict(CALLS) else 10 + FAM_ID[call]
        return _normal((T, k), _seed(self.root, "x", layer, call_id, T, salt), 0.0,
                       self.x_std, device).to(torch.bfloat16)


def _gemma3_dims():
    h, q, kv, inter = 1152, 1024, 256, 4096
    return {(0, "q"): (q, h), (0, "k"): (kv, h), (0, "v"): (kv, h), (0, "o"): (h, q),
            (0, "gate"): (inter, h), (0, "up"): (inter, h), (0, "down"): (h, inter)}


def _gemma4_sliding_dims(t: int):
    h, q, kv, inter = 5376, 8192, 4096, 21504
    return {(t, "q"): (q, h), (t, "k"): (kv, h), (t, "v"): (kv, h), (t, "o"): (h, q),
            (t, "gate"): (inter, h), (t, "up"): (inter, h), (t, "down"): (h, inter)}


def _gemma4_mixed_dims():
    d = _gemma4_sliding_dims(0)
    h, inter = 5376, 21504
    d.update({(1, "q"): (16384, h), (1, "k"): (8192, h), (1, "o"): (h, 16384),
              (1, "gate"): (inter, h), (1, "up"): (inter, h), (1, "down"): (h, inter)})
    return d


def workload(cid: int, variant: Optional[str] = None) -> Workload:
    """The five measured workloads (1-based id).  variant="passthrough" on
    workload 2 gives one band per layer (G = L)."""
    if cid == 1:
        return Workload(1, "one-family 4096x1152 r4 T4 (2 layers, 1 band)", 2, 1, 4, (4,),
                        {(0, "up"): (4096, 1152)}, (0, 0), x_std=1.0 / math.sqrt(1152))
    if cid == 2:
        g = 26 if variant == "passthrough" else 13
        return Workload(2, f"gemma3-1b decode G{g} r32 T1", 26, g, 32, (1,), _gemma3_dims(),
                        (0,) * 26, decomposed=True)
    if cid == 3:
        return Workload(3, "gemma3-1b prefill G1 r64 T2048", 26, 1, 64, (2048,), _gemma3_dims(),
                        (0,) * 26)
    if cid == 4:
        return Workload(4, "gemma4-31b sliding decode G5 r256 T1/T16", 60, 5, 256, (1, 16),
                        _gemma4_sliding_dims(0), (0,) * 60)
    if cid == 5:
        types = tuple(1 if l % 6 == 5 else 0 for l in range(60))
        return Workload(5, "gemma4-31b mixed prefill G1/type r1024 T512", 60, 1, 1024, (512,),
                        _gemma4_mixed_dims(), types, k_eq_v_types=(1,))
    raise ValueError(f"no workload {cid}")


def custom(num_layers: int, num_bands: int, rank: int, dims, layer_types=None,
           k_eq_v_types=(), x_std=1.0, cid: int = 99) -> Workload:
    """A small ad-hoc workload (edge-case tests)."""
    lt = tuple(layer_types) if layer_types is not None else (0,) * num_layers
    return Workload(cid, "custom", num_layers, num_bands, rank, (1,), dict(dims), lt,
                    tuple(k_eq_v_types), x_std=x_std)


def band_layers(seed: int, m: int, N: int, K: int, planted_rank: int = 0, planted_std: float = 1.0,
                device="cpu") -> torch.Tensor:
    """Per-layer weights of one band, bf16 [m, N, K]: the input of a
    decomposition.  planted_rank == 0: each layer i.i.d. N(0, 1/K), the
    distribution the oracle workloads decompose.  planted_rank = p > 0: a
    block B shared by all layers plus, per layer, a rank-p part P_l Q_l^T
    (P ~ N(0, planted_std^2 / K), Q ~ N(0, 1), so its entries are about
    planted_std * sqrt(p / K)) and no other per-layer term; the layers then
    differ from their mean by a matrix of rank <= m p, a spectrum with a gap.
    The planted product is how the input is drawn, not a step of the method."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(seed, "band_w", m, N, K, planted_rank))
    std = 1.0 / math.sqrt(K)
    if planted_rank == 0:
        w = torch.randn((m, N, K), generator=g, dtype=torch.float32) * std
    else:
        base = torch.randn((N, K), generator=g, dtype=torch.float32) * std
        P = torch.randn((m, N, planted_rank), generator=g, dtype=torch.float32) * (planted_std * std)
        Q = torch.randn((m, K, planted_rank), generator=g, dtype=torch.float32)
        w = base.unsqueeze(0) + torch.bmm(P, Q.transpose(1, 2).contiguous())
    return w.to(torch.bfloat16).to(device)


def sketch_matrix(seed: int, K: int, cols: int, device="cpu") -> torch.Tensor:
    """Standard normal fp32 [K, cols] test matrix for a randomized range finder
    (drawn on the CPU, then moved, so every device gets the same values)."""
    return _normal((K, cols), _seed(seed, "sketch", K, cols, 0), 0.0, 1.0, "cpu").to(device)
