"""GPU: the effective weight W_eff = diag(s) W0 + U V^T that a bundle stands
for ("Override the graph build" page: the variant that precomputes the
effective weight outside the graph), materialized through the C ABI and
checked element by element against the fp64 oracle (oracle.forward.
effective_weight, pinned by the factored = explicit identity), plus its
agreement with the factored call on the same bundle."""
import sys

import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
from oracle import forward
from oracle.compare import compare
from oracle.workload import OracleWorkload
from weight_shared_rank_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def ragged(rank, layer_types=(0, 1), k_eq_v=(1,)):
    dims = {}
    for t in sorted(set(layer_types)):
        q = 200 if t == 0 else 136
        dims.update({(t, "q"): (q, 264), (t, "k"): (72, 264), (t, "o"): (264, q),
                     (t, "gate"): (300, 264), (t, "up"): (300, 264), (t, "down"): (264, 296)})
        if t not in k_eq_v:
            dims[(t, "v")] = (72, 264)
    return synth.custom(len(layer_types), 1, rank, dims, layer_types=layer_types, k_eq_v_types=k_eq_v,
                        cid=60 + rank)


@pytest.mark.parametrize("rank", [0, 5, 64])
def test_materialize_matches_oracle(gpu_lib, rank):
    wl = ragged(rank)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(wl.num_layers):
        for fam in synth.FAMILIES:
            announce(f"materialize r={rank} layer {layer} {fam}")
            w = b.materialize(layer, fam)
            torch.cuda.synchronize()
            ref = forward.effective_weight(*ow.params(layer, fam))
            assert w.shape == ref.shape
            res = compare(np64(w), ref)
            assert res["ok"], f"layer {layer} {fam}: {res}"
        # tied v on type 1 is k's weight
        if wl.layer_types[layer] == 1:
            assert torch.equal(b.materialize(layer, "v"), b.materialize(layer, "k"))


def test_materialize_workload1_and_dense_product(gpu_lib):
    """Workload 1 (up 4096 x 1152, rank 4): W_eff against the oracle, and the
    dense product x W_eff^T against the factored call y (both bf16-rounded
    once, so they agree within the call tolerance)."""
    wl = synth.workload(1)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        announce(f"materialize workload 1 layer {layer}")
        w = b.materialize(layer, "up")
        x = wl.x(layer, "up", 4, DEV)
        y = b.linear(layer, "up", x)
        torch.cuda.synchronize()
        ref = forward.effective_weight(*ow.params(layer, "up"))
        assert compare(np64(w), ref)["ok"]
        dense = np64(x) @ np64(w).T
        res = compare(np64(y), dense)
        assert res["ok"], res


def test_materialize_arguments(gpu_lib):
    wl = ragged(5)
    b = sdev.load(wl, DEV)
    L = binding.lib()
    need = L.weightless_materialize_workspace_bytes(b.handle)
    assert need >= 264 * 32 * 2
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty((200, 264), dtype=torch.bfloat16, device=DEV)
    assert L.weightless_materialize(b.handle, 0, 0, out.data_ptr(), ws.data_ptr(), need - 256, None) == -5
    assert L.weightless_materialize(b.handle, 0, 0, out.data_ptr() + 2, ws.data_ptr(), need, None) == -1
    assert L.weightless_materialize(b.handle, 0, 0, 0, ws.data_ptr(), need, None) == -1
    assert L.weightless_materialize(b.handle, 5, 0, out.data_ptr(), ws.data_ptr(), need, None) == -4
    assert L.weightless_materialize(b.handle, 0, 0, b.arena.data_ptr(), ws.data_ptr(), need, None) == -1
    assert L.weightless_materialize(b.handle, 0, 0, out.data_ptr(), ws.data_ptr(), need, None) == 0
    torch.cuda.synchronize()
