"""Pins of the oracle's call resolution (CPU only): which band, which shared
block and which tied child a call of a layer uses.

The expected values are built by hand from tables written out here -- the
band of every layer, the member layers of every shared block, the layer type
of every layer -- and the explicit effective weight diag(s) W0 + U V^T of
each child, never through the oracle's own resolution code:

  * bands are contiguous and balanced ("Quality (Gemma 4 31B)" page,
    "Decomposition quality": 5 bands of 12 layers over 60 layers); here
    8 layers in 2 bands of 4;
  * attention families keep one W0 per (band, layer type, family), MLP
    families one W0 per (band, family) for every layer type ("Add a new model
    architecture" page, "Decompose HF weights: the mixed-attention case");
  * on a K=V-tied layer type v has no bundle and its output repeats k's
    (same section, attention_k_eq_v).
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import bf16, forward
from oracle.workload import OracleWorkload

# the mixed workload: 8 layers, 2 bands, two layer types, type 1 tied
BAND = [0, 0, 0, 0, 1, 1, 1, 1]
TYPE = [0, 1, 1, 0, 0, 1, 0, 1]
ATTN_MEMBERS = {(0, 0): [0, 3], (0, 1): [1, 2], (1, 0): [4, 6], (1, 1): [5, 7]}   # (band, type) -> layers
MLP_MEMBERS = {0: [0, 1, 2, 3], 1: [4, 5, 6, 7]}                                  # band -> layers
CALLS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))

_DIMS = {(0, "q"): (16, 24), (0, "k"): (8, 24), (0, "v"): (8, 24), (0, "o"): (24, 16),
         (0, "gate"): (20, 24), (0, "up"): (20, 24), (0, "down"): (24, 20),
         (1, "q"): (24, 24), (1, "k"): (8, 24), (1, "o"): (24, 24),
         (1, "gate"): (20, 24), (1, "up"): (20, 24), (1, "down"): (24, 20)}


def mixed_workload(rank=3, decomposed=False):
    wl = synth.custom(8, 2, rank, _DIMS, layer_types=TYPE, k_eq_v_types=(1,), cid=61)
    return dataclasses.replace(wl, decomposed=decomposed)


def np64(t):
    return t.detach().float().double().numpy()


def weff_loops(W0, s, U, V):
    """diag(s) W0 + U V^T by explicit loops."""
    N, K = W0.shape
    W = np.empty((N, K))
    for i in range(N):
        for j in range(K):
            W[i, j] = s[i] * W0[i, j] + sum(U[i, k] * V[j, k] for k in range(U.shape[1]))
    return W


def expected_direct(wl, layer, call, fams, x):
    """A directly drawn workload's call output from the hand tables."""
    outs = []
    for f in fams:
        if f == "v" and TYPE[layer] == 1:
            outs.append(outs[-1].copy())     # tied: k's output again
            continue
        key_type = TYPE[layer] if f in ("q", "k", "v", "o") else 0
        W0 = np64(wl.w0(BAND[layer], key_type, f))
        W = weff_loops(W0, np64(wl.s(layer, f)), np64(wl.u(layer, f)), np64(wl.v(layer, f)))
        outs.append(x @ W.T)
    return np.concatenate(outs, axis=1)


def test_direct_workload_calls_match_hand_tables():
    wl = mixed_workload()
    ow = OracleWorkload(wl, cache_w0=64)
    for layer in range(8):
        for call, fams in CALLS:
            x = np64(wl.x(layer, call, 3))
            got = ow.call(layer, call, x)
            want = expected_direct(wl, layer, call, fams, x)
            assert got.shape == want.shape, (layer, call)
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=f"layer {layer} {call}")
        # a single v call on a tied layer is k's projection
        xk = np64(wl.x(layer, "k", 2))
        if TYPE[layer] == 1:
            assert np.array_equal(ow.call(layer, "v", xk), ow.call(layer, "k", xk))


def test_direct_workload_shares_mlp_blocks_across_types():
    wl = mixed_workload()
    ow = OracleWorkload(wl, cache_w0=64)
    for band, layers in MLP_MEMBERS.items():
        for f in ("gate", "up", "down"):
            blocks = [ow.params(l, f)[0] for l in layers]
            assert all(np.array_equal(b, blocks[0]) for b in blocks), (band, f)
    # attention blocks differ between the two types of one band
    for f in ("q", "o"):
        assert not np.array_equal(ow.params(0, f)[0][:8, :8], ow.params(1, f)[0][:8, :8])


@pytest.mark.parametrize("fam", ["q", "k", "o", "gate", "down"])
def test_decomposed_blocks_are_group_means(fam):
    """W0 of a decomposed workload is the rounded mean of exactly its group's
    member layers (both layer types for an MLP family, one type for an
    attention family)."""
    wl = mixed_workload(rank=2, decomposed=True)
    ow = OracleWorkload(wl)
    groups = ({(b, None): ls for b, ls in MLP_MEMBERS.items()} if fam in ("gate", "up", "down")
              else ATTN_MEMBERS)
    for (band, t), layers in groups.items():
        mean = sum(np64(wl.layer_weight(l, fam)) for l in layers) / len(layers)
        want = bf16.round_bf16(mean)
        for l in layers:
            assert BAND[l] == band and (t is None or TYPE[l] == t)
            assert np.array_equal(ow.params(l, fam)[0], want), (fam, band, t, l)


def test_decomposed_full_rank_reproduces_each_layer():
    """At full rank the delta absorbs the whole residual, so each layer's
    call reproduces that layer's own weight (k's on a tied v slot) up to the
    bf16 rounding of the stored factors."""
    wl = mixed_workload(rank=24, decomposed=True)
    ow = OracleWorkload(wl)
    for layer in range(8):
        for call, fams in CALLS:
            x = np64(wl.x(layer, call, 2))
            outs = []
            for f in fams:
                src = "k" if (f == "v" and TYPE[layer] == 1) else f
                outs.append(x @ np64(wl.layer_weight(layer, src)).T)
            want = np.concatenate(outs, axis=1)
            got = ow.call(layer, call, x)
            assert got.shape == want.shape
            assert np.max(np.abs(got - want)) <= 2e-2 * np.max(np.abs(want)), (layer, call)


def test_band_table_is_contiguous():
    ow = OracleWorkload(mixed_workload())
    assert [ow.band(l) for l in range(8)] == BAND
