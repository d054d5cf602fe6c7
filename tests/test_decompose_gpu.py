"""GPU: the analytic decomposition of one band of one family ("Add a new
model architecture" page, "Decompose HF weights"; "Quality" page, "Why
sharing fails: reconstruction error") run through weightless_decompose and
checked against the oracle's fp64 decomposition of the same bf16 weights.

What is unique is compared exactly or to rounding: the band mean W0 bit for
bit (both take the fp64 mean and round it through fp32 to bf16), the row
scale s to fp32 rounding.  U and V are not unique (signs, rotations within
equal singular values), so the delta is compared through U V^T where the
spectrum has a gap at the rank, and through the reconstruction error
(which no rank-r delta can push below the truncated SVD's) where it has none.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import decompose
from weight_shared_rank_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def run_gpu(w, rank, oversample=16, power_iters=4, seed=5):
    m, n, k = w.shape
    l = binding.sketch_columns(n, k, rank, oversample)
    omega = synth.sketch_matrix(seed, k, l, DEV) if rank > 0 else None
    out = binding.decompose(w.to(DEV), rank, omega, oversample=oversample, power_iters=power_iters)
    torch.cuda.synchronize()
    return out


def oracle_of(w, rank):
    layers = [np64(w[i]) for i in range(w.shape[0])]
    return decompose.decompose_band(layers, rank, store=True)


def delta(U, V):
    return U @ V.T


def check_mean_and_scale(w, W0g, sg, W0o, members):
    # the band mean: bit-exact
    assert np.array_equal(np64(W0g), W0o), "W0 differs from the oracle's band mean"
    for i, mem in enumerate(members):
        np.testing.assert_allclose(np64(sg[i]), mem["s"], rtol=1e-6, atol=0, err_msg=f"s of layer {i}")


@pytest.mark.parametrize("m,n,k", [(1, 200, 136), (2, 64, 64)])
def test_zero_residual(gpu_lib, m, n, k):
    """Passthrough (one layer per band) and identical layers: W0 = W, s = 1
    exactly and the delta is exactly zero."""
    announce(f"decompose zero residual m={m} {n}x{k}")
    w1 = synth.band_layers(11, 1, n, k)
    w = w1.expand(m, n, k).contiguous()
    W0, s, U, V = run_gpu(w, rank=8)
    assert torch.equal(W0.cpu(), w1[0])
    assert torch.all(s == 1.0).item()
    assert U.abs().max().item() == 0.0 and V.abs().max().item() == 0.0


@pytest.mark.parametrize("m,n,k,p,rank", [(2, 200, 136, 4, 8), (3, 96, 264, 3, 9), (2, 72, 40, 2, 4)])
def test_gapped_delta_matches_oracle(gpu_lib, m, n, k, p, rank):
    """A planted rank-p part per layer: the residual has a gap at rank m p,
    so the truncated SVD's U V^T is unique and the GPU's must match it."""
    announce(f"decompose gapped m={m} {n}x{k} p={p} r={rank}")
    w = synth.band_layers(21, m, n, k, planted_rank=p, planted_std=4.0)
    W0, s, U, V = run_gpu(w, rank)
    W0o, members = oracle_of(w, rank)
    check_mean_and_scale(w, W0, s, W0o, members)
    for i, mem in enumerate(members):
        sig = mem["sigma"]
        assert sig[rank - 1] > 5 * sig[rank], "input has no gap at the rank"
        dg, do = delta(np64(U[i]), np64(V[i])), delta(mem["U"], mem["V"])
        rel = np.linalg.norm(dg - do) / np.linalg.norm(do)
        assert rel < 1.5e-2, f"layer {i}: |UV^T - oracle| / |oracle| = {rel:.3e}"
        err = decompose.rel_frobenius_error(np64(w[i]), W0o, np64(s[i]), np64(U[i]), np64(V[i]))
        assert abs(err - mem["err"]) < 1e-3, (err, mem["err"])


@pytest.mark.parametrize("m,n,k,rank", [(4, 256, 192, 16), (3, 136, 300, 24), (2, 100, 100, 100),
                                         (2, 300, 200, 120)])
def test_flat_spectrum_error(gpu_lib, m, n, k, rank):
    """i.i.d. layers (no gap, the randomized range finder's worst case): with
    16 extra sketch columns and 4 power rounds the GPU delta's reconstruction
    error stays within 1% of the truncated SVD's (an fp64 model of the same
    iteration lands 0.2-0.3% above it on these shapes), which it cannot beat
    beyond the bf16 rounding of the stored factors.  rank = min(N, K)
    recovers R exactly; the last case has a wide sketch (136 columns)."""
    announce(f"decompose flat m={m} {n}x{k} r={rank}")
    w = synth.band_layers(31, m, n, k)
    W0, s, U, V = run_gpu(w, rank)
    W0o, members = oracle_of(w, rank)
    check_mean_and_scale(w, W0, s, W0o, members)
    for i, mem in enumerate(members):
        err = decompose.rel_frobenius_error(np64(w[i]), W0o, np64(s[i]), np64(U[i]), np64(V[i]))
        assert err <= mem["err"] * 1.01 + 1e-4, (i, err, mem["err"])
        assert err >= mem["err"] * 0.99 - 1e-4, (i, err, mem["err"])


def test_rank_zero(gpu_lib):
    announce("decompose rank 0")
    w = synth.band_layers(41, 3, 64, 48)
    W0, s, U, V = run_gpu(w, 0)
    W0o, members = oracle_of(w, 0)
    check_mean_and_scale(w, W0, s, W0o, members)
    assert U.numel() == 0 and V.numel() == 0


@pytest.mark.parametrize("fam,n,k", [("gate", 4096, 1152), ("down", 1152, 4096)])
def test_gemma3_shapes(gpu_lib, fam, n, k):
    """One band of the Gemma 3 1B decomposition (26 layers in 13 bands: two
    layers per band, rank 32) at the family's real shape."""
    announce(f"decompose gemma3 {fam} {n}x{k} m=2 r=32")
    w = synth.band_layers(51, 2, n, k)
    W0, s, U, V = run_gpu(w, 32)
    W0o, members = oracle_of(w, 32)
    check_mean_and_scale(w, W0, s, W0o, members)
    for i, mem in enumerate(members):
        err = decompose.rel_frobenius_error(np64(w[i]), W0o, np64(s[i]), np64(U[i]), np64(V[i]))
        assert mem["err"] * 0.999 - 1e-4 <= err <= mem["err"] * 1.01 + 1e-4, (fam, i, err, mem["err"])


def test_decompose_bundle_roundtrip(gpu_lib):
    """The GPU outputs are in the layouts theta_bundle_load takes: a bundle
    loaded from them evaluates diag(s) W0 x + U (V^T x) of the decomposed
    factors (checked against the effective weight the library materializes
    from the same bundle)."""
    announce("decompose -> bundle roundtrip")
    m, n, k, rank = 2, 128, 96, 8
    w = synth.band_layers(61, m, n, k, planted_rank=4)
    W0, s, U, V = run_gpu(w, rank)
    spec = binding.make_spec(m, 1, {(0, "o"): (n, k)}, {(0, "o"): rank})
    srcs = [("w0", 0, 0, "o", W0)]
    for l in range(m):
        srcs += [("s", l, 0, "o", s[l].contiguous()), ("u", l, 0, "o", U[l].contiguous()),
                 ("v", l, 0, "o", V[l].contiguous())]
    b = binding.ThetaBundle(spec, srcs, device=DEV)
    for l in range(m):
        weff = np64(b.materialize(l, "o"))
        ref = np64(s[l])[:, None] * np64(W0) + np64(U[l]) @ np64(V[l]).T
        assert np.abs(weff - ref).max() <= 1e-2 * np.abs(ref).max()


def test_decompose_rejects_bad_arguments(gpu_lib):
    w = synth.band_layers(71, 2, 32, 16).to(DEV)
    with pytest.raises(binding.WlError):
        binding.decompose(w, 17, synth.sketch_matrix(1, 16, 16, DEV))  # rank > min(N, K)
    with pytest.raises(binding.WlError):
        binding.decompose(w, 4, synth.sketch_matrix(1, 16, 3, DEV))  # wrong sketch width


def test_concurrent_calls_match_sequential(gpu_lib):
    """Independent band calls on several streams from several host threads
    (each with its own workspace) give the same bits as one call at a time:
    a call's state lives in its arguments and workspace only."""
    from concurrent.futures import ThreadPoolExecutor
    announce("decompose: 6 bands on 3 streams against one at a time")
    rank, n, k = 8, 192, 136
    l = binding.sketch_columns(n, k, rank, 16)
    bands = [(synth.band_layers(81 + i, 2, n, k, planted_rank=3).to(DEV), synth.sketch_matrix(90 + i, k, l, DEV))
             for i in range(6)]
    torch.cuda.synchronize()
    seq = [binding.decompose(w, rank, om) for w, om in bands]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]

    def work(i):
        with torch.cuda.stream(streams[i]):
            out = [(j, binding.decompose(w, rank, om, stream=streams[i])) for j, (w, om) in enumerate(bands)
                   if j % 3 == i]
        streams[i].synchronize()
        return out
    with ThreadPoolExecutor(3) as ex:
        par = dict(p for outs in ex.map(work, range(3)) for p in outs)
    torch.cuda.synchronize()
    for j, ref in enumerate(seq):
        for a, b in zip(ref, par[j]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), j
