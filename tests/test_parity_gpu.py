"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
five synthetic workloads.

Tolerance (bf16 inputs, fp32 accumulation): per call max|d| <= 1e-2 max|y_ref|
and per token row ||d||_2 <= 5e-3 ||y_ref||_2 (oracle.compare).  The bundle
and the activations are drawn on the GPU by the seeded generator; the oracle
receives the same values, upcast exactly to fp64.
"""
import sys

import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
from oracle.compare import compare
from oracle.workload import OracleWorkload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def check(y, ref, label, rows=None):
    got = np64(y)
    if rows is not None:
        got = got[rows]
    res = compare(got, ref)
    assert res["ok"], f"{label}: {res}"
    return res


def run_call(bundle, layer, call, x):
    if call in ("qkv", "gate_up"):
        return bundle.stacked(layer, call, x)
    return bundle.linear(layer, call, x)


def decoded_tensors(ow):
    """Source tensors of a decomposed workload, from the oracle's
    decomposition (exactly representable in bf16 / fp32)."""
    def tensors(kind, index, ltype, fam):
        wl = ow.wl
        if kind == "w0":
            return torch.from_numpy(ow.decomposed_band(index, ltype, fam)[0]).to(torch.bfloat16)
        W0, per = ow.decomposed_band(ow.band(index), ltype, fam)
        m = per[index]
        if kind == "s":
            return torch.from_numpy(m["s"]).to(torch.float32)
        return torch.from_numpy(m[kind.upper()]).to(torch.bfloat16)
    return tensors


# --------------------------------------------------------------------------
# workload 1: one family, 2 layers share W0, r=4, T=4
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def w1(gpu_lib):
    wl = synth.workload(1)
    announce("load workload 1")
    b = sdev.load(wl, DEV)
    return wl, b, OracleWorkload(wl, DEV)


def test_workload1_parity(w1):
    wl, b, ow = w1
    for layer in range(2):
        x = wl.x(layer, "up", 4, DEV)
        announce(f"workload 1 layer {layer} up T=4")
        y = b.linear(layer, "up", x)
        torch.cuda.synchronize()
        check(y, ow.call(layer, "up", np64(x)), f"w1 layer {layer}")


@pytest.mark.parametrize("T", list(range(1, 17)) + [17, 31, 64, 130])
def test_workload1_token_sweep(w1, T):
    """T <= 16 runs the decode kernel, T > 16 the prefill GEMMs."""
    wl, b, ow = w1
    x = wl.x(1, "up", T, DEV, salt=T)
    announce(f"workload 1 layer 1 up T={T}")
    y = b.linear(1, "up", x)
    torch.cuda.synchronize()
    check(y, ow.call(1, "up", np64(x)), f"w1 T={T}")


# --------------------------------------------------------------------------
# workload 2: Gemma-3-1B decode, G=13 decomposed bundle, r=32, T=1
# --------------------------------------------------------------------------
def _decomposed_bundle(variant):
    wl = synth.workload(2, variant)
    ow = OracleWorkload(wl, DEV)
    announce(f"decompose workload 2 ({variant or 'G13'}) on the host")
    ow.prefetch_decompositions([(ow.band(l), 0, f) for l in range(wl.num_layers) for f in synth.FAMILIES],
                               workers=16)
    announce("load workload 2")
    return wl, sdev.load(wl, DEV, tensors=decoded_tensors(ow)), ow


@pytest.fixture(scope="module")
def w2(gpu_lib):
    return _decomposed_bundle(None)


@pytest.mark.timeout(900)
def test_workload2_all_layers(w2):
    wl, b, ow = w2
    worst = 0.0
    for layer in range(wl.num_layers):
        for call, _ in synth.CALLS:
            x = wl.x(layer, call, 1, DEV)
            announce(f"workload 2 layer {layer} {call} T=1")
            y = run_call(b, layer, call, x)
            torch.cuda.synchronize()
            res = check(y, ow.call(layer, call, np64(x)), f"w2 layer {layer} {call}")
            worst = max(worst, res["worst_row_rel"])
    announce(f"workload 2 worst row rel err {worst:.2e}")


@pytest.mark.timeout(900)
def test_workload2_passthrough_exact(gpu_lib):
    """G = L: every layer keeps its own weight, s = 1, U V^T = 0.  The output
    must match the dense product within tolerance, and equal bit for bit the
    same kernel run on a rank-0 bundle of the same W0 and s."""
    wl, b, ow = _decomposed_bundle("passthrough")
    for layer in range(wl.num_layers):
        for fam in synth.FAMILIES:
            W0, per = ow.decomposed_band(layer, 0, fam)
            assert np.all(per[layer]["s"] == 1.0) and not np.any(per[layer]["U"] @ per[layer]["V"].T)
    # rank-0 twin of the same bundle
    wl0 = synth.custom(26, 26, 0, dict(wl.dims), cid=2)
    b0 = sdev.load(wl0, DEV, tensors=decoded_tensors(ow))
    for layer in range(wl.num_layers):
        for call, fams in synth.CALLS:
            x = wl.x(layer, call, 1, DEV)
            announce(f"workload 2 passthrough layer {layer} {call}")
            y = run_call(b, layer, call, x)
            y0 = run_call(b0, layer, call, x)
            torch.cuda.synchronize()
            dense = np.concatenate([np64(x) @ np64(wl.layer_weight(layer, f, DEV)).T for f in fams], axis=1)
            check(y, dense, f"passthrough layer {layer} {call}")
            assert torch.equal(y.float(), y0.float()), f"passthrough layer {layer} {call}: differs from rank 0"


# --------------------------------------------------------------------------
# workload 3: Gemma-3-1B prefill, G=1, r=64, T=2048
# --------------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_workload3_prefill_all_layers(gpu_lib):
    wl = synth.workload(3)
    ow = OracleWorkload(wl, DEV, cache_w0=8)
    announce("load workload 3")
    b = sdev.load(wl, DEV)
    for layer in range(wl.num_layers):
        for fam in synth.FAMILIES:
            x = wl.x(layer, fam, 2048, DEV)
            announce(f"workload 3 layer {layer} {fam} T=2048")
            y = b.linear(layer, fam, x)
            torch.cuda.synchronize()
            check(y, ow.call(layer, fam, np64(x)), f"w3 layer {layer} {fam}")
    for layer in (0, 25):
        for call in ("qkv", "gate_up"):
            x = wl.x(layer, call, 2048, DEV)
            announce(f"workload 3 layer {layer} stacked {call}")
            y = b.stacked(layer, call, x)
            torch.cuda.synchronize()
            check(y, ow.call(layer, call, np64(x)), f"w3 layer {layer} {call}")


# --------------------------------------------------------------------------
# workload 4: Gemma-4-31B sliding decode, G=5, r=256, T=1 and 16
# --------------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_workload4_sampled_layers(gpu_lib):
    """Every call on the first and last layer of each band (oracle cost)."""
    wl = synth.workload(4)
    ow = OracleWorkload(wl, DEV, cache_w0=8)
    announce("load workload 4 (8.7 GB arena)")
    b = sdev.load(wl, DEV)
    layers = sorted({l for band in range(5) for l in (12 * band, 12 * band + 11)})
    for layer in layers:
        for T in (1, 16):
            for call, _ in synth.CALLS:
                x = wl.x(layer, call, T, DEV)
                announce(f"workload 4 layer {layer} {call} T={T}")
                y = run_call(b, layer, call, x)
                torch.cuda.synchronize()
                check(y, ow.call(layer, call, np64(x)), f"w4 layer {layer} {call} T={T}")
    del b
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_workload4_mid_token_counts(gpu_lib):
    """Layer 0 at T = 4 and 8: the several-token decode paths at the real
    shapes (two-tile stream workgroups for q|k|v and gate|up, the 16-wave
    two-tile kernel for down's long K slices at T = 8, one-tile o)."""
    wl = synth.workload(4)
    ow = OracleWorkload(wl, DEV, cache_w0=8)
    announce("load workload 4 (8.7 GB arena)")
    b = sdev.load(wl, DEV)
    for T in (4, 8):
        for call, _ in synth.CALLS:
            x = wl.x(0, call, T, DEV)
            announce(f"workload 4 layer 0 {call} T={T}")
            y = run_call(b, 0, call, x)
            torch.cuda.synchronize()
            check(y, ow.call(0, call, np64(x)), f"w4 layer 0 {call} T={T}")
    del b
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# workload 5: Gemma-4-31B mixed prefill, G=1 per type, r=1024, T=512
# --------------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_workload5_sampled(gpu_lib):
    """Every call on the first and last layer of each layer type; the oracle
    evaluates a sample of 64 token rows of each output (rows are independent)."""
    wl = synth.workload(5)
    ow = OracleWorkload(wl, DEV, cache_w0=8)
    announce("load workload 5 (17.2 GB arena)")
    b = sdev.load(wl, DEV)
    rows = np.sort(np.random.default_rng(5).choice(512, 64, replace=False))
    rows[-1] = 511
    for layer in (0, 5, 58, 59):
        for call, _ in synth.CALLS:
            x = wl.x(layer, call, 512, DEV)
            announce(f"workload 5 layer {layer} (type {wl.layer_types[layer]}) {call} T=512")
            y = run_call(b, layer, call, x)
            torch.cuda.synchronize()
            ref = ow.call(layer, call, np64(x)[rows])
            check(y, ref, f"w5 layer {layer} {call}", rows=rows)
            if call == "qkv" and wl.layer_types[layer] == 1:
                nq, nk = wl.shape(1, "q")[0], wl.shape(1, "k")[0]
                assert torch.equal(y[:, nq:nq + nk], y[:, nq + nk:]), "tied v slot differs from k"
    del b
    torch.cuda.empty_cache()
