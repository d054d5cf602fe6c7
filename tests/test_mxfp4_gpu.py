"""GPU: bundles whose shared block W0 is stored in MXFP4 (OCP microscaling:
E2M1 codes, one E8M0 scale per 32 elements; spec w0_format mxfp4, the
4-bit quantized-shared-block variant, "Quality (Gemma 4 31B)" page,
"Verdict").  The codes and scales the library computes at load must equal
the oracle's (oracle.quant) exactly, and every call path on such a bundle
must match the oracle evaluated on the dequantized W0."""
import sys

import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
from oracle import quant
from oracle.compare import compare
from oracle.workload import OracleWorkload, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def ragged(rank, cid):
    # K = 264: rows padded to 384 codes (three 128-k quads, a partial block)
    dims = {(0, "q"): (200, 264), (0, "k"): (72, 264), (0, "v"): (72, 264), (0, "o"): (264, 200),
            (0, "gate"): (300, 264), (0, "up"): (300, 264), (0, "down"): (264, 296)}
    return synth.custom(2, 1, rank, dims, cid=cid)


def call(b, layer, c, x):
    return b.stacked(layer, c, x) if c in ("qkv", "gate_up") else b.linear(layer, c, x)


def test_mxfp4_codes_and_scales_are_exact(gpu_lib):
    """With s = 1 and rank 0 the materialized weight is the dequantized W0
    itself (E2M1 value times 2^(b - 127) is exact in bf16): equal, value for
    value, to the oracle's coding of the same bf16 rows -- including rows
    scaled far from unit magnitude, an all-zero row, exact ties of the E2M1
    rounding, and values that saturate at 6 times the block scale."""
    wl = synth.custom(1, 1, 0, {(0, "q"): (96, 264), (0, "o"): (264, 96)}, cid=93)
    rowscale = torch.logspace(-30, 30, 96, base=2.0, dtype=torch.float32, device=DEV)
    ties = torch.tensor([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.75, -5.0, 6.0] * 2,
                        dtype=torch.float32, device=DEV)

    def tensors(kind, index, ltype, fam):
        if kind == "w0":
            w = wl.w0(index, ltype, fam, DEV)
            if fam == "q":
                w = (w.float() * rowscale[:, None]).to(torch.bfloat16)
                w[5] = 0
                w[7, :24] = ties.to(torch.bfloat16)      # block max 7 -> scale 1: exact ties, one saturating
            return w
        return torch.ones(wl.shape(0, fam)[0], dtype=torch.float32, device=DEV)
    b = sdev.load(wl, DEV, tensors=tensors, w0_format="mxfp4")
    for fam in ("q", "o"):
        announce(f"mxfp4 codes {fam}")
        got = np64(b.materialize(0, fam))
        w = to64(tensors("w0", 0, 0, fam))
        ref = quant.dequantize_mxfp4(*quant.quantize_mxfp4(w), w.shape[1])
        assert np.array_equal(got, ref), f"{fam}: {np.argwhere(got != ref)[:5]}"


@pytest.mark.parametrize("rank", [0, 5, 64])
@pytest.mark.parametrize("T", [1, 5, 16, 17, 40])
def test_mxfp4_calls_match_oracle(gpu_lib, rank, T):
    """K = 264 (a partial last block and quad), odd row counts, every call
    type, decode and prefill."""
    wl = ragged(rank, cid=102 + rank)
    ow = OracleWorkload(wl, DEV, w0_format="mxfp4")
    b = sdev.load(wl, DEV, w0_format="mxfp4")
    for layer in range(2):
        for c in ("qkv", "o", "gate_up", "down", "q", "v"):
            x = wl.x(layer, c, T, DEV)
            announce(f"mxfp4 r={rank} T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            torch.cuda.synchronize()
            res = compare(np64(y), ow.call(layer, c, np64(x)))
            assert res["ok"], f"layer {layer} {c}: {res}"
        x = wl.x(layer, "gate_up", T, DEV)
        h = b.gate_up_act(layer, "gelu_tanh", x)
        torch.cuda.synchronize()
        assert compare(np64(h), ow.gate_up_act(layer, np64(x), "gelu_tanh"))["ok"]


@pytest.mark.timeout(600)
def test_mxfp4_long_k_and_gemma4_decode(gpu_lib):
    """A long-K shape (V^T split in two K slices at T = 1) and the
    Gemma-4-31B sliding shapes of the first layer at decode (T = 1 and 16)
    and prefill (T = 40), every call type."""
    wl = synth.custom(1, 1, 40, {(0, "q"): (136, 16392), (0, "k"): (40, 16392), (0, "v"): (40, 16392),
                                 (0, "down"): (520, 16384)}, cid=98)
    ow = OracleWorkload(wl, DEV, w0_format="mxfp4")
    b = sdev.load(wl, DEV, w0_format="mxfp4")
    for c in ("qkv", "down", "k"):
        for T in (1, 3):
            x = wl.x(0, c, T, DEV)
            announce(f"mxfp4 long K {c} T={T}")
            y = call(b, 0, c, x)
            torch.cuda.synchronize()
            assert compare(np64(y), ow.call(0, c, np64(x)))["ok"], (c, T)
    del b
    wl = synth.workload(4)
    ow = OracleWorkload(wl, DEV, cache_w0=4, w0_format="mxfp4")
    b = sdev.load(wl, DEV, w0_format="mxfp4")
    for layer, Ts in ((0, (1, 16, 40)),):
        for T in Ts:
            for c, _ in synth.CALLS:
                x = wl.x(layer, c, T, DEV)
                announce(f"mxfp4 workload 4 layer {layer} {c} T={T}")
                y = call(b, layer, c, x)
                torch.cuda.synchronize()
                res = compare(np64(y), ow.call(layer, c, np64(x)))
                assert res["ok"], f"layer {layer} {c} T={T}: {res}"
    del b
    torch.cuda.empty_cache()
