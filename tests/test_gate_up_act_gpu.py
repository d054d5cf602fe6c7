"""GPU: the gate|up stack with the MLP activation fused into its epilogue
(h = act(gate) * up, "Quality (Gemma 4 31B)" page, "Activation function
fix"; the activation is a parameter), through the C ABI against the fp64
oracle, on the decode path (T <= 16), the prefill GEMM with gate and up rows
paired in one tile, and the prefill K-split path with its finish kernel."""
import sys

import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
from oracle.compare import compare
from oracle.workload import OracleWorkload
from weight_shared_rank_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda"
ACTS = ("gelu_tanh", "silu", "gelu")


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def mlp_workload(n, k, rank, cid):
    dims = {(0, "gate"): (n, k), (0, "up"): (n, k)}
    return synth.custom(2, 1, rank, dims, cid=cid)


def check(b, ow, wl, layer, act, T, rows=None):
    x = wl.x(layer, "gate_up", T, DEV)
    announce(f"gate_up_act {wl.name}/{wl.cid} layer {layer} {act} T={T}")
    h = b.gate_up_act(layer, act, x)
    torch.cuda.synchronize()
    xr = np64(x) if rows is None else np64(x)[rows]
    got = np64(h) if rows is None else np64(h)[rows]
    res = compare(got, ow.gate_up_act(layer, xr, act))
    assert res["ok"], f"layer {layer} {act} T={T}: {res}"


@pytest.mark.parametrize("T", [1, 5, 16, 17, 40, 200])
@pytest.mark.parametrize("act", ACTS)
def test_gate_up_act_ragged(gpu_lib, act, T):
    """300 rows per half, K=264: row tails in 16-row decode tiles and in the
    paired prefill tiles."""
    wl = mlp_workload(300, 264, 5, cid=81)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        check(b, ow, wl, layer, act, T)


@pytest.mark.parametrize("rank", [0, 64])
@pytest.mark.parametrize("T", [3, 33])
def test_gate_up_act_odd_rows_and_ranks(gpu_lib, rank, T):
    wl = mlp_workload(301, 136, rank, cid=82 + rank)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    check(b, ow, wl, 1, "gelu_tanh", T)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [40, 200])
def test_gate_up_act_split_k(gpu_lib, T):
    """Few rows and a long K: the prefill plan splits K, so h is formed by
    the finish kernel from the fp32 partials and the delta slice."""
    wl = mlp_workload(1024, 4096, 96, cid=85)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for act in ("gelu_tanh", "silu"):
        check(b, ow, wl, 0, act, T)


@pytest.mark.timeout(900)
def test_gate_up_act_gemma4_shapes(gpu_lib):
    """Gemma-4-31B gate|up (21504 x 5376 per half): decode at T=1 and 16 on
    the sliding workload, prefill at T=512 on the mixed workload (64 sampled
    token rows; rows are independent)."""
    wl = synth.workload(4)
    ow = OracleWorkload(wl, DEV, cache_w0=4)
    b = sdev.load(wl, DEV)
    for layer in (0, 59):
        for T in (1, 16):
            check(b, ow, wl, layer, "gelu_tanh", T)
    del b
    torch.cuda.empty_cache()
    wl = synth.workload(5)
    ow = OracleWorkload(wl, DEV, cache_w0=4)
    b = sdev.load(wl, DEV)
    rows = np.sort(np.random.default_rng(9).choice(512, 64, replace=False))
    rows[-1] = 511
    for layer in (0, 5):
        check(b, ow, wl, layer, "gelu_tanh", 512, rows=rows)
    del b
    torch.cuda.empty_cache()


def test_gate_up_act_arguments(gpu_lib):
    L = binding.lib()
    wl = mlp_workload(300, 264, 5, cid=81)
    b = sdev.load(wl, DEV)
    x = wl.x(0, "gate_up", 4, DEV)
    h = torch.empty((4, 300), dtype=torch.bfloat16, device=DEV)
    ws = b.workspace(4)
    args = (x.data_ptr(), 4, h.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert L.weightless_gate_up_act(b.handle, 0, 3, *args) == -4
    assert L.weightless_gate_up_act(b.handle, 0, -1, *args) == -4
    assert L.weightless_gate_up_act(b.handle, 2, 0, *args) == -4
    assert L.weightless_gate_up_act(b.handle, 0, 0, *args) == 0
    uneq = synth.custom(1, 1, 4, {(0, "gate"): (300, 264), (0, "up"): (296, 264)}, cid=86)
    bu = sdev.load(uneq, DEV)
    assert L.weightless_gate_up_act(bu.handle, 0, 0, *args) == -2
    torch.cuda.synchronize()
