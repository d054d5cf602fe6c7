"""GPU edge cases through the C ABI: ragged shapes (row tails, K tails, rank
padding, children straddling tiles), K=V tying, stacked versus single calls,
run-to-run determinism, rank 0, T = 0, workspace errors, host-resident
sources and graph replay."""
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


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def np64(t):
    return t.detach().float().cpu().double().numpy()


def ragged(rank=5, layer_types=(0, 0, 0), k_eq_v=(), bands=2):
    dims = {}
    for t in sorted(set(layer_types)):
        q = 200 if t == 0 else 136
        dims.update({(t, "q"): (q, 264), (t, "k"): (72, 264), (t, "v"): (72, 264), (t, "o"): (264, q),
                     (t, "gate"): (300, 264), (t, "up"): (300, 264), (t, "down"): (264, 296)})
    return synth.custom(len(layer_types), bands, rank, dims, layer_types=layer_types, k_eq_v_types=k_eq_v,
                        cid=50 + rank)


def call(b, layer, c, x):
    return b.stacked(layer, c, x) if c in ("qkv", "gate_up") else b.linear(layer, c, x)


@pytest.mark.parametrize("rank", [0, 5, 64, 100])
@pytest.mark.parametrize("T", [1, 5, 16, 17, 40])
def test_ragged_shapes(gpu_lib, rank, T):
    """Against the oracle: decode (T <= 16) and prefill (T > 16) on ragged
    rows, K tails and ranks 0, 5, 64 and 100 (padded to 128: several rank
    steps per epilogue wave)."""
    wl = ragged(rank)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(wl.num_layers):
        for c in ["qkv", "o", "gate_up", "down"] + list(synth.FAMILIES):
            x = wl.x(layer, c, T, DEV)
            announce(f"ragged r={rank} T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            torch.cuda.synchronize()
            res = compare(np64(y), ow.call(layer, c, np64(x)))
            assert res["ok"], f"layer {layer} {c}: {res}"


@pytest.mark.parametrize("T", [1, 16, 33])
def test_stacked_equals_singles_bitwise(gpu_lib, T):
    wl = ragged(7)
    b = sdev.load(wl, DEV)
    for layer in range(wl.num_layers):
        for c, fams in (("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up"))):
            x = wl.x(layer, c, T, DEV)
            announce(f"stacked vs singles T={T} layer {layer} {c}")
            ys = b.stacked(layer, c, x)
            cat = torch.cat([b.linear(layer, f, x) for f in fams], dim=1)
            torch.cuda.synchronize()
            assert torch.equal(ys.float(), cat.float()), f"layer {layer} {c} T={T}"


@pytest.mark.parametrize("T", [1, 16, 24])
def test_k_eq_v_mixed_types(gpu_lib, T):
    wl = ragged(6, layer_types=(0, 1, 0, 1), k_eq_v=(1,), bands=2)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(4):
        x = wl.x(layer, "qkv", T, DEV)
        announce(f"k_eq_v T={T} layer {layer}")
        y = b.stacked(layer, "qkv", x)
        yv = b.linear(layer, "v", x)
        yk = b.linear(layer, "k", x)
        torch.cuda.synchronize()
        assert compare(np64(y), ow.call(layer, "qkv", np64(x)))["ok"]
        nq, nk = wl.shape(wl.layer_types[layer], "q")[0], 72
        if wl.layer_types[layer] == 1:
            assert torch.equal(y[:, nq:nq + nk], y[:, nq + nk:])
            assert torch.equal(yv, yk)
        assert y.shape[1] == nq + 2 * nk


def test_determinism_and_t0(gpu_lib):
    wl = synth.workload(1)
    b = sdev.load(wl, DEV)
    for T in (4, 16, 200):
        x = wl.x(0, "up", T, DEV)
        announce(f"determinism T={T}")
        y1 = b.linear(0, "up", x)
        y2 = b.linear(0, "up", x)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
    y = torch.full((0, 4096), 7, dtype=torch.bfloat16, device=DEV)
    b.linear(0, "up", torch.empty((0, 1152), dtype=torch.bfloat16, device=DEV), y=y)
    # stacked calls (decode with two-tile stream workgroups, prefill) and the
    # paired gate|up activation kernel repeat bit for bit too
    wr = ragged(64)
    br = sdev.load(wr, DEV)
    for T in (16, 200):
        for c in ("qkv", "gate_up"):
            x = wr.x(0, c, T, DEV)
            announce(f"determinism stacked {c} T={T}")
            y1, y2 = br.stacked(0, c, x), br.stacked(0, c, x)
            torch.cuda.synchronize()
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), (c, T)
        x = wr.x(0, "gate_up", T, DEV)
        h1, h2 = br.gate_up_act(0, "gelu_tanh", x), br.gate_up_act(0, "gelu_tanh", x)
        torch.cuda.synchronize()
        assert torch.equal(h1.view(torch.int16), h2.view(torch.int16)), ("act", T)


def test_workspace_too_small_and_aliasing(gpu_lib):
    wl = synth.workload(1)
    b = sdev.load(wl, DEV)
    x = wl.x(0, "up", 4, DEV)
    small = torch.zeros(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(binding.WlError) as e:
        b.linear(0, "up", x, ws=small)
    assert e.value.status == -5
    big = torch.empty((4, 4096 + 1152), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.WlError) as e:
        b.linear(0, "up", big[:, :1152].contiguous(), y=None)  # fine: separate buffers
        b.linear(0, "up", big.view(-1)[:4 * 1152].view(4, 1152), y=big.view(-1)[1000:1000 + 4 * 4096].view(4, 4096))
    assert e.value.status == -1


def test_host_sources_match_device_sources(gpu_lib):
    wl = ragged(5)
    bd = sdev.load(wl, DEV)
    bh = binding.ThetaBundle(sdev.spec_of(wl), [(k, i, t, f, v.cpu()) for (k, i, t, f, v) in sdev.sources_of(wl, DEV)])
    for T in (3, 20):
        x = wl.x(2, "qkv", T, DEV)
        announce(f"host sources T={T}")
        assert torch.equal(bd.stacked(2, "qkv", x), bh.stacked(2, "qkv", x))


def test_graph_replay(gpu_lib):
    """A captured graph of decode and prefill calls replays correctly; checked
    on several replays with eager work and synchronizations in between."""
    wl = ragged(9)
    b = sdev.load(wl, DEV)
    xs = wl.x(1, "qkv", 3, DEV)
    xp = wl.x(1, "gate_up", 40, DEV)
    ref_s = b.stacked(1, "qkv", xs)
    ref_p = b.stacked(1, "gate_up", xp)
    torch.cuda.synchronize()
    ys = torch.empty_like(ref_s)
    yp = torch.empty_like(ref_p)
    ws_d = b.workspace(3)
    ws_p = b.workspace(40)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        b.stacked(1, "qkv", xs, y=ys, ws=ws_d)
        b.stacked(1, "gate_up", xp, y=yp, ws=ws_p)
    for rep in range(5):
        announce(f"graph replay {rep}")
        ys.zero_()
        yp.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ref_s) and torch.equal(yp, ref_p), f"replay {rep}"
        b.stacked(1, "qkv", xs)       # eager work between replays
        torch.cuda.synchronize()


def test_call_validation(gpu_lib):
    """Argument errors of loaded-bundle calls return before any launch."""
    import ctypes
    L = binding.lib()
    wl = ragged(5)
    b = sdev.load(wl, DEV)
    x = wl.x(0, "qkv", 4, DEV)
    y = torch.empty((4, 1000), dtype=torch.bfloat16, device=DEV)
    ws = b.workspace(4)
    h = b.handle
    args = lambda xp=x.data_ptr(), yp=y.data_ptr(), T=4, wsb=ws.numel(): (xp, T, yp, ws.data_ptr(), wsb, None)
    assert L.weightless_linear(h, 3, 0, *args()) == -4            # layer out of range
    assert "layer" in binding.last_error()
    assert L.weightless_linear(h, -1, 0, *args()) == -4
    assert L.weightless_linear(h, 0, 7, *args()) == -4            # family out of range
    assert L.weightless_stacked_linear(h, 0, 2, *args()) == -4    # stack out of range
    assert L.weightless_linear(h, 0, 0, *args(T=-1)) == -1        # negative T
    assert L.weightless_linear(h, 0, 0, *args(xp=0)) == -1        # NULL x
    assert L.weightless_linear(h, 0, 0, *args(xp=x.data_ptr() + 2)) == -1   # x not 16-byte aligned
    assert L.weightless_linear(h, 0, 0, *args(wsb=16)) == -5      # workspace too small
    assert L.weightless_linear(h, 0, 0, *args(T=0)) == 0          # T = 0 is a no-op
    assert L.weightless_out_dim(h, 0, -1, 0) == 200 + 72 + 72
    assert L.weightless_out_dim(h, 0, 0, -1) == 200
    wl0 = synth.custom(2, 1, 4, {(0, "q"): (64, 64), (0, "k"): (32, 64)})
    b0 = sdev.load(wl0, DEV)
    assert L.weightless_stacked_linear(b0.handle, 0, 0, *args()) == -4      # v absent, not tied
    assert L.weightless_linear(b0.handle, 0, 5, *args()) == -4              # up absent


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [40, 200])
def test_split_k_prefill(gpu_lib, T):
    """Few-row GEMMs with long K take the K-split path (fp32 partials, a
    delta slice, elementwise finish); stacked and single-family calls of one
    group plan differently and must both fit the workspace and match the
    oracle.  Row counts that are not multiples of 4 exercise the scalar
    finish path; type 1 ties v to k."""
    dims = {}
    for t in (0, 1):
        dims.update({(t, "q"): (4100, 4096), (t, "k"): (518, 4096), (t, "o"): (1000, 8192),
                     (t, "gate"): (1024, 4096), (t, "up"): (1024, 4096), (t, "down"): (4096, 6144)})
        if t == 0:
            dims[(t, "v")] = (518, 4096)
    wl = synth.custom(2, 1, 96, dims, layer_types=(0, 1), k_eq_v_types=(1,), cid=77)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in (0, 1):
        for c in ("qkv", "o", "gate_up", "down", "q", "k", "v"):
            x = wl.x(layer, c, T, DEV)
            announce(f"split-K prefill T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            torch.cuda.synchronize()
            ref_call = "k" if (c == "v" and wl.layer_types[layer] == 1) else c   # tied: v is k's output
            res = compare(np64(y), ow.call(layer, ref_call, np64(x)))
            assert res["ok"], f"layer {layer} {c}: {res}"


@pytest.mark.parametrize("rank", [5, 70])
def test_long_k_decode_splits_vt(gpu_lib, rank):
    """At T = 1 with an FP8 shared block a K of 16384 or more splits the V^T
    rows in two K slices whose fp32 partials the epilogue adds (with bf16,
    calls of fewer than 4096 rows split them too): ragged rows and ranks,
    single and stacked calls, both formats, against the oracle."""
    dims = {(0, "q"): (136, 16392), (0, "k"): (40, 16392), (0, "v"): (40, 16392), (0, "o"): (16392, 136),
            (0, "gate"): (72, 16384), (0, "up"): (72, 16384), (0, "down"): (16384, 72)}
    wl = synth.custom(2, 1, rank, dims, cid=79)
    for fmt in ("bf16", "fp8"):
        ow = OracleWorkload(wl, DEV, w0_format=fmt)
        b = sdev.load(wl, DEV, w0_format=fmt)
        for layer in range(2):
            for c in ("qkv", "gate_up", "q", "k", "gate"):
                x = wl.x(layer, c, 1, DEV)
                announce(f"long-K decode r={rank} {fmt} layer {layer} {c}")
                y = call(b, layer, c, x)
                torch.cuda.synchronize()
                res = compare(np64(y), ow.call(layer, c, np64(x)))
                assert res["ok"], f"{fmt} layer {layer} {c}: {res}"
            x = wl.x(layer, "gate_up", 1, DEV)
            h = b.gate_up_act(layer, "gelu_tanh", x)
            torch.cuda.synchronize()
            res = compare(np64(h), ow.gate_up_act(layer, np64(x), "gelu_tanh"))
            assert res["ok"], f"{fmt} layer {layer} gate_up_act: {res}"


@pytest.mark.parametrize("T", [1, 5, 16])
def test_small_call_decode_splits_vt(gpu_lib, T):
    """bf16 decode calls of fewer than 4096 rows with K >= 2048 split their
    V^T rows in two K slices (o here has 4104 rows and keeps them whole):
    ragged rows, K and rank, single, stacked and fused-activation calls,
    against the oracle."""
    dims = {(0, "q"): (200, 4104), (0, "k"): (40, 4104), (0, "v"): (40, 4104), (0, "o"): (4104, 200),
            (0, "gate"): (96, 2056), (0, "up"): (96, 2056), (0, "down"): (2056, 96)}
    wl = synth.custom(2, 1, 37, dims, cid=83)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        for c in ("qkv", "gate_up", "q", "o", "down"):
            x = wl.x(layer, c, T, DEV)
            announce(f"small-call decode T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            torch.cuda.synchronize()
            res = compare(np64(y), ow.call(layer, c, np64(x)))
            assert res["ok"], f"T={T} layer {layer} {c}: {res}"
        x = wl.x(layer, "gate_up", T, DEV)
        h = b.gate_up_act(layer, "silu", x)
        torch.cuda.synchronize()
        res = compare(np64(h), ow.gate_up_act(layer, np64(x), "silu"))
        assert res["ok"], f"T={T} layer {layer} gate_up_act: {res}"


@pytest.mark.parametrize("T", [1, 2])
def test_long_k_one_token_vt_blocks(gpu_lib, T):
    """One-token bf16 calls with K >= 5120 stream their V^T tiles (the whole
    K) in 8-step blocks; here K = 5130, so the last 32-k step is partial and
    the block count leaves a tail of single steps, with 4100-row children
    (no V^T split) and a ragged rank.  T = 2 takes the other kernels on the
    same bundle."""
    dims = {(0, "q"): (4100, 5128), (0, "k"): (1030, 5128), (0, "v"): (1030, 5128), (0, "o"): (5128, 4104),
            (0, "gate"): (4104, 5128), (0, "up"): (4104, 5128), (0, "down"): (5128, 4104)}
    wl = synth.custom(2, 1, 45, dims, cid=85)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        for c in ("qkv", "gate_up", "q", "o", "down"):
            x = wl.x(layer, c, T, DEV)
            announce(f"long-K one-token V^T blocks T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            torch.cuda.synchronize()
            res = compare(np64(y), ow.call(layer, c, np64(x)))
            assert res["ok"], f"T={T} layer {layer} {c}: {res}"


@pytest.mark.parametrize("T", [40, 200])
def test_split_k_finish_with_unaligned_scale(gpu_lib, T):
    """A single-family call's s is a row slice of its group's s: after a q of
    4098 rows, k's s starts 8 bytes past a 16-byte boundary.  k (520 rows, a
    multiple of 4, long K) takes the split-K finish path, which must not use
    16-byte loads of s there."""
    dims = {(0, "q"): (4098, 4096), (0, "k"): (520, 4096), (0, "v"): (520, 4096)}
    wl = synth.custom(1, 1, 32, dims, cid=78)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for c in ("k", "v", "qkv"):
        x = wl.x(0, c, T, DEV)
        announce(f"split-K finish, unaligned s, T={T} {c}")
        y = call(b, 0, c, x)
        torch.cuda.synchronize()
        res = compare(np64(y), ow.call(0, c, np64(x)))
        assert res["ok"], f"{c}: {res}"


@pytest.mark.parametrize("T", [1, 16, 40, 130])
def test_outputs_with_two_byte_alignment(gpu_lib, T):
    """y (and the fused gate|up h) need only 2-byte alignment: outputs written
    at an odd element offset are bitwise the aligned outputs (vector stores are
    taken only where the destination allows them)."""
    wl = ragged(5, layer_types=(0, 1), k_eq_v=(1,), bands=1)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        for c in ("qkv", "gate_up", "o", "down"):
            x = wl.x(layer, c, T, DEV)
            announce(f"2-byte aligned y T={T} layer {layer} {c}")
            y = call(b, layer, c, x)
            n = y.shape[1]
            buf = torch.zeros(T * n + 1, dtype=torch.bfloat16, device=DEV)
            yo = buf[1:].view(T, n)
            if c in ("qkv", "gate_up"):
                b.stacked(layer, c, x, y=yo)
            else:
                b.linear(layer, c, x, y=yo)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), yo.view(torch.int16)), f"layer {layer} {c}"
        x = wl.x(layer, "gate_up", T, DEV)
        h = b.gate_up_act(layer, "gelu_tanh", x)
        n = h.shape[1]
        buf = torch.zeros(T * n + 1, dtype=torch.bfloat16, device=DEV)
        ho = buf[1:].view(T, n)
        b.gate_up_act(layer, "gelu_tanh", x, h=ho)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ho.view(torch.int16)), f"layer {layer} gate_up_act"


@pytest.mark.parametrize("T", [7, 8, 13, 16])
def test_long_k_slices_several_tokens(gpu_lib, T):
    """Calls whose K slices are long (K = 16392: 65 k-steps of 32 per slice at
    8 slices; K = 8200: 33) with T >= 8 run the four-tile stream kernel with
    twice the waves, in 2-step blocks; ragged rows (100 and 300: partial
    64-row groups) and a K tail, against the oracle.  T = 7 takes the
    one-tile kernel."""
    dims = {(0, "o"): (300, 16392), (0, "down"): (100, 16392), (0, "q"): (300, 8200)}
    wl = synth.custom(2, 1, 5, dims, cid=61)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    for layer in range(2):
        for c in ("o", "down", "q"):
            x = wl.x(layer, c, T, DEV)
            announce(f"long K slices T={T} layer {layer} {c}")
            y = b.linear(layer, c, x)
            torch.cuda.synchronize()
            res = compare(np64(y), ow.call(layer, c, np64(x)))
            assert res["ok"], f"layer {layer} {c} T={T}: {res}"


@pytest.fixture(scope="module")
def four_tile_bundle(gpu_lib):
    # o: 1000 x 1064 (K slices of 5 k-steps, the last slice empty, a K tail);
    # down: 33000 x 4104 (4 slices of 33 k-steps, a K tail); both row counts
    # end in a partial 64-row group
    dims = {(0, "o"): (1000, 1064), (0, "down"): (33000, 4104)}
    wl = synth.custom(1, 1, 5, dims, cid=62)
    return wl, OracleWorkload(wl, DEV), sdev.load(wl, DEV)


@pytest.mark.parametrize("T", [8, 11, 16])
def test_four_row_tiles_many_tokens(four_tile_bundle, T):
    """From eight tokens on, calls whose several-token split stays within 8
    K slices at four row tiles per workgroup run the four-tile stream kernel:
    single k-steps for the short slices of o here, two-step blocks for the
    long slices of down; against the oracle, and bitwise run to run."""
    wl, ow, b = four_tile_bundle
    for c in ("o", "down"):
        x = wl.x(0, c, T, DEV)
        announce(f"four row tiles T={T} {c}")
        y = b.linear(0, c, x)
        y2 = b.linear(0, c, x)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), c
        res = compare(np64(y), ow.call(0, c, np64(x)))
        assert res["ok"], f"{c} T={T}: {res}"


@pytest.mark.parametrize("fam,N", [("gate", 4100), ("k", 264)])
def test_fused_z_ragged_large_calls(gpu_lib, fam, N):
    """Small-rank prefill calls with ragged rows, tokens and K (a K tail of 8):
    the gate-shaped call has 33 x 17 = 561 tiles of 128 x 128, enough for the
    fused-Z tile that runs two workgroups per CU; the k-shaped call takes the
    128 x 64 fused-Z tile with partial row and token tiles."""
    wl = synth.custom(1, 1, 40, {(0, fam): (N, 1160)}, cid=95)
    ow = OracleWorkload(wl, DEV)
    b = sdev.load(wl, DEV)
    x = wl.x(0, fam, 2050, DEV)
    announce(f"fused-Z ragged {fam} N={N} T=2050")
    y = b.linear(0, fam, x)
    torch.cuda.synchronize()
    res = compare(np64(y), ow.call(0, fam, np64(x)))
    assert res["ok"], res
    y2 = b.linear(0, fam, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
