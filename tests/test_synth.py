"""The seeded generator: same key, same bytes; different keys, different
streams; shapes and dtypes as the workloads state."""
import math

import torch

import synth


def test_same_seed_same_bytes():
    wl = synth.workload(1)
    a = wl.w0(0, 0, "up")
    b = wl.w0(0, 0, "up")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(wl.x(1, "up", 4), wl.x(1, "up", 4))


def test_keys_give_distinct_streams():
    wl = synth.workload(1)
    assert not torch.equal(wl.s(0, "up"), wl.s(1, "up"))
    assert not torch.equal(wl.u(0, "up"), wl.u(1, "up"))
    assert not torch.equal(wl.x(0, "up", 4), wl.x(1, "up", 4))


def test_workload_shapes_and_dtypes():
    wl = synth.workload(1)
    assert wl.w0(0, 0, "up").shape == (4096, 1152) and wl.w0(0, 0, "up").dtype == torch.bfloat16
    assert wl.s(0, "up").dtype == torch.float32 and wl.s(0, "up").shape == (4096,)
    assert wl.u(0, "up").shape == (4096, 4) and wl.v(0, "up").shape == (1152, 4)
    assert wl.x(0, "up", 4).shape == (4, 1152)
    s = wl.s(0, "up")
    assert abs(float(s.mean()) - 1.0) < 0.01 and abs(float(s.std()) - 0.05) < 0.005
    w = wl.w0(0, 0, "up").float()
    assert abs(float(w.std()) - 1 / math.sqrt(1152)) < 1e-3


def test_gemma_workloads():
    w2 = synth.workload(2)
    assert w2.num_layers == 26 and w2.num_bands == 13 and w2.decomposed
    assert synth.workload(2, "passthrough").num_bands == 26
    w5 = synth.workload(5)
    assert sum(w5.layer_types) == 10 and w5.layer_types[5] == 1 and w5.layer_types[0] == 0
    assert not w5.has(1, "v") and w5.shape(1, "v") == (8192, 5376)
    assert w5.shape(1, "q") == (16384, 5376) and w5.shape(0, "q") == (8192, 5376)
    w4 = synth.workload(4)
    import synth.device as sdev
    assert [sdev.band_of_layer(l, w4.num_layers, w4.num_bands) for l in (0, 11, 12, 59)] == [0, 0, 1, 4]
