"""weightless_linear_noalloc: the call on the library's fixed device workspace
gives what weightless_linear gives with a caller workspace, call after call.

Both entry points run the same kernels, so the outputs are compared bit for
bit.  Two calls in a row, the second with a smaller input (fewer tokens and a
family with fewer rows), so the second call sees the first call's leftovers
in the shared array; decode (T <= 16) and prefill (T > 16) calls; and a call
whose workspace would exceed the array is refused before anything runs.
"""
import ctypes
import sys

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


def _bundle():
    dims = {(0, "q"): (1000, 1024), (0, "k"): (264, 1024), (0, "v"): (264, 1024), (0, "o"): (1024, 1000 + 24),
            (0, "gate"): (2056, 1024), (0, "up"): (2056, 1024), (0, "down"): (1024, 2056 + 8)}
    wl = synth.custom(2, 1, 40, dims, cid=91)
    return wl, sdev.load(wl, DEV)


@pytest.mark.parametrize("first,second", [((1, "gate", 16), (0, "k", 3)),
                                          ((1, "down", 96), (0, "o", 40)),
                                          ((0, "up", 200), (1, "v", 1))])
def test_noalloc_matches_workspace_call(gpu_lib, first, second):
    wl, b = _bundle()
    ow = OracleWorkload(wl, DEV)
    for layer, fam, T in (first, second):
        x = wl.x(layer, fam, T, DEV, salt=7)
        announce(f"noalloc layer {layer} {fam} T={T}")
        y_ws = b.linear(layer, fam, x)
        y_na = b.linear_noalloc(layer, fam, x)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), (layer, fam, T)
        res = compare(np64(y_na), ow.call(layer, fam, np64(x)))
        assert res["ok"], f"layer {layer} {fam} T={T}: {res}"


def test_noalloc_refuses_oversized_calls(gpu_lib):
    """A bundle whose prefill workspace exceeds the fixed array: WL_ENOSPACE,
    returned on the host before any launch; decode calls still run."""
    dims = {(0, "down"): (1024, 1024)}
    wl = synth.custom(1, 1, 1024, dims, cid=92)
    b = sdev.load(wl, DEV)
    T = 40000                      # Z = X V alone is T x 1024 bf16 = 82 MB
    assert b.workspace_bytes(T) > binding.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((T, 1024), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((T, 1024), dtype=torch.bfloat16, device=DEV)
    st = binding.lib().weightless_linear_noalloc(b.handle, 0, binding.FAMILY["down"], x.data_ptr(), T,
                                                 y.data_ptr(), None)
    assert st == -5 and "fixed workspace" in binding.last_error()
    x1 = wl.x(0, "down", 2, DEV)
    torch.cuda.synchronize()
    assert torch.equal(b.linear_noalloc(0, "down", x1).view(torch.int16), b.linear(0, "down", x1).view(torch.int16))
