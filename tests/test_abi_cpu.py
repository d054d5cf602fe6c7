"""The C ABI on the host: the library loads, exports every declared symbol,
sizes arenas and workspaces, and rejects bad arguments before anything is
enqueued (no device work here; every call below fails validation or touches
no HIP API)."""
import ctypes
import os
import re

import pytest

import synth
import synth.device as sdev
from weight_shared_rank_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_ARENA = 1 << 32  # never dereferenced: every use below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIBPATH):
        from weight_shared_rank_amd import build
        build.build(verbose=False)
    return binding.lib()


def declared_functions():
    with open(os.path.join(ROOT, "include", "weightless.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert set(decl) == set(binding.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def spec_for(cid, **kw):
    return sdev.spec_of(synth.workload(cid, **kw))


@pytest.mark.parametrize("cid,lo,hi", [(1, 9.5e6, 10.3e6), (2, 4.8e8, 4.9e8), (3, 1.1e8, 1.13e8),
                                       (4, 8.6e9, 8.8e9), (5, 1.70e10, 1.74e10)])
def test_arena_sizes(L, cid, lo, hi):
    n = binding.theta_bundle_arena_bytes(spec_for(cid))
    assert lo <= n <= hi and n % 256 == 0


def test_arena_counts_each_w0_once(L):
    """Workload 4 (G=5): W0 is stored once per band, per-layer data per layer."""
    wl = synth.workload(4)
    w0 = sum(n * k for (t, f), (n, k) in wl.dims.items()) * 2
    per_layer = sum(n * 4 + (n + k) * 256 * 2 for (t, f), (n, k) in wl.dims.items())
    n = binding.theta_bundle_arena_bytes(spec_for(4))
    assert abs(n - (5 * w0 + 60 * per_layer)) < 60 * 16 * 256 + 5 * 4 * 256


def bad_spec(**changes):
    sp = spec_for(2)
    for k, v in changes.items():
        setattr(sp, k, v)
    return sp


@pytest.mark.parametrize("changes,frag", [
    ({"num_layers": 0}, "num_layers"),
    ({"num_bands": 0}, "num_bands"),
    ({"num_bands": 27}, "num_bands"),
    ({"num_layer_types": 3}, "num_layer_types"),
    ({"k_eq_v_type_mask": 2}, "k_eq_v_type_mask"),
])
def test_invalid_spec_fields(L, changes, frag):
    sp = bad_spec(**changes)
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert frag in binding.last_error()


def test_invalid_shapes(L):
    sp = spec_for(2)
    sp.in_dim[0][0] = 1150                  # K % 8 != 0
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert "multiple of 8" in binding.last_error()
    sp = spec_for(2)
    sp.rank[0][1] = 300                     # rank > N = 256
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert "rank" in binding.last_error()
    sp = spec_for(2)
    sp.in_dim[0][1] = 1024                  # k's K differs from q's inside the QKV group
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert "in_dim" in binding.last_error()
    sp = spec_for(5)
    sp.out_dim[1][4] = 2048                 # MLP shape differs between layer types
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert "MLP" in binding.last_error()
    sp = spec_for(2)
    lt = (ctypes.c_int8 * 26)(*([0] * 25 + [1]))
    sp.layer_type = ctypes.cast(lt, ctypes.POINTER(ctypes.c_int8))
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 0
    assert "layer_type" in binding.last_error()


def load_status(L, sp, srcs, arena=FAKE_ARENA, nbytes=None):
    n = len(srcs)
    arr = (binding.WlSrc * max(n, 1))(*srcs)
    h = ctypes.c_void_p()
    if nbytes is None:
        nbytes = L.theta_bundle_arena_bytes(ctypes.byref(sp))
    st = L.theta_bundle_load(ctypes.byref(sp), arr, n, arena, nbytes, None, ctypes.byref(h))
    return st, binding.last_error()


def one_family_sources(valid_ptr=0x1000):
    wl = synth.workload(1)
    srcs = []
    for kind, idx, fam in [("w0", 0, "up")] + [(k, l, "up") for l in range(2) for k in ("s", "u", "v")]:
        s = binding.WlSrc()
        s.kind = binding.SRC_KIND[kind]
        s.index = idx
        s.layer_type = 0
        s.family = binding.FAMILY[fam]
        s.dtype = binding.WL_DTYPE_F32 if kind == "s" else binding.WL_DTYPE_BF16
        s.on_device = 1
        s.ptr = valid_ptr
        srcs.append(s)
    return wl, srcs


def test_load_argument_errors(L):
    wl, srcs = one_family_sources()
    sp = sdev.spec_of(wl)
    st, msg = load_status(L, sp, srcs, arena=0)
    assert st == -1 and "arena" in msg
    st, msg = load_status(L, sp, srcs, arena=FAKE_ARENA + 16)
    assert st == -1 and "aligned" in msg
    st, msg = load_status(L, sp, srcs, nbytes=1000)
    assert st == -5
    st, msg = load_status(L, sp, srcs[:-1])
    assert st == -1 and "missing" in msg
    st, msg = load_status(L, sp, srcs + [srcs[0]])
    assert st == -1 and "duplicates" in msg
    bad = binding.WlSrc.from_buffer_copy(srcs[1])
    bad.dtype = binding.WL_DTYPE_BF16       # s must be float32
    st, msg = load_status(L, sp, [srcs[0], bad] + srcs[2:])
    assert st == -3
    extra = binding.WlSrc.from_buffer_copy(srcs[1])
    extra.family = binding.FAMILY["gate"]   # gate is absent in this bundle
    st, msg = load_status(L, sp, srcs + [extra])
    assert st == -1 and "not part" in msg
    nullp = binding.WlSrc.from_buffer_copy(srcs[2])
    nullp.ptr = None
    st, msg = load_status(L, sp, [srcs[0], srcs[1], nullp] + srcs[3:])
    assert st == -1 and "NULL" in msg
    h = ctypes.c_void_p()
    assert L.theta_bundle_load(None, None, 0, FAKE_ARENA, 0, None, ctypes.byref(h)) == -1


def test_tied_v_takes_no_sources(L):
    """On a K=V-tied layer type no v source is expected; passing one is an error."""
    wl = synth.custom(2, 1, 4, {(0, "q"): (64, 64), (0, "k"): (32, 64), (0, "v"): (32, 64)},
                      k_eq_v_types=(0,))
    sp = sdev.spec_of(wl)
    srcs = []
    for kind, idx, fam in [("w0", 0, "q"), ("w0", 0, "k")] + [(k, l, f) for l in range(2) for f in ("q", "k")
                                                             for k in ("s", "u", "v")]:
        s = binding.WlSrc()
        s.kind, s.index, s.layer_type, s.family = binding.SRC_KIND[kind], idx, 0, binding.FAMILY[fam]
        s.dtype = binding.WL_DTYPE_F32 if kind == "s" else binding.WL_DTYPE_BF16
        s.on_device, s.ptr = 1, 0x1000
        srcs.append(s)
    extra = binding.WlSrc.from_buffer_copy(srcs[0])
    extra.family = binding.FAMILY["v"]
    st, msg = load_status(L, sp, srcs + [extra], nbytes=10)  # nbytes too small is checked before sources
    assert st == -5
    st, msg = load_status(L, sp, srcs + [extra], arena=FAKE_ARENA, nbytes=1 << 30)
    assert st == -1 and "not part" in msg


def test_empty_bundle_and_null_handles(L):
    """A spec with every family absent needs only the 256-byte zero block;
    loads that fail validation and calls on a NULL handle return before any
    HIP call."""
    sp = binding.make_spec(4, 2, {}, {})
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp)) == 256
    h = ctypes.c_void_p()
    assert L.theta_bundle_load(ctypes.byref(sp), None, 0, FAKE_ARENA, 0, None, ctypes.byref(h)) == -5
    assert L.theta_bundle_load(ctypes.byref(sp), None, 0, 0, 256, None, ctypes.byref(h)) == -1
    assert L.theta_bundle_load(ctypes.byref(sp), None, 0, FAKE_ARENA, 256, None, None) == -1
    assert L.theta_bundle_free(None) == 0
    assert L.weightless_linear(None, 0, 0, FAKE_ARENA, 1, FAKE_ARENA, FAKE_ARENA, 1, None) == -1
    assert L.weightless_stacked_linear(None, 0, 0, FAKE_ARENA, 1, FAKE_ARENA, FAKE_ARENA, 1, None) == -1
    assert L.weightless_workspace_bytes(None, 1) == 0
    assert L.weightless_out_dim(None, 0, 0, -1) == 0
    assert L.weightless_materialize_workspace_bytes(None) == 0
    assert L.weightless_materialize(None, 0, 0, FAKE_ARENA, FAKE_ARENA, 1 << 20, None) == -1


def test_fp8_spec_and_sources(L):
    """w0_format: unknown values are rejected; an FP8 bundle is smaller (one
    byte per W0 element, rows padded to 16 bytes, one fp32 scale per row) and
    takes W0 only from device memory (checked before any HIP call)."""
    import synth
    import synth.device as sdev
    wl = synth.workload(1)
    sp = sdev.spec_of(wl)
    sp8 = sdev.spec_of(wl, "fp8")
    n16, n8 = L.theta_bundle_arena_bytes(ctypes.byref(sp)), L.theta_bundle_arena_bytes(ctypes.byref(sp8))
    w0 = 4096 * 1152
    assert n16 - n8 == w0 - 4096 * 4
    sp8.w0_format = 3
    assert L.theta_bundle_arena_bytes(ctypes.byref(sp8)) == 0
    assert "w0_format" in binding.last_error()
    # MXFP4: half a byte per element (rows padded to 128 elements) and one
    # E8M0 byte per 32 elements
    sp4 = sdev.spec_of(wl, "mxfp4")
    n4 = L.theta_bundle_arena_bytes(ctypes.byref(sp4))
    assert n16 - n4 == 2 * w0 - (w0 // 2 + 4096 * 1152 // 32)
    sp8.w0_format = 1
    import numpy as np
    host = np.zeros((4096, 1152), np.uint16)
    srcs = (binding.WlSrc * 1)()
    srcs[0].kind, srcs[0].index, srcs[0].layer_type, srcs[0].family = 0, 0, 0, binding.FAMILY["up"]
    srcs[0].dtype, srcs[0].on_device, srcs[0].ptr = 0, 0, host.ctypes.data
    h = ctypes.c_void_p()
    assert L.theta_bundle_load(ctypes.byref(sp8), srcs, 1, FAKE_ARENA, n8, None, ctypes.byref(h)) == -1
    assert "device" in binding.last_error()


def test_decompose_workspace_and_argument_errors(L):
    """weightless_decompose: workspace sizing, and every argument error is
    reported before any HIP call."""
    ws = L.weightless_decompose_workspace_bytes(4096, 1152, 32, 8)
    # fp32 residual + 2 (N x l) + 2 (K x l) + (l x K) + (l x l) + N x r + K x r
    # + 16 max(N, K) x l split-K partials, l = 40
    expect = 4 * (4096 * 1152 + 2 * 4096 * 40 + 2 * 1152 * 40 + 40 * 1152 + 40 * 40 + 4096 * 32 + 1152 * 32
                  + 16 * 4096 * 40)
    assert expect <= ws <= expect + 10 * 256
    assert L.weightless_decompose_workspace_bytes(0, 8, 1, 0) == 0
    assert L.weightless_decompose_workspace_bytes(8, 8, -1, 0) == 0
    assert binding.sketch_columns(100, 64, 60, 8) == 64
    big = 1 << 30
    args = dict(w=FAKE_ARENA, m=2, N=64, K=48, rank=8, over=4, q=2, omega=FAKE_ARENA, w0=FAKE_ARENA,
                s=FAKE_ARENA, u=FAKE_ARENA, v=FAKE_ARENA, ws=FAKE_ARENA, wsb=big)

    def call(**kw):
        a = dict(args, **kw)
        return L.weightless_decompose(a["w"], a["m"], a["N"], a["K"], a["rank"], a["over"], a["q"], a["omega"],
                                      a["w0"], a["s"], a["u"], a["v"], a["ws"], a["wsb"], None)

    assert call(rank=49) == -2 and "rank" in binding.last_error()
    assert call(m=0) == -1
    assert call(q=17) == -1
    assert call(w=None) == -1 and "NULL" in binding.last_error()
    assert call(omega=None) == -1
    assert call(ws=FAKE_ARENA + 16) == -1 and "aligned" in binding.last_error()
    assert call(wsb=1024) == -5


def test_library_shares_torchs_hip_runtime(L):
    """Loading the library before anything imports torch still leaves one HIP
    runtime in the process (torch's): a second, system runtime beside it
    would find no device.  Run in a fresh interpreter, binding first."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from weight_shared_rank_amd import binding\n"
            "binding.lib()\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps), sorted(maps))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[0] == "1", out.stdout
