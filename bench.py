"""Benchmark of the weightless linear on one MI355X.

A decode step is one pass of every layer's linears of the Gemma-4-31B-shaped
sliding-attention workload at T=1 (60 layers x [stacked q|k|v, o, stacked
gate|up, down], G=5 bands, rank 256), replayed from a captured HIP graph with
the bundle and activations resident in HBM.  value = algorithmic bytes read
per step (W0 + s + U + V^T + x of every call) / step time.

The same run also times
  * the same step at T=16,
  * the Gemma-3-1B-shaped decode step (G=13, r=32, T=1),
  * prefill steps (MFMA path): Gemma-4-31B mixed attention (10 full + 50
    sliding layers, G=1 per type, r=1024, T=512) and Gemma-3-1B (G=1, r=64,
    T=2048, 7 single-family calls per layer; and, as a secondary figure, the
    same layers as 4 calls with q|k|v and gate|up stacked), in TFLOP/s,
  * the roofline figure: the step's GPU time from HIP events recorded on the
    replay stream around the timed replays, per call, and per call type the
    durations of eager calls between HIP events on the launch stream, and
  * the fp64 CPU oracle on a bounded sample of the headline workload,
  * the GPU decomposition of the Gemma-3-1B-shaped model (13 bands x 7
    families, rank 32) against the oracle's exact decomposition.

Prints one JSON line.  Runs on one GPU only.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
CALLS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))


def band_of_layer(layer, num_layers, num_bands):
    from synth.device import band_of_layer as b
    return b(layer, num_layers, num_bands)


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def w0_bytes(N, K, w0_format):
    """Bytes of one W0 block: bf16 2NK; FP8 NK codes plus 4N of row scales;
    MXFP4 NK/2 codes plus one scale byte per 32 elements."""
    if w0_format == "fp8":
        return N * K + 4 * N
    if w0_format == "mxfp4":
        return N * K // 2 + N * ((K + 31) // 32)
    return 2 * N * K


def call_bytes(wl, layer, fams, T, w0_format="bf16"):
    """Algorithmic bytes a call must read: W0 (2NK in bf16) + 4N (s) + 2Nr
    (U) + 2Kr (V^T) per child, plus 2TK (x) once; and the bytes it writes
    (2TN)."""
    lt = wl.layer_types[layer]
    rd = 0
    wr = 0
    K = None
    for f in fams:
        N, K = wl.shape(lt, f)
        if not wl.has(lt, f):        # tied v: output copy, no bundle read
            wr += 2 * T * N
            continue
        r = wl.clamped_rank(lt, f)
        rd += w0_bytes(N, K, w0_format) + 4 * N + 2 * N * r + 2 * K * r
        wr += 2 * T * N
    return rd + 2 * T * K, wr


def call_flops(wl, layer, fams, T):
    lt = wl.layer_types[layer]
    fl = 0
    for f in fams:
        if not wl.has(lt, f):
            continue
        N, K = wl.shape(lt, f)
        r = wl.clamped_rank(lt, f)
        fl += 2 * T * N * K + 2 * T * K * r + 2 * T * N * r
    return fl


class Step:
    """Every call of every layer (or of the given layers), with preallocated
    inputs and outputs."""

    def __init__(self, wl, bundle, T, calls, dev, layers=None, w0_format="bf16"):
        import torch
        self.items = []
        self.bytes_rd = 0
        # the same bytes with each band's W0 counted once for the step (the
        # floor if every re-read of a band-shared W0 hit a cache)
        self.bytes_band_unique = 0
        seen_w0 = set()
        self.bytes_wr = 0
        self.flops = 0
        self.per_call = {}
        for layer in (range(wl.num_layers) if layers is None else layers):
            for name, fams in calls:
                lt = wl.layer_types[layer]
                fams_here = [f for f in fams if (lt, f) in wl.dims or (f == "v" and lt in wl.k_eq_v_types)]
                x = wl.x(layer, name, T, dev)
                stacked = len(fams) > 1
                width = bundle.out_dim(layer, stack=name) if stacked else bundle.out_dim(layer, family=name)
                y = torch.empty((T, width), dtype=torch.bfloat16, device=dev)
                rd, wr = call_bytes(wl, layer, fams_here, T, w0_format)
                fl = call_flops(wl, layer, fams_here, T)
                self.items.append((layer, name, stacked, x, y))
                self.bytes_rd += rd
                self.bytes_band_unique += rd
                for f in fams_here:
                    if not wl.has(lt, f):
                        continue
                    key = (band_of_layer(layer, wl.num_layers, wl.num_bands), 0 if f in ("gate", "up", "down") else lt, f)
                    if key in seen_w0:
                        N, K = wl.shape(lt, f)
                        self.bytes_band_unique -= w0_bytes(N, K, w0_format)
                    seen_w0.add(key)
                self.bytes_wr += wr
                self.flops += fl
                pc = self.per_call.setdefault(name, {"calls": 0, "bytes": 0, "flops": 0})
                pc["calls"] += 1
                pc["bytes"] += rd
                pc["flops"] += fl
        self.bundle = bundle
        self.ws = bundle.workspace(T)

    def run(self):
        b, ws = self.bundle, self.ws
        for layer, name, stacked, x, y in self.items:
            if stacked:
                b.stacked(layer, name, x, y=y, ws=ws)
            else:
                b.linear(layer, name, x, y=y, ws=ws)


def time_graph(step, steps, warmup, with_events=False):
    """Capture the step in a HIP graph; time `steps` replays after `warmup`
    (host clock, synchronized on both sides).  with_events: also return the
    per-step GPU time from HIP events recorded on the replay stream around
    the same timed replays (the launches of the step run on that stream)."""
    import torch
    step.run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step.run()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t_host = (time.perf_counter() - t0) / steps
    if with_events:
        return t_host, g, e0.elapsed_time(e1) * 1e-3 / steps
    return t_host, g


def time_launches(step, reps):
    """Per-call-type average duration with HIP events recorded on the launch
    stream around each call, in step order (so W0 re-reads across layers see
    the same cache state as in the step).  The GPU is first parked on a short
    spin so the host enqueues every call before the GPU reaches them: the
    event pairs then bracket GPU work only, not host launch gaps."""
    import torch
    names = list(step.per_call)
    evs = []
    torch.cuda.synchronize()
    # ~60 us of host enqueue work per call; spin the GPU that long (2.4 GHz)
    torch.cuda._sleep(int(2.4e9 * 60e-6 * len(step.items) * reps) + 10_000_000)
    for _ in range(reps):
        for layer, name, stacked, x, y in step.items:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if stacked:
                step.bundle.stacked(layer, name, x, y=y, ws=step.ws)
            else:
                step.bundle.linear(layer, name, x, y=y, ws=step.ws)
            e1.record()
            evs.append((name, e0, e1))
    torch.cuda.synchronize()
    tot = {n: 0.0 for n in names}
    cnt = {n: 0 for n in names}
    for name, e0, e1 in evs:
        tot[name] += e0.elapsed_time(e1) * 1e-3
        cnt[name] += 1
    return {n: tot[n] / cnt[n] for n in names}


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "weight_shared_rank_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(key, sha):
    """HBM bytes per call, read plus written, from the committed rocprofv3
    counter summary (profiles/counters.json: calibrated FETCH_SIZE and
    WRITE_SIZE), with the two parts, if it was taken on the current kernel
    source; else (None, None, None)."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None, None, None
    with open(p) as f:
        d = json.load(f)
    rec = d.get(key)
    if not rec or rec.get("source_sha") != sha:
        return None, None, None
    rd, wr = rec.get("hbm_bytes_per_call"), rec.get("hbm_write_bytes_per_call")
    return (rd + wr if rd is not None and wr is not None else None), rd, wr


def decode_section(wl, T, steps, warmup, dev, reps=3, w0_format="bf16"):
    import synth.device as sdev
    import torch
    log(f"load {wl.name} ({w0_format} W0)")
    bundle = sdev.load(wl, dev, w0_format=w0_format)
    torch.cuda.synchronize()
    step = Step(wl, bundle, T, CALLS, dev, w0_format=w0_format)
    t_step, g, t_ev = time_graph(step, steps, warmup, with_events=True)
    durs = time_launches(step, reps)
    launches = sum(pc["calls"] for pc in step.per_call.values())
    per_call = {}
    for n, pc in step.per_call.items():
        b_per = pc["bytes"] / pc["calls"]
        per_call[n] = {"bytes": b_per, "us": durs[n] * 1e6, "GBps": b_per / durs[n] / 1e9,
                       "hbm_frac": b_per / durs[n] / 1e9 / HBM_PEAK_GBS}
    kern_time = sum(durs[n] * pc["calls"] for n, pc in step.per_call.items())
    out = {"step_s": t_step, "bytes_read": step.bytes_rd, "bytes_written": step.bytes_wr,
           "GBps": step.bytes_rd / t_step / 1e9, "launches": launches,
           "bytes_band_unique": step.bytes_band_unique, "GBps_band_unique": step.bytes_band_unique / t_step / 1e9,
           "kernel_GBps": step.bytes_rd / kern_time / 1e9,
           "avg_launch_us": kern_time / launches * 1e6, "bytes_per_launch": step.bytes_rd / launches,
           "graph_event_call_us": t_ev / launches * 1e6, "graph_event_GBps": step.bytes_rd / t_ev / 1e9,
           "per_call": per_call}
    del g, step, bundle
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def prefill_section(wl, T, calls, steps, warmup, dev, reps=1):
    import synth.device as sdev
    import torch
    log(f"load {wl.name}")
    bundle = sdev.load(wl, dev)
    torch.cuda.synchronize()
    step = Step(wl, bundle, T, calls, dev)
    t_step, g, t_ev = time_graph(step, steps, warmup, with_events=True)
    durs = time_launches(step, reps)
    launches = sum(pc["calls"] for pc in step.per_call.values())
    per_call = {n: {"flops": pc["flops"] / pc["calls"], "us": durs[n] * 1e6,
                    "TFLOPs": pc["flops"] / pc["calls"] / durs[n] / 1e12} for n, pc in step.per_call.items()}
    kern_time = sum(durs[n] * pc["calls"] for n, pc in step.per_call.items())
    out = {"step_s": t_step, "flops": step.flops, "TFLOPs": step.flops / t_step / 1e12,
           "mfma_frac": step.flops / t_step / 1e12 / BF16_PEAK_TFLOPS,
           "call_TFLOPs": step.flops / kern_time / 1e12, "calls": launches,
           "avg_call_us": kern_time / launches * 1e6, "flops_per_call": step.flops / launches,
           "graph_event_call_us": t_ev / launches * 1e6, "graph_event_TFLOPs": step.flops / t_ev / 1e12,
           "per_call": per_call}
    del g, step, bundle
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def dense_comparison(wl, T, nlayers, steps, warmup, dev):
    """The weightless step against the dense weight it stands for, on the
    first nlayers layers (one band of the headline workload).  W_eff =
    diag(s) W0 + U V^T of every family is materialized by the library; the
    dense step then runs (a) the same decode kernels on a rank-0 bundle whose
    per-layer W0 is W_eff and s = 1, and (b) torch.matmul (hipBLASLt) on the
    same W_eff, as another system's reference.  Same x, same call order."""
    import torch
    import synth
    import synth.device as sdev
    layers = list(range(nlayers))
    bundle = sdev.load(wl, dev)
    wstep = Step(wl, bundle, T, CALLS, dev, layers=layers)
    t_w, g = time_graph(wstep, steps, warmup)
    del g
    # materialize every family of every layer
    weff = {}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mat_bytes = 0
    e0.record()
    for l in layers:
        for f in synth.FAMILIES:
            if (0, f) in wl.dims:
                weff[(l, f)] = bundle.materialize(l, f)
                mat_bytes += weff[(l, f)].numel() * 2
    e1.record()
    torch.cuda.synchronize()
    t_mat = e0.elapsed_time(e1) * 1e-3
    dims = {k: v for k, v in wl.dims.items() if k[0] == 0}
    dwl = synth.custom(nlayers, nlayers, 0, dims, cid=wl.cid)

    def tensors(kind, index, ltype, fam):
        if kind == "w0":
            return weff[(index, fam)]
        return torch.ones(wl.shape(0, fam)[0], dtype=torch.float32, device=dev)
    dense = sdev.load(dwl, dev, tensors=tensors)
    dstep = Step(dwl, dense, T, CALLS, dev)
    # same activations as the weightless step
    for (l, n, st, x, y), (l2, n2, st2, x2, y2) in zip(wstep.items, dstep.items):
        x2.copy_(x)
    t_d, g = time_graph(dstep, steps, warmup)
    del g
    dense_bytes = sum(weff[k].numel() * 2 for k in weff)
    # torch.matmul on the concatenated dense weights of each call
    wcat = {}
    for l in layers:
        for name, fams in CALLS:
            wcat[(l, name)] = torch.cat([weff[(l, f)] for f in fams], dim=0)
    ys = [torch.empty((T, wcat[(l, n)].shape[0]), dtype=torch.bfloat16, device=dev)
          for (l, n, st, x, y) in wstep.items]

    class _Mm:
        def run(self):
            for (l, n, st, x, y), yo in zip(wstep.items, ys):
                torch.matmul(x, wcat[(l, n)].t(), out=yo)
    try:
        t_t, g = time_graph(_Mm(), steps, warmup)
        del g
    except Exception as e:          # reference only: never fail the bench on it
        log(f"hipBLASLt reference skipped: {e}")
        t_t = float("nan")
    del dense, bundle, weff, wcat
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"layers": nlayers, "tokens": T,
            "weightless_ms": t_w * 1e3, "weightless_GBps": wstep.bytes_rd / t_w / 1e9,
            "weightless_bytes": wstep.bytes_rd,
            "dense_ms": t_d * 1e3, "dense_GBps": dense_bytes / t_d / 1e9, "dense_bytes": dense_bytes,
            "hipblaslt_dense_ms": t_t * 1e3, "hipblaslt_dense_GBps": dense_bytes / t_t / 1e9,
            "weightless_over_dense": t_w / t_d, "weightless_over_hipblaslt_dense": t_w / t_t,
            "materialize_ms": t_mat * 1e3, "materialize_GBps_written": mat_bytes / t_mat / 1e9}


def gate_up_act_section(wl, T, steps, warmup, dev, act="gelu_tanh"):
    """The gate|up stack of every layer with the MLP activation fused
    (weightless_gate_up_act, h [T, N]) against the stacked call (y [T, 2N])
    followed by the activation and product in torch: graph-replayed, per
    call."""
    import torch
    import torch.nn.functional as F
    import synth.device as sdev
    bundle = sdev.load(wl, dev)
    n = wl.shape(0, "gate")[0]
    xs = [wl.x(l, "gate_up", T, dev) for l in range(wl.num_layers)]
    ys = [torch.empty((T, 2 * n), dtype=torch.bfloat16, device=dev) for _ in xs]
    hs = [torch.empty((T, n), dtype=torch.bfloat16, device=dev) for _ in xs]
    ws = bundle.workspace(T)

    class _Fused:
        def run(self):
            for l, (x, h) in enumerate(zip(xs, hs)):
                bundle.gate_up_act(l, act, x, h=h, ws=ws)

    class _Unfused:
        def run(self):
            for l, (x, y, h) in enumerate(zip(xs, ys, hs)):
                bundle.stacked(l, "gate_up", x, y=y, ws=ws)
                torch.mul(F.gelu(y[:, :n], approximate="tanh"), y[:, n:], out=h)
    t_f, g = time_graph(_Fused(), steps, warmup)
    del g
    t_u, g = time_graph(_Unfused(), steps, warmup)
    del g, bundle
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    L = wl.num_layers
    return {"tokens": T, "layers": L, "fused_us_per_call": t_f / L * 1e6, "unfused_us_per_call": t_u / L * 1e6,
            "speedup": t_u / t_f, "h_bytes_written_per_call": 2 * T * n, "y_bytes_written_per_call": 4 * T * n}


def cpu_baseline(wl, T, budget_s, dev):
    """The fp64 oracle (as it stands) on one layer's four calls of the
    headline workload, repeated until about budget_s of CPU time."""
    import numpy as np
    from oracle import forward
    from oracle.workload import OracleWorkload
    ow = OracleWorkload(wl, dev, cache_w0=8)
    layer = 0
    prepared = []
    nbytes = 0
    for name, fams in CALLS:
        x = wl.x(layer, name, T, dev).float().cpu().double().numpy()
        children = [ow.params(layer, f) for f in fams]
        prepared.append((x, children))
        nbytes += call_bytes(wl, layer, fams, T)[0]
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max((i.get("num_threads", 1) for i in info), default=1)
    except Exception:
        cores = os.cpu_count()
    n = 0
    t0 = time.perf_counter()
    while True:
        for x, children in prepared:
            forward.stacked(x, children)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 5000:
            break
    blas = "unknown BLAS"
    try:
        import threadpoolctl
        libs = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return {"value": nbytes * n / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle ({blas}), layer 0 of the headline workload (4 calls, {nbytes/1e9:.3f} GB "
                      f"of bundle bytes), repeated {n}x in {el:.1f} s; W0/s/U/V pre-upcast to fp64 outside the timing"}


def _host_info():
    """Threads the host BLAS uses and its name."""
    cores, blas = os.cpu_count(), "unknown BLAS"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        libs = [i for i in info if i.get("user_api") == "blas"]
        if libs:
            cores = libs[0].get("num_threads", cores)
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return cores, blas


def _oracle_children(ow, wl, layer, fams):
    """fp64 parameters of a call's children (k's bundle again for a tied v),
    upcast outside any timing."""
    out = []
    for f in fams:
        if ow.tied(layer, f):
            out.append("dup")
        elif (wl.layer_types[layer], f) in wl.dims:
            out.append(ow.params(layer, f))
    return out


def oracle_calls_timing(wl, T, layers, calls, dev, repeats=1, budget_s=None):
    """The fp64 oracle (as it stands: oracle.forward on numpy's BLAS) on
    every call of the given layers.  Each call is timed `repeats` times and
    its median kept (or, with budget_s, the layers' calls are repeated until
    about budget_s has passed).  Returns seconds per pass over the calls,
    algorithmic bytes and flops of one pass, and the pass count."""
    import statistics
    import numpy as np
    from oracle import forward
    from oracle.workload import OracleWorkload
    ow = OracleWorkload(wl, dev, cache_w0=16)
    prepared = []
    nbytes = nflops = 0
    for layer in layers:
        for name, fams in calls:
            fams_here = [f for f in fams if (wl.layer_types[layer], f) in wl.dims or ow.tied(layer, f)]
            x = wl.x(layer, name, T, dev).float().cpu().double().numpy()
            prepared.append((x, _oracle_children(ow, wl, layer, fams_here)))
            nbytes += call_bytes(wl, layer, fams_here, T)[0]
            nflops += call_flops(wl, layer, fams_here, T)
    del ow

    def one(x, ch):
        return forward.stacked(x, ch) if len(ch) > 1 else forward.factored(x, *ch[0])
    if budget_s is not None:
        n = 0
        t0 = time.perf_counter()
        while True:
            for x, ch in prepared:
                one(x, ch)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 5000:
                break
        return el / n, nbytes, nflops, n
    per_call = []
    for x, ch in prepared:
        ts = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            one(x, ch)
            ts.append(time.perf_counter() - t0)
        per_call.append(statistics.median(ts))
    return sum(per_call), nbytes, nflops, repeats


def oracle_prefill_baselines(dev):
    """The fp64 oracle beside the prefill figures: the Gemma-4-31B mixed
    prefill (T=512) on one sliding and one full-attention layer, every call
    once; the Gemma-3-1B prefill (T=2048) on one layer's seven single-family
    calls, median of 3."""
    import synth
    cores, blas = _host_info()
    w5 = synth.workload(5)
    full = w5.layer_types.index(1)
    t5, _, f5, _ = oracle_calls_timing(w5, 512, [0, full], CALLS, dev, repeats=1)
    singles = tuple((f, (f,)) for f in synth.FAMILIES)
    t3, _, f3, _ = oracle_calls_timing(synth.workload(3), 2048, [0], singles, dev, repeats=3)
    return {"value": f5 / t5 / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle ({blas}) on the gemma4-31b mixed prefill at T=512: layer 0 (sliding) and "
                      f"layer {full} (full attention), each call once: {f5 / 1e12:.3f} TFLOP in {t5:.2f} s; "
                      f"parameters pre-upcast to fp64 outside the timing",
            "gemma3_1b_T2048": {"value": f3 / t3 / 1e12, "unit": "TFLOP/s",
                                "sample": f"layer 0, 7 single-family calls, median of 3 per call: "
                                          f"{f3 / 1e9:.1f} GFLOP in {t3:.3f} s"}}


def oracle_small_decode_baselines(dev, budget_s=2.0):
    """The fp64 oracle on the two small decode workloads: the one-family
    workload (both layers' calls, T=4, median of 3) and the Gemma-3-1B
    shapes at T=1 (one layer's four calls, repeated for about budget_s)."""
    import synth
    cores, blas = _host_info()
    w1 = synth.workload(1)
    t1, b1, _, _ = oracle_calls_timing(w1, 4, [0, 1], (("up", ("up",)),), dev, repeats=3)
    w2 = synth.custom(26, 13, 32, dict(synth.workload(2).dims), cid=2)
    t2, b2, _, n2 = oracle_calls_timing(w2, 1, [0], CALLS, dev, budget_s=budget_s)
    return {"cores": cores, "blas": blas,
            "one_family_T4": {"GBps": b1 / t1 / 1e9, "us_per_call": t1 / 2 * 1e6,
                              "sample": "both layers' up calls, median of 3 each"},
            "gemma3_1b_T1": {"GBps": b2 / t2 / 1e9, "us_per_layer": t2 * 1e6,
                             "sample": f"layer 0's four calls repeated {n2}x"}}


def workload1_section(dev, steps, warmup, copies=64):
    """The one-family workload (W0 4096 x 1152 shared by 2 layers, r=4, T=4)
    as back-to-back graph-replayed calls, layer 0 then layer 1 (the second
    re-reads the first's W0).  cold: the calls rotate through `copies`
    bundle copies (distinct arenas, a working set of copies x 9.6 MB, over
    twice the 256 MB Infinity Cache), so each pair starts from HBM; warm:
    every pair on one bundle."""
    import torch
    import synth
    import synth.device as sdev
    wl = synth.workload(1)
    bundles = [sdev.load(wl, dev) for _ in range(copies)]
    xs = [wl.x(l, "up", 4, dev) for l in (0, 1)]
    y = torch.empty((4, 4096), dtype=torch.bfloat16, device=dev)
    ws = bundles[0].workspace(4)
    nbytes = sum(call_bytes(wl, l, ["up"], 4)[0] for l in (0, 1))

    class _Run:
        def __init__(self, bs):
            self.bs = bs

        def run(self):
            for b in self.bs:
                for l in (0, 1):
                    b.linear(l, "up", xs[l], y=y, ws=ws)
    t_cold, g = time_graph(_Run(bundles), steps, warmup)
    del g
    t_warm, g = time_graph(_Run([bundles[0]] * copies), steps, warmup)
    del g, bundles
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    calls = 2 * copies
    return {"calls_per_replay": calls, "copies": copies, "bytes_per_call": nbytes / 2,
            "cold_us_per_call": t_cold / calls * 1e6, "cold_GBps": nbytes * copies / t_cold / 1e9,
            "warm_us_per_call": t_warm / calls * 1e6, "warm_GBps": nbytes * copies / t_warm / 1e9}


def band_reuse_ab(dev, steps, warmup):
    """Band reuse of W0, as an A/B of graph-replayed decode steps (T=1) with
    the same kernels, launches and bytes, where only the W0 addresses
    differ: a bundle whose consecutive layers share W0 (a band) against one
    with a distinct W0 per layer.  The step-time difference is what the
    re-reads of a shared W0 save (Infinity Cache or L2 hits).
      gemma3-1b shapes, 26 layers: G=13 (two layers per band) vs G=26;
      gemma4-31b sliding shapes, 12 layers: G=1 (one band, as band 0 of the
      G=5 bundle) vs G=12."""
    import torch
    import synth
    import synth.device as sdev
    out = []
    for name, dims, L, (g_shared, g_distinct), r in (
            ("gemma3-1b", dict(synth.workload(2).dims), 26, (13, 26), 32),
            ("gemma4-31b-sliding", dict(synth.workload(4).dims), 12, (1, 12), 256)):
        rec = {"shapes": name, "layers": L, "rank": r}
        for label, G in (("shared", g_shared), ("distinct", g_distinct)):
            wl = synth.custom(L, G, r, dims, cid=70 + G)
            bundle = sdev.load(wl, dev)
            step = Step(wl, bundle, 1, CALLS, dev)
            t, g = time_graph(step, steps, warmup)
            rec[label] = {"bands": G, "step_us": t * 1e6, "GBps": step.bytes_rd / t / 1e9,
                          "bytes_band_unique": step.bytes_band_unique}
            rec["bytes_read_per_step"] = step.bytes_rd
            del g, step, bundle
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        rec["saving_us"] = rec["distinct"]["step_us"] - rec["shared"]["step_us"]
        rec["saving_frac"] = rec["saving_us"] / rec["distinct"]["step_us"]
        log(f"band reuse A/B {name}: shared {rec['shared']['step_us']:.1f} us, distinct "
            f"{rec['distinct']['step_us']:.1f} us per step")
        out.append(rec)
    return out


def profile_band_reuse(dev):
    """For a rocprofv3 counter run: decode calls (T=1) in a fixed order, so
    that the counters of each stream launch can be matched to a label (the
    labels are printed in launch order).  Each case flushes the Infinity
    Cache (a 1 GiB read), then runs a call on one layer and the same call on
    another layer:
      31B o (W0 88 MB, fits the 256 MB Infinity Cache) and gate|up (W0
      462 MB, does not): layer 0 then layer 1 (same band, same W0), and
      layer 0 then layer 12 (another band);
      gemma3-1b shapes, model order over layers 0..3 (every call of layer 0,
      then of layer 1, ...): G=13 (layers 2b, 2b+1 share W0) and G=26.
    Ends with a plain 1 GiB device copy whose counters calibrate FETCH_SIZE."""
    import torch
    import synth
    import synth.device as sdev
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    labels = []

    def flush():
        flush_buf.sum()

    def call(b, wl, layer, name, tag):
        x = wl.x(layer, name, 1, dev)
        if name in ("qkv", "gate_up"):
            b.stacked(layer, name, x)
        else:
            b.linear(layer, name, x)
        labels.append(tag)

    wl4 = synth.workload(4)
    b4 = sdev.load(wl4, dev)
    torch.cuda.synchronize()
    for name in ("o", "gate_up"):
        for rep in range(2):
            flush()
            call(b4, wl4, 0, name, f"31b {name} L0 cold")
            call(b4, wl4, 1, name, f"31b {name} L1 same band")
            flush()
            call(b4, wl4, 0, name, f"31b {name} L0 cold")
            call(b4, wl4, 12, name, f"31b {name} L12 other band")
    del b4
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    for G in (13, 26):
        wl = synth.custom(26, G, 32, dict(synth.workload(2).dims), cid=70 + G)
        b = sdev.load(wl, dev)
        torch.cuda.synchronize()
        flush()
        for layer in range(4):
            for name, _ in CALLS:
                call(b, wl, layer, name, f"gemma3 G{G} {name} L{layer}")
        del b
        torch.cuda.synchronize()
    src = torch.ones(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile": "band-reuse", "stream_launch_labels": labels, "copy_bytes": src.numel() * 2}),
          flush=True)


def decompose_flops(m, n, k, rank, over, q):
    """Algorithmic fp32 flops of the GPU decomposition of one band: per layer
    the products with the residual (R Omega, q rounds of R^T Y and R Z,
    B = Q^T R: 2 N K l each), the Cholesky-QR passes (Gram and Y T, 2 n l^2
    each; one pass between products, three on the final basis), B B^T and
    the two factor products."""
    l = min(rank + over, n, k)
    if rank == 0:
        return 0
    per = 2 * n * k * l * (1 + 2 * q + 1)
    passes_y = (1 + (q - 1) + 3) if q > 0 else 3          # row-space bases (n = N)
    passes_z = q                                           # column-space bases (n = K)
    per += passes_y * 4 * n * l * l + passes_z * 4 * k * l * l
    per += 2 * l * l * k + 2 * n * l * rank + 2 * k * l * rank
    return m * per


def decompose_section(dev, rank=32, over=16, q=4, cpu_budget=0.0, streams=16):
    """GPU decomposition of the Gemma-3-1B-shaped model: 26 layers in 13
    bands (two layers per band), 7 families, rank 32: 91 band decompositions
    (182 matrices) from seeded i.i.d. N(0, 1/in) bf16 layer weights already
    resident in HBM.  Timed twice: one band call at a time on one stream, and
    the bands spread over `streams` host threads, each with its own stream
    and workspace (the calls are independent; a call's host factorizations
    then overlap the other calls' device work).  The model figure is the
    concurrent one; the one-stream figure is reported beside it.  Then the
    same model with one ALS sweep per band (weightless_decompose_als), and
    the mean relative error of band 0's seven families with and without it."""
    import torch
    import synth
    from weight_shared_rank_amd import binding
    wl = synth.workload(2)
    shapes = [wl.shape(0, f) for f in synth.FAMILIES]
    inputs = []
    for b in range(13):
        for fi, (n, k) in enumerate(shapes):
            w = synth.band_layers(1000 + 16 * b + fi, 2, n, k, device=dev)
            om = synth.sketch_matrix(7 + fi, k, binding.sketch_columns(n, k, rank, over), dev)
            inputs.append((w, om))
    flops = sum(decompose_flops(2, w.shape[1], w.shape[2], rank, over, q) for w, _ in inputs)
    torch.cuda.synchronize()
    from concurrent.futures import ThreadPoolExecutor
    pool = ThreadPoolExecutor(streams)
    sts = [torch.cuda.Stream(device=dev) for _ in range(streams)]

    def run(batch, nst, sweeps=None):
        if nst == 1:
            for w, om in batch:
                binding.decompose(w, rank, om, oversample=over, power_iters=q, als_sweeps=sweeps)
            torch.cuda.synchronize()
            return

        def work(i):
            with torch.cuda.stream(sts[i]):
                for w, om in batch[i::nst]:
                    binding.decompose(w, rank, om, oversample=over, power_iters=q, stream=sts[i], als_sweeps=sweeps)
            sts[i].synchronize()
        list(pool.map(work, range(nst)))
        torch.cuda.synchronize()

    run(inputs[:7], 1)          # warm-up: one band of every family
    run(inputs[7:7 + 2 * streams], streams)
    t0 = time.perf_counter()
    run(inputs, 1)
    el1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    run(inputs, streams)
    el = time.perf_counter() - t0
    run(inputs[:2 * streams], streams, 1)   # warm-up of the ALS path
    t0 = time.perf_counter()
    run(inputs, streams, 1)
    el_als = time.perf_counter() - t0
    pool.shutdown()
    from oracle import decompose as odec

    def band_error(sweeps):
        errs = []
        for w, om in inputs[:7]:
            W0, sv, U, V = (t.float().cpu().double().numpy() for t in
                            binding.decompose(w, rank, om, oversample=over, power_iters=q, als_sweeps=sweeps))
            wl64 = w.float().cpu().double().numpy()
            errs += [odec.rel_frobenius_error(wl64[i], W0, sv[i], U[i], V[i]) for i in range(2)]
        return float(sum(errs) / len(errs))
    out = {"workload": "gemma3-1b decomposition: 13 bands x 7 families (q, k, v, o, gate, up, down), two layers "
                       "per band, rank 32, oversample 16, 4 power rounds",
           "matrices": 2 * len(inputs), "streams": streams, "seconds": el, "matrices_per_s": 2 * len(inputs) / el,
           "fp32_flops": flops, "fp32_TFLOPs": flops / el / 1e12,
           "one_stream_seconds": el1, "one_stream_matrices_per_s": 2 * len(inputs) / el1,
           "als_1_sweep": {"seconds": el_als, "matrices_per_s": 2 * len(inputs) / el_als,
                           "band0_mean_error_one_shot": band_error(None), "band0_mean_error_als_1": band_error(1)}}
    if cpu_budget > 0:
        import numpy as np
        from oracle import decompose
        # the oracle's exact decomposition (numpy SVD) of bands of the gate family until the budget is spent
        w = inputs[4][0].float().cpu().double().numpy()
        n = 0
        t1 = time.perf_counter()
        while True:
            decompose.decompose_band([w[0], w[1]], rank, store=True)
            n += 2
            if time.perf_counter() - t1 >= cpu_budget:
                break
        cel = time.perf_counter() - t1
        out["cpu_oracle"] = {"matrices_per_s": n / cel, "sample": f"{n} gate matrices (4096 x 1152) decomposed by "
                             f"the fp64 oracle (full SVD) in {cel:.1f} s"}
    return out


def band_reuse(dev, reps=5):
    """Band reuse of W0 (decode, T=1).  For two consecutive layers l, l+1 of
    one band, the second call reads the same W0 bytes as the first.  Three
    timings per call type, each the median over reps, GPU time from HIP
    events with the GPU parked so host gaps do not count:
      cold:   Infinity Cache flushed (1 GiB written), then the call on layer l
      reuse:  the call on layer l+1 issued right after the call on layer l
      model:  the call on layer l+1 when every call of layer l ran in
              between (model order)
      repeat: the call on layer l issued right after the same call (everything
              it reads was just read)
    A re-read served by the 256 MB Infinity Cache shows as an effective rate
    above the cold (HBM) rate.  Bytes are the call's algorithmic read bytes."""
    import statistics
    import torch
    import synth
    import synth.device as sdev
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)   # 1 GiB, read to evict

    class _Flush:
        def zero_(self):
            flush_buf.sum()    # reads 1 GiB (4x the Infinity Cache), writes nothing large
    flush = _Flush()
    out = {"method": "median GPU time over %d reps; before each cold measurement 1 GiB is read (a read-only "
                     "pass, so no dirty lines are left to write back)" % reps, "cases": []}

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        return e0, e1

    for wl, layer in ((synth.workload(1), 0), (synth.custom(26, 13, 32, dict(synth.workload(2).dims), cid=2), 0),
                      (synth.workload(4), 0)):
        bundle = sdev.load(wl, dev)
        calls = [c for c in CALLS if all((0, f) in wl.dims for f in c[1])] or [("up", ("up",))]
        if wl.cid == 1:
            calls = [("up", ("up",))]
        xs = {(l, c): wl.x(l, c, 1, dev) for l in (layer, layer + 1) for c, _ in calls}
        ws = bundle.workspace(1)

        def run(l, c):
            x = xs[(l, c)]
            return (lambda: bundle.stacked(l, c, x, ws=ws)) if c in ("qkv", "gate_up") else \
                (lambda: bundle.linear(l, c, x, ws=ws))
        for c, fams in calls:
            nbytes = call_bytes(wl, layer + 1, list(fams), 1)[0]
            w0 = sum(2 * wl.shape(0, f)[0] * wl.shape(0, f)[1] for f in fams)
            cold, reuse, model, repeat = [], [], [], []
            for _ in range(reps):
                torch.cuda.synchronize()
                flush.zero_()
                torch.cuda._sleep(20_000_000)
                ev_cold = timed(run(layer, c))
                ev_reuse = timed(run(layer + 1, c))
                torch.cuda.synchronize()
                cold.append(ev_cold[0].elapsed_time(ev_cold[1]) * 1e-3)
                reuse.append(ev_reuse[0].elapsed_time(ev_reuse[1]) * 1e-3)
                flush.zero_()
                torch.cuda._sleep(20_000_000)
                for c2, _ in calls:
                    run(layer, c2)()
                for c2, _ in calls:
                    if c2 == c:
                        break
                    run(layer + 1, c2)()
                ev_model = timed(run(layer + 1, c))
                torch.cuda.synchronize()
                model.append(ev_model[0].elapsed_time(ev_model[1]) * 1e-3)
                torch.cuda._sleep(20_000_000)
                run(layer, c)()
                ev_rep = timed(run(layer, c))
                torch.cuda.synchronize()
                repeat.append(ev_rep[0].elapsed_time(ev_rep[1]) * 1e-3)
            tc, tr, tm, tp = (statistics.median(v) for v in (cold, reuse, model, repeat))
            between = sum(2 * wl.shape(0, f)[0] * wl.shape(0, f)[1] for c2, fs in calls if c2 != c for f in fs)
            out["cases"].append({
                "workload": wl.name, "call": c, "layers": [layer, layer + 1], "same_band": band_of_layer(layer, wl.num_layers, wl.num_bands) == band_of_layer(layer + 1, wl.num_layers, wl.num_bands),
                "w0_MB": w0 / 1e6, "bytes_read_MB": nbytes / 1e6, "other_w0_between_in_model_order_MB": between / 1e6,
                "cold_us": tc * 1e6, "reuse_us": tr * 1e6, "model_order_us": tm * 1e6, "same_layer_repeat_us": tp * 1e6,
                "cold_GBps": nbytes / tc / 1e9, "reuse_GBps": nbytes / tr / 1e9, "model_order_GBps": nbytes / tm / 1e9,
                "same_layer_repeat_GBps": nbytes / tp / 1e9,
                "reuse_served_by_infinity_cache": tr < 0.8 * tc,
                "model_order_served_by_infinity_cache": tm < 0.8 * tc})
            log(f"band reuse {wl.name} {c}: cold {tc*1e6:.1f} us, reuse {tr*1e6:.1f} us, model order {tm*1e6:.1f} us, "
                f"repeat {tp*1e6:.1f} us")
        del bundle
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--only", default="all", choices=["all", "decode", "decode1", "decode2", "prefill", "dense", "act",
                                                             "fp8", "decompose", "small", "reuse"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--band-reuse", action="store_true",
                    help="report whether a band-shared W0 re-read by the next layer is served from the 256 MB "
                         "Infinity Cache or from HBM (prints one JSON line)")
    ap.add_argument("--profile", choices=["decode", "prefill", "band-reuse"],
                    help="for rocprofv3 counter runs: one eager step (decode: the headline workload at T=1; "
                         "prefill: the Gemma-4-31B mixed prefill at T=512), then a plain 1 GiB device copy whose "
                         "counters calibrate FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the weightless linear here runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    from weight_shared_rank_amd import binding
    binding.lib()

    wl4 = synth.workload(4)
    if args.profile == "band-reuse":
        profile_band_reuse(dev)
        return
    if args.profile:
        import synth.device as sdev
        wlp, T = (wl4, 1) if args.profile == "decode" else (synth.workload(5), 512)
        bundle = sdev.load(wlp, dev)
        step = Step(wlp, bundle, T, CALLS, dev)
        torch.cuda.synchronize()
        step.run()
        torch.cuda.synchronize()
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "bytes_per_call": step.bytes_rd / len(step.items),
                          "flops_per_call": step.flops / len(step.items),
                          "calls": len(step.items), "copy_bytes": src.numel() * 2}), flush=True)
        return

    res = {}
    if args.band_reuse:
        print(json.dumps(band_reuse(dev)), flush=True)
        return
    if args.only in ("all", "decode", "decode1"):
        res["decode4_t1"] = decode_section(wl4, 1, args.steps, args.warmup, dev)
        log(f"decode T=1: {res['decode4_t1']['GBps']:.1f} GB/s")
    if args.only in ("all", "decode", "fp8"):
        res["decode4_fp8_t1"] = decode_section(wl4, 1, args.steps, args.warmup, dev, w0_format="fp8")
        log(f"decode T=1, FP8 W0: {res['decode4_fp8_t1']['GBps']:.1f} GB/s, "
            f"{res['decode4_fp8_t1']['step_s'] * 1e3:.3f} ms per step")
    if args.only in ("all", "decode", "fp8"):
        res["decode4_mxfp4_t1"] = decode_section(wl4, 1, args.steps, args.warmup, dev, w0_format="mxfp4")
        log(f"decode T=1, MXFP4 W0: {res['decode4_mxfp4_t1']['GBps']:.1f} GB/s, "
            f"{res['decode4_mxfp4_t1']['step_s'] * 1e3:.3f} ms per step")
    if args.only in ("all", "decode", "dense"):
        res["dense_vs_weightless"] = dense_comparison(wl4, 1, 12, args.steps, args.warmup, dev)
        log(f"dense comparison: weightless {res['dense_vs_weightless']['weightless_ms']:.3f} ms, dense "
            f"{res['dense_vs_weightless']['dense_ms']:.3f} ms, hipBLASLt dense "
            f"{res['dense_vs_weightless']['hipblaslt_dense_ms']:.3f} ms per 12-layer step")
    if args.only in ("all", "decode", "act"):
        res["gate_up_act_decode"] = gate_up_act_section(wl4, 1, args.steps, args.warmup, dev)
        log(f"gate|up act, decode T=1: fused {res['gate_up_act_decode']['fused_us_per_call']:.1f} us, unfused "
            f"{res['gate_up_act_decode']['unfused_us_per_call']:.1f} us per call")
    if args.only in ("all", "decode"):
        res["decode4_t16"] = decode_section(wl4, 16, args.steps, args.warmup, dev)
        log(f"decode T=16: {res['decode4_t16']['GBps']:.1f} GB/s")
    if args.only in ("all", "decode", "decode2"):
        res["decode2_t1"] = decode_section(synth.custom(26, 13, 32, dict(synth.workload(2).dims), cid=2),
                                           1, args.steps * 5, args.warmup, dev)
        log(f"gemma3 decode T=1: {res['decode2_t1']['GBps']:.1f} GB/s")
    if args.only in ("all", "prefill"):
        res["prefill5"] = prefill_section(synth.workload(5), 512, CALLS, max(2, args.steps // 4), 2, dev)
        log(f"prefill w5: {res['prefill5']['TFLOPs']:.1f} TFLOP/s")
        res["gate_up_act_prefill"] = gate_up_act_section(synth.workload(5), 512, max(2, args.steps // 4), 2, dev)
        log(f"gate|up act, prefill T=512: fused {res['gate_up_act_prefill']['fused_us_per_call']:.1f} us, unfused "
            f"{res['gate_up_act_prefill']['unfused_us_per_call']:.1f} us per call")
        singles = tuple((f, (f,)) for f in synth.FAMILIES)
        res["prefill3"] = prefill_section(synth.workload(3), 2048, singles, args.steps, args.warmup, dev)
        log(f"prefill w3: {res['prefill3']['TFLOPs']:.1f} TFLOP/s")
        # secondary: the same layers with q|k|v and gate|up as stacked calls (4 calls per layer instead of 7)
        res["prefill3_stacked"] = prefill_section(synth.workload(3), 2048, CALLS, args.steps, args.warmup, dev)
        log(f"prefill w3, stacked calls: {res['prefill3_stacked']['TFLOPs']:.1f} TFLOP/s")

    if args.only in ("all", "small"):
        res["workload1"] = workload1_section(dev, args.steps, args.warmup)
        log(f"one-family workload: cold {res['workload1']['cold_us_per_call']:.2f} us, warm "
            f"{res['workload1']['warm_us_per_call']:.2f} us per call")
    if args.only in ("all", "reuse"):
        res["band_reuse_ab"] = band_reuse_ab(dev, args.steps, args.warmup)
    if args.only in ("all", "decompose"):
        res["decompose_gemma3"] = decompose_section(dev, cpu_budget=0.0 if args.no_cpu else 4.0)
        log(f"decomposition: {res['decompose_gemma3']['matrices_per_s']:.1f} matrices/s, "
            f"{res['decompose_gemma3']['seconds']:.2f} s for the gemma3 model on "
            f"{res['decompose_gemma3']['streams']} streams (one stream: "
            f"{res['decompose_gemma3']['one_stream_seconds']:.2f} s)")
        als = res["decompose_gemma3"]["als_1_sweep"]
        log(f"decomposition with one ALS sweep: {als['seconds']:.2f} s; band 0 mean error "
            f"{als['band0_mean_error_one_shot']:.4f} -> {als['band0_mean_error_als_1']:.4f}")

    line = {"metric": "weightless-linear decode GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak)",
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded normal bundles and activations of the stated shapes)"}
    if "decode4_t1" in res:
        d = res["decode4_t1"]
        line.update({"value": round(d["GBps"], 2), "ms_per_step": round(d["step_s"] * 1e3, 4),
                     "config": {"workload": "gemma4-31b-sliding decode: 60 layers x (qkv stacked, o, gate_up "
                                            "stacked, down), G=5, rank 256, T=1, graph-replayed step",
                                "tokens": 1, "layers": 60, "bands": 5, "rank": 256,
                                "bytes_read_per_step": d["bytes_read"], "hbm_frac": d["GBps"] / HBM_PEAK_GBS}})
        sha = source_sha("decode.hip", "common.h", "internal.h")
        traffic, t_rd, t_wr = traffic_from_profile("decode", sha)
        line["roofline"] = {"bound": "hbm",
                            "kernel": "stream_kernel + epilogue_kernel (one decode call is these two launches; "
                                      "the stream launch moves ~95% of the bytes)",
                            "timing": "HIP events on the replay stream around the timed graph replays, "
                                      "per call (each call's two launches back to back)",
                            "achieved": round(d["graph_event_GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(d["graph_event_GBps"] / HBM_PEAK_GBS, 4),
                            "bytes_per_call": d["bytes_per_launch"], "avg_call_us": round(d["graph_event_call_us"], 3),
                            "eager_call_us": round(d["avg_launch_us"], 3),
                            "traffic": traffic, "traffic_read": t_rd, "traffic_written": t_wr,
                            "source_sha": sha}
    line["detail"] = res
    if "prefill5" in res:
        p = res["prefill5"]
        psha = source_sha("prefill.hip", "common.h", "internal.h")
        ptraffic, pt_rd, pt_wr = traffic_from_profile("prefill", psha)
        line["prefill"] = {"metric": "prefill TFLOP/s", "value": round(p["TFLOPs"], 2), "unit": "TFLOP/s",
                           "mfma_frac": round(p["mfma_frac"], 4), "peak": BF16_PEAK_TFLOPS,
                           "ms_per_step": round(p["step_s"] * 1e3, 3),
                           "workload": "gemma4-31b mixed prefill: 10 full + 50 sliding layers, G=1 per type, "
                                       "rank 1024, T=512, graph-replayed step",
                           "roofline": {"bound": "mfma",
                                        "kernel": "gemm_kernel (Z = X V, then the main GEMM with the s and U z "
                                                  "epilogue; GEMMs with few rows split K, adding reduce_z_kernel / "
                                                  "finish_kernel: 2-4 launches per call)",
                                        "timing": "HIP events on the replay stream around the timed graph "
                                                  "replays, per call",
                                        "achieved": round(p["graph_event_TFLOPs"], 2), "peak": BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(p["graph_event_TFLOPs"] / BF16_PEAK_TFLOPS, 4),
                                        "flops_per_call": p["flops_per_call"],
                                        "avg_call_us": round(p["graph_event_call_us"], 2),
                                        "eager_call_us": round(p["avg_call_us"], 2),
                                        "traffic": ptraffic, "traffic_read": pt_rd, "traffic_written": pt_wr,
                                        "source_sha": psha}}
        if "prefill3" in res:
            line["prefill"]["gemma3_1b_T2048_TFLOPs"] = round(res["prefill3"]["TFLOPs"], 2)
        if "prefill3_stacked" in res:
            line["prefill"]["gemma3_1b_T2048_stacked_TFLOPs"] = round(res["prefill3_stacked"]["TFLOPs"], 2)
    if not args.no_cpu and args.only in ("all", "decode"):
        log("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(wl4, 1, args.cpu_budget, dev)
    if not args.no_cpu and args.only in ("all", "prefill") and "prefill" in line:
        log("cpu baseline, prefill")
        line["prefill"]["cpu_baseline"] = oracle_prefill_baselines(dev)
    if not args.no_cpu and args.only in ("all", "small"):
        log("cpu baseline, small workloads")
        res["oracle_small_decode"] = oracle_small_decode_baselines(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
