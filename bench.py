#!/usr/bin/env python3
"""Benchmark of the deformable sampling core on one MI355X.

Headline: DCN core forward effective GB/s (input + offset + mask + output
bytes per launch / launch time), as a fraction of the 8 TB/s HBM3E peak, and
Gsamples/s, on the FlashInternImage-T stage-1 shape in bf16 (DCNv4 with
fp32 accumulation, N=64, 56x56, C=64, G=4, K=3, offsets N(0, 2^2) px).  One
step = one forward launch over the whole batch.  Beside it, in the same JSON
line: the byte-weighted aggregate of the bf16 sweep over the four
FlashInternImage-T stage shapes (and each stage), the same shape in fp16,
the core op of a whole FlashInternImage-T forward (the stage shapes at their
depths, 30 launches), the DCNv3 large-channel stage at stride 1 and 2, the
DCNv4 stage-1 shapes with DCNv4's packed offset+mask tensor, the fp32
forward + backward and the half-precision backward, the whole DCNv4 layer
around the core (projections, core, centre-feature gate) at the fp16 shape,
and the CPU oracle timed on the host cores (which also checks the headline
batch element by element).

Inputs are seeded synthetic tensors (no dataset, no weights).  Timing uses
R rotating copies of every tensor (R * bytes > 512 MB, twice the 256 MB
Infinity Cache) so each launch reads its inputs from HBM, and the K timed
launches are captured in one HIP graph replayed between two events on the
stream the kernels run on, so host launch overhead does not pad the small
kernels.  Eager-launch timing is reported too, with the p10 / median / p90
of the launches timed one by one.  Per-workload rocprofv3 counters (HBM
bytes, L2 hit, VALU busy and instruction counts, occupancy, LDS use) come
from the committed profiles/traffic_counters.json when it was taken on the
current kernel sources.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import deformable_convolution_core_amd as dcn  # noqa: E402
from deformable_convolution_core_amd import inputs  # noqa: E402

METRIC = "DCN core fwd effective GB/s (% HBM roofline) + Gsamples/s, FlashInternImage-T"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 600e6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "deformable_convolution_core_amd", "csrc", f)
                  for f in ("dcn_kernels.hpp", "dcn_core.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what
    the compiler sees, so a comment edit keeps the hash (string literals in
    these sources hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_hash(sources=None) -> str:
    """First 16 hex digits of the sha256 of the kernel sources' code text."""
    h = hashlib.sha256()
    for text in (sources if sources is not None else [open(p).read() for p in KERNEL_SOURCES]):
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def rotating_sets(w, backward=False, packed=False):
    """R device copies of the workload's tensors (+ outputs).  packed: the
    offsets and mask travel as DCNv4's single record tensor instead."""
    per = w.min_bytes_backward() if backward else w.min_bytes_forward()
    R = max(2, math.ceil(ROTATE_BYTES / per))
    host = inputs.make(w, with_grad=backward)
    if packed:
        host["offset"] = inputs.pack_offset_mask(host["offset"], host.pop("mask"), w.G, w.P)
    sets = []
    for _ in range(R):
        d = {k: v.to("cuda") for k, v in host.items()}
        if backward:
            d["gi"] = torch.empty_like(d["input"])
            d["goff"] = torch.empty_like(d["offset"])
            d["gm"] = torch.empty_like(d["mask"]) if "mask" in d else None
            if w.dtype != "f32":   # half precision sums grad_input in a binary32 workspace
                d["ws"] = torch.empty(d["input"].numel(), dtype=torch.float32, device="cuda")
        else:
            d["out"] = torch.empty(w.shapes()["output"], dtype=d["input"].dtype, device="cuda")
        sets.append(d)
    return sets


def launcher(w, backward=False, packed=False):
    """A function launching one forward (or backward) of w on a tensor set
    through the C ABI (the _ex entry points, flags from the workload)."""
    lib = dcn.load_library()
    dt = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    flags = ((dcn.FLAG_SOFTMAX if w.softmax else 0) | (dcn.FLAG_REMOVE_CENTER if w.remove_center else 0)
             | (dcn.FLAG_PACKED if packed else 0))
    import ctypes
    vp = ctypes.c_void_p

    def ptr(t):
        return None if t is None else vp(t.data_ptr())

    def fwd(d, stream):
        rc = lib.dcn_core_forward_ex(ptr(d["input"]), ptr(d["offset"]), ptr(d.get("mask")), ptr(d["out"]),
                                     w.N, w.H, w.W, w.G, w.Cg, w.K, w.stride, w.pad, w.dilation,
                                     float(w.offset_scale), flags, dt, vp(stream))
        if rc:
            raise dcn.DCNError(rc, lib.dcn_status_string(rc).decode())

    def bwd(d, stream):
        ws = d.get("ws")
        rc = lib.dcn_core_backward_ws(ptr(d["input"]), ptr(d["offset"]), ptr(d.get("mask")),
                                      ptr(d["grad_out"]), ptr(d["gi"]), ptr(d["goff"]), ptr(d["gm"]),
                                      w.N, w.H, w.W, w.G, w.Cg, w.K, w.stride, w.pad, w.dilation,
                                      float(w.offset_scale), flags, dt, ptr(ws),
                                      0 if ws is None else ws.numel() * 4, vp(stream))
        if rc:
            raise dcn.DCNError(rc, lib.dcn_status_string(rc).decode())

    return bwd if backward else fwd


LAST_SPREAD = {}


def time_launches(w, steps, warmup, backward=False, packed=False):
    """Mean per-launch time (ms) of `steps` launches over rotating buffers:
    graph-replayed (primary) and eager.  The eager launches are also timed
    one by one (an event after each, on the kernels' stream; the host runs
    ahead, so consecutive events bracket one kernel each): their p10, median
    and p90 land in LAST_SPREAD."""
    sets = rotating_sets(w, backward, packed)
    R = len(sets)
    launch = launcher(w, backward, packed)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        h = stream.cuda_stream
        for i in range(warmup):
            launch(sets[i % R], h)
        torch.cuda.synchronize()
        # eager
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            launch(sets[i % R], h)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        eager_ms = ev[0].elapsed_time(ev[-1]) / steps
        each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        q = lambda f: each[min(len(each) - 1, int(f * len(each)))]
        LAST_SPREAD.clear()
        LAST_SPREAD.update(p10_us=round(q(0.1) * 1e3, 3), median_us=round(q(0.5) * 1e3, 3),
                           p90_us=round(q(0.9) * 1e3, 3))
    # graph of exactly `steps` launches
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(steps):
            launch(sets[i % R], h)
    torch.cuda.synchronize()
    g.replay()                      # warm replay
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
    del g, sets
    torch.cuda.empty_cache()
    return graph_ms, eager_ms, R


def forward_record(w, steps, warmup, packed=False):
    ms, eager_ms, R = time_launches(w, steps, warmup, packed=packed)
    gbps = w.min_bytes_forward() / (ms * 1e-3) / 1e9
    rec = dict(workload=w.name, dtype=w.dtype, softmax=bool(w.softmax),
               layout="packed offset+mask" if packed else "separate offset and mask",
               shape=dict(N=w.N, H=w.H, W=w.W, C=w.C, G=w.G, Cg=w.Cg, K=w.K, stride=w.stride,
                          Ho=w.Ho, Wo=w.Wo),
               us=round(ms * 1e3, 3), eager_us=round(eager_ms * 1e3, 3), eager_each=dict(LAST_SPREAD),
               min_bytes=w.min_bytes_forward(), GBps=round(gbps, 1),
               frac_hbm=round(gbps / HBM_PEAK_GBPS, 4),
               Gsamples_s=round(w.samples() / (ms * 1e-3) / 1e9, 3), rotating_sets=R)
    if not packed:
        rec["counters"] = counter_record(w.name)
        rec["valu"] = valu_record(w.name, ms)
    return rec


FII_T_DEPTHS = (4, 4, 18, 4)   # DCN layers per FlashInternImage-T stage (the T config's depths)


def fii_t_sweep(steps, warmup):
    """The core op of one FlashInternImage-T forward over a batch of 64: the
    four bf16 stage shapes at their depths (30 launches, each layer on its
    own tensors), captured in one graph and replayed.  Reports the core-op
    time per batch and per image."""
    layers = []
    for depth, name in zip(FII_T_DEPTHS, inputs.BF16_SWEEP):
        w = inputs.WORKLOADS[name]
        host = inputs.make(w, with_grad=False)
        for _ in range(depth):
            d = {k: v.to("cuda") for k, v in host.items()}
            d["out"] = torch.empty(w.shapes()["output"], dtype=d["input"].dtype, device="cuda")
            layers.append((w, launcher(w), d))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        h = stream.cuda_stream
        for _ in range(warmup):
            for w, launch, d in layers:
                launch(d, h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        h = torch.cuda.current_stream().cuda_stream
        for w, launch, d in layers:
            launch(d, h)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = sum(w.min_bytes_forward() for w, _, _ in layers)
    n_img = layers[0][0].N
    del g, layers
    torch.cuda.empty_cache()
    return dict(depths=list(FII_T_DEPTHS), launches=sum(FII_T_DEPTHS), batch=n_img,
                us_per_batch=round(ms * 1e3, 2), us_per_image=round(ms * 1e3 / n_img, 3),
                images_per_s_core_op=round(n_img / (ms * 1e-3), 1), min_bytes=nbytes,
                GBps=round(nbytes / (ms * 1e-3) / 1e9, 1))


def graph_time(fn, steps, warmup):
    """Mean ms of fn() over `steps` calls captured in one graph (on a side
    stream) and replayed between two events."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / steps


def eager_time(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def layer_record(w, steps, warmup):
    """The DCNv4 layer around the core at workload w's shape, with the
    centre-feature gate: value and offset+mask projections (matrix-core
    GEMM), HIP core on the packed records, HIP gate, output projection.
    Random weights (no checkpoint).  Forward in a graph; forward + backward
    eager (autograd), and the same forward + backward captured in a graph.
    Also the gate kernel and the value projection alone,
    against HBM (the projection also on the platform BLAS)."""
    from deformable_convolution_core_amd.layer import DCNv4
    dt = inputs.DTYPES[w.dtype]
    torch.manual_seed(0)
    layer = DCNv4(w.C, kernel_size=w.K, group=w.G, offset_scale=w.offset_scale, center_feature_scale=True,
                  device="cuda", dtype=torch.float32)
    with torch.no_grad():
        layer.offset_mask.weight.mul_(1.5)
    layer = layer.to(dt)
    x = inputs.normal((w.N, w.H, w.W, w.C), w.seed_base + 21, 1.0, w.dtype).to("cuda")
    gout = inputs.normal((w.N, w.H, w.W, w.C), w.seed_base + 22, 1.0, w.dtype).to("cuda")
    with torch.no_grad():
        fwd_ms = graph_time(lambda: layer(x), steps, warmup)
    xi = x.clone().requires_grad_(True)

    def fwd_bwd():
        layer.zero_grad(set_to_none=True)
        xi.grad = None
        layer(xi).backward(gout)
    fb_ms = eager_time(fwd_bwd, max(5, steps // 4), 3)
    # the same step captured in a graph: its GPU time without the host's
    # per-call autograd and launch work (the eager figure is bound by that)
    fb_graph_ms, fb_graph_note = None, None
    try:
        fb_graph_ms = graph_time(fwd_bwd, max(5, steps // 4), 3)
    except RuntimeError as e:
        fb_graph_note = f"capture refused: {e}"[:200]
    # the gate alone: read y, v, z; write out
    M = w.N * w.H * w.W
    y = torch.randn(M, w.C, device="cuda", dtype=dt)
    v = torch.randn(M, w.C, device="cuda", dtype=dt)
    z = torch.randn(M, w.G, device="cuda", dtype=dt)
    out = torch.empty_like(y)
    gate_ms = graph_time(lambda: dcn.center_gate_forward(y, v, z, group=w.G, out=out), steps, warmup)
    gate_bytes = (3 * M * w.C + M * w.G) * w.elem_bytes
    # the value projection alone: this package's matrix-core GEMM against the platform BLAS
    wv, bv = layer.value_proj.weight, layer.value_proj.bias
    xm = x.reshape(M, w.C)
    ym = torch.empty(M, w.C, device="cuda", dtype=dt)
    lin_ms = graph_time(lambda: dcn.linear(xm, wv, bv, out=ym), steps, warmup)
    blas_ms = graph_time(lambda: torch.nn.functional.linear(xm, wv, bv), steps, warmup)
    lin_bytes = (2 * M * w.C + w.C * w.C + w.C) * w.elem_bytes
    # the offset+mask projection's weight and bias gradients alone: this
    # package's matrix-core reduction against the batched BLAS path
    from deformable_convolution_core_amd.layer import weight_grad
    O = layer.offset_mask.weight.shape[0]
    gom = torch.randn(M, O, device="cuda", dtype=dt)
    wg_ms = eager_time(lambda: dcn.linear_weight_grad(gom, xm), steps, warmup)
    wg_blas_ms = eager_time(lambda: (weight_grad(gom, xm), gom.sum(0, dtype=torch.float32)), steps, warmup)
    wg_bytes = M * (O + w.C) * w.elem_bytes
    del layer, x, xi, gout, y, v, z, out, xm, ym, gom
    torch.cuda.empty_cache()
    return dict(workload=f"DCNv4 layer (value, offset+mask, gate, output projections + core) at {w.name}",
                dtype=w.dtype, center_feature_scale=True, forward_us=round(fwd_ms * 1e3, 2),
                forward_backward_us_eager=round(fb_ms * 1e3, 2),
                forward_backward_us_graph=None if fb_graph_ms is None else round(fb_graph_ms * 1e3, 2),
                **({} if fb_graph_note is None else {"forward_backward_graph_note": fb_graph_note}),
                images_per_s_forward=round(w.N / (fwd_ms * 1e-3), 1),
                gate_kernel=dict(us=round(gate_ms * 1e3, 3), min_bytes=gate_bytes,
                                 GBps=round(gate_bytes / (gate_ms * 1e-3) / 1e9, 1),
                                 frac_hbm=round(gate_bytes / (gate_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)),
                value_projection=dict(shape=f"{M}x{w.C} @ {w.C}x{w.C}", us=round(lin_ms * 1e3, 3),
                                      GBps=round(lin_bytes / (lin_ms * 1e-3) / 1e9, 1),
                                      frac_hbm=round(lin_bytes / (lin_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                      platform_blas_us=round(blas_ms * 1e3, 3)),
                offset_mask_weight_grad=dict(shape=f"({M}x{O})^T @ {M}x{w.C}", us=round(wg_ms * 1e3, 3),
                                             GBps=round(wg_bytes / (wg_ms * 1e-3) / 1e9, 1),
                                             frac_hbm=round(wg_bytes / (wg_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                             batched_blas_us=round(wg_blas_ms * 1e3, 3)))


def cpu_baseline(w):
    """The oracle as it stands, on the host cores, over whole batches of the
    headline workload, repeated until at least ~10 s of wall time."""
    import oracle   # test infrastructure, used here only for this timing leg
    t = inputs.make(w, with_grad=False)
    x, o, m = (inputs.to_f64(t[k]) for k in ("input", "offset", "mask"))
    kw = dict(K=w.K, stride=w.stride, pad=w.pad, dilation=w.dilation, offset_scale=w.offset_scale,
              softmax=w.softmax, group=w.G, with_absum=False)
    oracle.forward(x, o, m, **kw)           # warm (page-in, thread start)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(x, o, m, **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 1000:
            break
    per = el / reps
    cores = oracle.max_threads()
    # the same batch through the HIP path, compared element by element with
    # the oracle (binary32 coordinates, the kernels' contract)
    from tests import tolerance
    ref, S = oracle.forward(x, o, m, **dict(kw, with_absum=True), coord_mode=oracle.COORD_BINARY32)
    lib = dcn.load_library()
    d = {k: v.to("cuda") for k, v in t.items()}
    out = dcn.forward(d["input"], d["offset"], d["mask"], kernel_size=w.K, stride=w.stride, pad=w.pad,
                      dilation=w.dilation, offset_scale=w.offset_scale, softmax=w.softmax, group=w.G)
    torch.cuda.synchronize()
    st = tolerance.compare(out.float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    del lib
    return dict(value=round(w.min_bytes_forward() / per / 1e9, 3), unit="GB/s", cores=cores,
                kind="oracle", cpu_model=cpu_model(),
                sample=f"{reps} full batches of {w.name} (N={w.N}), binary64 C loops with OpenMP, "
                       f"{per * 1e3:.1f} ms per batch",
                parity=dict(ok=st["ok"], max_ratio=round(st["max_ratio"], 4), norm_rel=st["norm_rel"],
                            n_bad=st["n_bad"], n=st["n"],
                            bound="|gpu - ref| <= 2e-2 |ref| + (n_terms + 32) 2^-24 S per element"))


def parity_per_config(names):
    """Part of the CPU leg: each forward workload (and the backward of the
    56x56 DCNv4 shape in every dtype) runs through the HIP path on its whole
    batch, in the launch configuration timed above, and image 0 of the result
    is compared element by element with the oracle on image 0 (binary32
    coordinates, the kernels' contract)."""
    import oracle   # test infrastructure, used here only within the CPU leg
    from tests import tolerance
    res = {}

    def comp(got, ref, S, n, dtype):
        st = tolerance.compare(got, ref, S, n, dtype)
        return dict(ok=st["ok"], max_ratio=round(st["max_ratio"], 4), norm_rel=st["norm_rel"], n_bad=st["n_bad"],
                    n=st["n"])

    for name in names:
        w = inputs.WORKLOADS[name]
        t = inputs.make(w, with_grad=False)
        d = {k: v.to("cuda") for k, v in t.items()}
        out = dcn.forward(d["input"], d["offset"], d["mask"], kernel_size=w.K, stride=w.stride, pad=w.pad,
                          dilation=w.dilation, offset_scale=w.offset_scale, softmax=w.softmax, group=w.G)
        torch.cuda.synchronize()
        f64 = {k: inputs.to_f64(v[:1]) for k, v in t.items()}
        ref, S = oracle.forward(f64["input"], f64["offset"], f64["mask"], K=w.K, stride=w.stride, pad=w.pad,
                                dilation=w.dilation, offset_scale=w.offset_scale, softmax=w.softmax, group=w.G,
                                coord_mode=oracle.COORD_BINARY32)
        res[name] = comp(out[:1].float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    w5 = inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"]
    for dt in ("f32", "f16", "bf16"):
        w = w5 if dt == "f32" else inputs.scaled(w5, dtype=dt)
        t = inputs.make(w, with_grad=True)
        d = {k: v.to("cuda") for k, v in t.items()}
        gi, goff, gm = dcn.backward(d["input"], d["offset"], d["mask"], d["grad_out"], kernel_size=w.K,
                                    stride=w.stride, pad=w.pad, dilation=w.dilation, offset_scale=w.offset_scale,
                                    softmax=w.softmax, group=w.G)
        torch.cuda.synchronize()
        f64 = {k: inputs.to_f64(v[:1]) for k, v in t.items()}
        r = oracle.backward(f64["input"], f64["offset"], f64["mask"], f64["grad_out"], K=w.K, stride=w.stride,
                            pad=w.pad, dilation=w.dilation, offset_scale=w.offset_scale, softmax=w.softmax,
                            group=w.G, coord_mode=oracle.COORD_BINARY32)
        res[f"{w5.name}@{dt} backward"] = {
            key: comp(got[:1].float().cpu().numpy().reshape(r[key].shape), r[key], S, n, dt)
            for key, got, S, n in (("grad_input", gi, r["gi_abs"], r["gi_cnt"]),
                                   ("grad_offset", goff, r["goff_abs"], 4 * w.Cg),
                                   ("grad_mask", gm, r["gmask_abs"], 4 * w.Cg))}
    return res


def _counters(name):
    """The committed rocprofv3 counter record of a workload, if it was taken
    on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        d = json.load(open(TRAFFIC_FILE))
    except ValueError:
        return None
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("workloads", {}).get(name)


def backward_counter_record(name, dtype):
    """Per-kernel counters of the backward at workload `name` in `dtype`
    (owner and gradient kernels) from the committed record, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        d = json.load(open(TRAFFIC_FILE))
    except ValueError:
        return None
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("backward", {}).get(f"{name}@{dtype}")


def traffic_record(name, min_bytes):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters, if they were taken on the current kernel sources."""
    e = _counters(name)
    return None if e is None else e.get("hbm_bytes_per_launch")


COUNTER_KEYS = ("valu_busy_pct", "occupancy_pct", "lds_util_pct", "l2_hit", "hbm_bytes_per_launch",
                "sq_insts_valu", "sq_insts_lds", "sq_waves")


def counter_record(name):
    """VALU busy, occupancy, LDS utilisation, L2 hit rate, HBM bytes and
    instruction counts of the workload's kernel from the committed rocprofv3
    counters (None if stale or missing)."""
    e = _counters(name)
    if e is None:
        return None
    return {k: e.get(k) for k in COUNTER_KEYS if k in e}


# VALU issue ceiling: 1024 SIMDs (256 CUs x 4) at 2.4 GHz, one wave64
# instruction per SIMD every 4 clocks (16 lanes per clock).
VALU_PEAK_G = 1024 * 2.4 / 4.0


def valu_record(name, ms):
    """The workload's VALU wave-instructions per launch (SQ_INSTS_VALU from the
    committed counters) issued at the measured launch time, against the
    16-lane issue ceiling.  On this GPU plain binary32 fma/add/mul and bitwise
    ops with VGPR operands issue up to ~1.45x that ceiling and the
    mixed-precision, convert and shift ops at ~0.85-0.93x (measured), so the
    fraction is an issue-rate figure, not a hard bound."""
    e = _counters(name)
    if e is None or not e.get("sq_insts_valu"):
        return None
    g = e["sq_insts_valu"] / (ms * 1e-3) / 1e9
    return dict(insts=e["sq_insts_valu"], achieved=round(g, 1), peak=VALU_PEAK_G, unit="G wave-instr/s",
                frac=round(g / VALU_PEAK_G, 4))


def copy_bandwidth(mb=1024, steps=20):
    """A device-to-device copy of `mb` MB (read + write bytes over time): the
    bandwidth a plain stream reaches on this GPU, beside the nameplate."""
    n = mb * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms = graph_time(lambda: dst.copy_(src), steps, 3)
    gbps = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes_per_copy=2 * n * 4, us=round(ms * 1e3, 2), GBps=round(gbps, 1),
                frac_hbm=round(gbps / HBM_PEAK_GBPS, 4))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def profile_mode(w, args):
    """Launch one workload eagerly `steps` times over rotating buffers, then
    (optionally) copy a buffer of known size `steps` times: a target for
    rocprofv3 counter passes (per-dispatch counters of a plain copy calibrate
    FETCH_SIZE / WRITE_SIZE)."""
    sets = rotating_sets(w, args.backward)
    launch = launcher(w, args.backward)
    h = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup + args.steps):
        launch(sets[i % len(sets)], h)
    torch.cuda.synchronize()
    log(f"profiled {args.warmup + args.steps} launches of {w.name} "
        f"({'backward' if args.backward else 'forward'}), rotating sets {len(sets)}")
    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
        for b in bufs:
            b.fill_(1.0)
        for i in range(args.steps):
            bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4])
        torch.cuda.synchronize()
        log(f"copied {args.copy_mb} MiB x {args.steps} (read {args.copy_mb} MiB + write {args.copy_mb} MiB each)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=inputs.HEADLINE, choices=list(inputs.WORKLOADS))
    ap.add_argument("--quick", action="store_true", help="headline only (no sweep, no CPU leg)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for counter runs: eager launches of --workload only (plus --copy-mb), no JSON")
    ap.add_argument("--backward", action="store_true", help="with --profile: launch the backward")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="with --profile: also run plain device copies of this many MB (counter calibration)")
    ap.add_argument("--dtype", choices=("f32", "f16", "bf16"), default=None,
                    help="with --profile: run the workload's shape in this dtype")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sampling core needs no communication and this "
              "build runs on a single MI355X; rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dcn.load_library()
    torch.cuda.set_device(0)

    w = inputs.WORKLOADS[args.workload]
    w5 = inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"]
    if args.profile:
        profile_mode(w if args.dtype is None else inputs.scaled(w, dtype=args.dtype), args)
        return
    log(f"headline {w.name}: steps={args.steps} warmup={args.warmup}")
    head = forward_record(w, args.steps, args.warmup)
    log(f"headline {head['us']} us, {head['GBps']} GB/s")
    cp = copy_bandwidth()
    log(f"device-to-device copy {cp['GBps']} GB/s; headline at {head['GBps'] / cp['GBps']:.3f} of it")

    extra = {"copy_bandwidth": cp, "frac_measured_copy": round(head["GBps"] / cp["GBps"], 4)}
    if not args.quick:
        # the bf16 FlashInternImage-T stage sweep; its byte-weighted aggregate
        # stands beside the headline (its first stage)
        sweep = [head if name == w.name else forward_record(inputs.WORKLOADS[name], args.steps, args.warmup)
                 for name in inputs.BF16_SWEEP]
        for r in sweep:
            log(f"{r['workload']}: {r['us']} us, {r['GBps']} GB/s")
        tot_bytes = sum(r["min_bytes"] for r in sweep)
        tot_us = sum(r["us"] for r in sweep)
        extra["bf16_sweep"] = sweep
        extra["bf16_sweep_aggregate"] = dict(
            min_bytes=tot_bytes, us=round(tot_us, 3), GBps=round(tot_bytes / tot_us / 1e3, 1),
            frac_hbm=round(tot_bytes / tot_us / 1e3 / HBM_PEAK_GBPS, 4))
        log(f"bf16 sweep aggregate {extra['bf16_sweep_aggregate']['GBps']} GB/s "
            f"({extra['bf16_sweep_aggregate']['frac_hbm']} of HBM)")
        others = []
        for name in ("c2_dcnv4_f16_56", "c4s1_dcnv3_bf16_128", "c4s2_dcnv3_bf16_128", "c5_dcnv4_f32_56_fwdbwd"):
            r = forward_record(inputs.WORKLOADS[name], args.steps, args.warmup)
            log(f"{name}: {r['us']} us, {r['GBps']} GB/s")
            others.append(r)
        extra["other_forward"] = others
        # DCNv4's own tensor layout: offsets and mask in one record per (pixel, group)
        packed = []
        for name in ("c2_dcnv4_f16_56", "c3a_dcnv4_bf16_56"):
            r = forward_record(inputs.WORKLOADS[name], args.steps, args.warmup, packed=True)
            log(f"{name} packed: {r['us']} us, {r['GBps']} GB/s")
            packed.append(r)
        extra["packed_forward"] = packed
        bwd = []
        for dt in ("f32", "f16", "bf16"):
            wb = w5 if dt == "f32" else inputs.scaled(w5, dtype=dt)
            bms, beager, R = time_launches(wb, max(20, args.steps // 4), min(args.warmup, 10), backward=True)
            bwd.append(dict(workload=f"{w5.name} ({dt})", dtype=dt, us=round(bms * 1e3, 3),
                            eager_us=round(beager * 1e3, 3), eager_each=dict(LAST_SPREAD),
                            min_bytes=wb.min_bytes_backward(),
                            GBps=round(wb.min_bytes_backward() / (bms * 1e-3) / 1e9, 1),
                            frac_hbm=round(wb.min_bytes_backward() / (bms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            counters=backward_counter_record(w5.name, dt)))
            log(f"backward {w5.name} {dt}: {bwd[-1]['us']} us")
        extra["backward"] = bwd[0]
        extra["backward_half"] = bwd[1:]
        lay = layer_record(inputs.WORKLOADS["c2_dcnv4_f16_56"], max(20, args.steps // 4), 5)
        extra["dcnv4_layer"] = lay
        log(f"DCNv4 layer at c2_dcnv4_f16_56: forward {lay['forward_us']} us, forward+backward "
            f"{lay['forward_backward_us_eager']} us eager, {lay['forward_backward_us_graph']} us in a graph; "
            f"gate {lay['gate_kernel']['us']} us ({lay['gate_kernel']['GBps']} GB/s); value projection "
            f"{lay['value_projection']['us']} us ({lay['value_projection']['GBps']} GB/s, platform BLAS "
            f"{lay['value_projection']['platform_blas_us']} us); offset+mask weight gradient "
            f"{lay['offset_mask_weight_grad']['us']} us (batched BLAS {lay['offset_mask_weight_grad']['batched_blas_us']} us)")
        fii = fii_t_sweep(max(5, args.steps // 20), 2)
        extra["fii_t_core_op"] = fii
        log(f"FlashInternImage-T core op: {fii['us_per_batch']} us per batch of {fii['batch']}, "
            f"{fii['us_per_image']} us per image")

    cpu = None
    if not args.quick and not args.no_cpu_baseline:
        cpu = cpu_baseline(w)
        log(f"cpu oracle {cpu['value']} GB/s on {cpu['cores']} threads; headline parity {cpu.get('parity')}")
        names = [r["workload"] for r in extra["bf16_sweep"] + extra["other_forward"]]
        par = parity_per_config(names)
        for r in extra["bf16_sweep"] + extra["other_forward"]:
            r["parity"] = par.get(r["workload"])
        for r in [extra["backward"]] + extra["backward_half"]:
            r["parity"] = par.get(f"{w5.name}@{r['dtype']} backward")
        bad = [k for k, v in par.items() if not all(x["ok"] for x in (v.values() if "ok" not in v else [v]))]
        log(f"per-config parity (image 0 vs the oracle): {len(par) - len(bad)} of {len(par)} within bound"
            + (f"; outside: {bad}" if bad else ""))

    agg = extra.get("bf16_sweep_aggregate")
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: DCNv4 core forward, {w.dtype} in/out with fp32 accumulation, "
                               f"N={w.N}, {w.H}x{w.W}, C={w.C}, G={w.G} (Cg={w.Cg}), K={w.K}, "
                               f"stride {w.stride}, pad {w.pad}, raw mask, offsets N(0, {w.offset_sigma}^2) px "
                               f"(FlashInternImage-T stage 1)",
                   "global_batch": w.N, "parallelism": "single GPU"},
        "Gsamples_s": head["Gsamples_s"],
        "frac_hbm_peak": head["frac_hbm"],
        "headline_aggregate": None if agg is None else dict(
            workload="bf16 FlashInternImage-T stage sweep (56/28/14/7 px), byte-weighted", **agg),
        "eager_ms_per_step": round(head["eager_us"] / 1e3, 6),
        "eager_each": head["eager_each"],
        "roofline": {"bound": "hbm", "achieved": head["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": head["frac_hbm"],
                     "traffic": traffic_record(w.name, head["min_bytes"]),
                     "valu": head.get("valu")},
        "counters": head.get("counters"),
        "cpu_baseline": cpu,
        "kernel_hash": kernel_hash(),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
