#!/usr/bin/env python3
"""Benchmark of deformable aggregation on one MI355X.

One step = one pass of the whole hot path on one batch: da_forward then
da_backward (location, weight and feature gradients, the latter gathered per
feature row through a caller-side workspace) on the nuScenes-shaped workload (bs=1, 6 cameras, 4 scales 64x176 / 32x88 / 16x44 /
8x22, C=256, G=8, 900 anchors, 13 keypoints), inputs resident in HBM.

Prints ONE JSON line.  value = bilinear sample-channels per second over
forward + backward (bs*A*P*K*S*C per step / step time); the step time is the
wall time of K replays of one HIP graph holding a captured step (the library
launches kernels only, so the graph replays exactly the calls' kernels), between
device synchronisations; --launch eager times K eager steps instead, and
eager_ms_per_step always reports that figure.  forward / backward avg_us are
eager calls (HIP events on the call's stream); their graph_us (graph launch only)
is the same call's time with eight calls back to back in one captured graph.

The roofline entries divide the compulsory bytes of each direction (every input
tensor read once, every output tensor written once) by the HIP-event time of
that call and compare the rate with the HBM peak.  Their "effective" entry
counts every access instead (all four corner rows of every sample; in the
backward also one feature-gradient term per sample, corner and channel) and
compares that rate with the measured rate at which the vector memory path
delivers cache-resident bytes to the CUs (vector_memory_reference).  traffic is
the counter-measured bytes beyond L2 of the same call, read from
profiles/traffic_nuscenes.json while the kernel sources are unchanged.
cpu_baseline is the plain fp64 C oracle, single-threaded, on the same workload
(with the host's CPU model and core counts); cpu_baseline_forward_parallel times
the oracle's forward spread over all usable host cores.  copy_reference is a
plain device copy's rate, and each roofline entry also gives its fraction of
that (frac_of_copy).  --cold adds per-call times after a 512 MiB write that
evicts the inputs from L2 and the MALL.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_nuscenes.json")


AGG_SOURCES = ("da_forward.hip", "da_backward.hip", "da_api.cpp", "da_internal.h", "da_device.h")


def kernel_source_hash():
    """Hash of the aggregation's kernel and launch sources: counter-derived traffic
    is reported only for the code it was measured on."""
    import hashlib
    from view_deformable_feature_amd.build import CSRC
    h = hashlib.sha256()
    for f in sorted(os.path.join(CSRC, x) for x in AGG_SOURCES):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per call from the committed rocprofv3 counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t


def copy_calibration(nbytes):
    """A plain device-to-device copy of known size, to scale the FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


FWD_KERNELS = "da_forward call: da_forward_sliced_kernel, fwd_reduce_kernel"
BWD_KERNELS = ("da_backward call: prep_kernel, count_kernel (+ count_tiles_kernel for levels "
               "above 16384 rows), scan_tiles_kernel (+ scan_totals_kernel above 256 tiles), "
               "bucket_kernel (+ zeroing blocks), "
               "gather_kernel (+ group dot products), finalize_kernel")
BWD_ATOMIC_KERNELS = ("da_backward_atomic call: fill_zero_kernel, da_backward_anchor_kernel "
                      "(binary32 atomics into grad_feat)")


def compulsory_bytes(wl, out_bytes=4):
    """(forward, backward) bytes that must cross HBM once per call: every input tensor
    read once and every output tensor written once.  Forward: features, locations,
    weights in, out (out_bytes per element) out.  Backward: the same inputs and
    grad_out in; grad_feat (binary32), grad_loc and grad_weights out.  No call can
    move less, so bytes / call time is at most the HBM peak whenever the call
    starts with its inputs outside the on-chip caches."""
    e = wl.feat_elem_bytes
    feat = wl.bs * wl.num_feat * wl.C * e
    loc = wl.bs * wl.anchors * wl.pts * wl.num_cams * 2 * 4
    weights = wl.num_samples * wl.groups * 4
    out = wl.bs * wl.anchors * wl.C * out_bytes
    b_fwd = feat + loc + weights + out
    b_bwd = feat + loc + weights + out + wl.bs * wl.num_feat * wl.C * 4 + loc + weights
    return b_fwd, b_bwd


def effective_bytes(wl, out_bytes=4):
    """Bytes each direction reads or writes counting every access (the effective
    gathered bytes): all four corner rows of every sample, locations, weights and out
    (or grad_out) of out_bytes per element, plus the backward's gradients with one
    binary32 feature-gradient term per (sample, corner, channel).  Most of these are
    re-reads served by the on-chip caches."""
    n_s = wl.num_samples
    n_pk = wl.bs * wl.anchors * wl.pts * wl.num_cams
    e = wl.feat_elem_bytes
    C, G = wl.C, wl.groups
    b_fwd = 4 * C * e * n_s + 8 * n_pk + 4 * G * n_s + out_bytes * wl.bs * wl.anchors * C
    b_bwd = (out_bytes * wl.bs * wl.anchors * C + 4 * C * e * n_s + 16 * C * n_s + 16 * n_pk
             + 8 * G * n_s)
    return b_fwd, b_bwd


def vector_memory_reference(reps=5):
    """GB/s that a plain streaming kernel of 16-byte loads (libbwprobe.so) reaches
    when its buffer is resident in each CU's vector L1 (16 KiB buffer), in each XCD's
    L2 (2 MiB buffer, 64 KiB per pass, beyond L1), in the Infinity Cache (64 MiB:
    beyond the 8 x 4 MiB of L2, within the 256 MiB MALL) and in HBM only (1 GiB).  The
    L1-resident rate is the fastest the vector memory path delivers bytes to the CUs:
    the roof of the effective bytes."""
    import ctypes
    import torch
    from view_deformable_feature_amd.build import PROBE_PATH
    lib = ctypes.CDLL(PROBE_PATH)
    lib.bwprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                 ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                 ctypes.c_uint64, ctypes.c_void_p]
    lib.bwprobe_read.restype = ctypes.c_int
    blocks = 256 * 16
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    res = {}
    for name, buf_bytes, chunk, passes in (("l1_resident", 16 << 10, 16 << 10, 256),
                                           ("l2_resident", 2 << 20, 64 << 10, 64),
                                           ("mall_resident", 64 << 20, 64 << 10, 16),
                                           ("hbm", 1 << 30, 64 << 10, 16)):
        buf = torch.ones(buf_bytes // 4, dtype=torch.float32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def run():
            rc = lib.bwprobe_read(ctypes.c_void_p(buf.data_ptr()), buf_bytes, chunk, passes,
                                  blocks, ctypes.c_void_p(sink.data_ptr()), sink.numel(), stream)
            if rc:
                raise RuntimeError(f"bwprobe_read failed ({rc})")
        run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        res[name] = round(blocks * chunk * passes / float(np.median(ts)) / 1e9, 1)
    return {"l1_resident_gbs": res["l1_resident"], "l2_resident_gbs": res["l2_resident"],
            "mall_resident_gbs": res["mall_resident"], "hbm_gbs": res["hbm"],
            "unit": "GB/s", "kind": f"16-byte loads streaming a 16 KiB / 2 MiB / 64 MiB / 1 GiB "
                                    f"buffer, {blocks} workgroups of 256 threads, median of "
                                    f"{reps}"}


def effective_entry(bytes_, secs, vref):
    """The effective bytes over the call time, against the vector-memory delivery rate
    measured by vector_memory_reference (its L1-resident figure: no load returns data
    to the CUs faster)."""
    a = bytes_ / secs / 1e9
    peak = vref["l1_resident_gbs"]
    return {"bytes": int(bytes_), "achieved": round(a, 1), "peak": peak, "unit": "GB/s",
            "frac": round(a / peak, 4),
            "peak_source": "measured: streaming 16-byte loads from an L1-resident buffer"}


def host_info():
    """CPU model and core counts of the host that runs the oracle baselines."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu": model, "nproc": os.cpu_count(), "usable_cores": usable}


def cpu_forward_parallel(wl, inp, min_seconds=3.0):
    """The oracle's forward spread over the host's usable cores by anchor (OpenMP,
    race-free: every anchor writes its own row); a second CPU reference beside the
    one-thread loop, forward only."""
    import oracle
    args = [inp[k] for k in ("feat", "spatial_shape", "scale_start_index", "loc", "weights")]
    threads = host_info()["usable_cores"] or 1
    oracle.forward_parallel(*args, threads=threads)          # warm up, spawn the threads
    reps, t0, used = 0, time.perf_counter(), 0
    while True:
        _, used = oracle.forward_parallel(*args, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return dict(value=wl.sample_channels * reps / el, unit="sample-channels/s", cores=used,
                kind="oracle, forward only, OpenMP over anchors",
                sample=f"full {wl.name} workload, forward, {reps} passes in {el:.1f} s")


def copy_reference(nbytes=1 << 30, reps=10):
    """GB/s (bytes read + written) of a plain device-to-device copy of nbytes: what a
    pure streaming kernel reaches on this GPU, printed beside the vendor peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return {"achieved": round(2 * nbytes / float(np.median(ts)) / 1e9, 1), "unit": "GB/s",
            "bytes_per_copy": nbytes, "kind": "device-to-device copy, read + write, median of "
                                              f"{reps}"}


def cpu_baseline(wl, inp, min_seconds=10.0):
    """Time the fp64 oracle (forward + backward) on the host; single-threaded C."""
    import oracle
    args = [inp[k] for k in ("feat", "spatial_shape", "scale_start_index", "loc", "weights")]
    oracle.forward(*args, anchor_ids=[0])          # load / build outside the timed region
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(*args)
        oracle.backward(*args, inp["grad_out"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return dict(value=wl.sample_channels * reps / el, unit="sample-channels/s", cores=1,
                kind="oracle",
                sample=f"full {wl.name} workload, forward + backward, {reps} passes in {el:.1f} s "
                       f"(fp64 C loop, one thread)", host=host_info())


def bench_pack(args):
    """Level packing (section 6, feature_maps_format) of the workload's per-scale
    camera maps [B, N, C, H_s, W_s] into [B, num_feat, C], and back.  Each direction
    reads and writes the whole tensor once: algorithmic bytes = 2 x tensor bytes."""
    import torch
    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd import workloads as W
    wl = W.WORKLOADS[args.workload]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.feat_dtype]
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    maps = [torch.randn((wl.bs, wl.num_cams, wl.C, h, w), device="cuda", generator=gen).to(dt)
            for h, w in wl.levels]
    _, _, nf = vdf.pack_layout(list(wl.levels), wl.num_cams, wl.C, dt)
    packed = torch.empty((wl.bs, nf, wl.C), device="cuda", dtype=dt)
    outs = [torch.empty_like(m) for m in maps]
    nbytes = packed.numel() * packed.element_size()
    # the C entry points with their arguments marshalled once: a pack of the
    # nuScenes maps takes ~35 us, less than one pass through the Python checks
    import ctypes
    from view_deformable_feature_amd import _lib
    from view_deformable_feature_amd.pack import _problem, _scale_hw
    lib = _lib.load()
    prob = _problem(wl.bs, wl.num_cams, len(wl.levels), wl.C, dt)
    hw = _scale_hw(list(wl.levels))
    hwp = hw.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    in_ptrs = (ctypes.c_void_p * len(maps))(*[m.data_ptr() for m in maps])
    out_ptrs = (ctypes.c_void_p * len(outs))(*[m.data_ptr() for m in outs])
    pk = ctypes.c_void_p(packed.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    vdf.da_pack_levels(maps, out=packed)                  # checked once through the binding
    vdf.da_unpack_levels(packed, list(wl.levels), wl.num_cams, out=outs)
    res = {}
    for name, fn in (("pack", lambda: lib.da_pack_levels(ctypes.byref(prob), hwp, in_ptrs, pk,
                                                         stream)),
                     ("unpack", lambda: lib.da_unpack_levels(ctypes.byref(prob), hwp, pk,
                                                             out_ptrs, stream))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e-3 / args.steps
    t = res["pack"] + res["unpack"]
    a = 2 * nbytes / res["pack"] / 1e9
    rec = {"metric": "level packing: bytes read + written per second (pack then unpack)",
           "value": 4 * nbytes / t, "unit": "B/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": wl.feat_dtype, "data": "synthetic",
           "config": {"workload": f"{wl.name} feature maps: {wl.num_cams} cameras, scales "
                                  + "/".join(f"{h}x{w_}" for h, w_ in wl.levels)
                                  + f", C={wl.C}, bs={wl.bs}", "tensor_bytes": nbytes},
           "pack_us": res["pack"] * 1e6, "unpack_us": res["unpack"] * 1e6,
           "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "pack_kernel (pack direction)",
                        "algorithmic_bytes": 2 * nbytes,
                        "avg_launch_us": round(res["pack"] * 1e6, 2)},
           "roofline_unpack": {"bound": "hbm",
                               "achieved": round(2 * nbytes / res["unpack"] / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(2 * nbytes / res["unpack"] / 1e9 / HBM_PEAK_GBS, 4)}}
    print(json.dumps(rec), flush=True)


def dcn_bytes(wl, out_bytes=4):
    """(forward, backward) algorithmic bytes of one deformable-convolution call, the
    DCNv4 notes' worst-case accounting: every (pixel, group, tap) sample reads its
    four corner vectors of D channels and its offsets and scalar; each output
    element is written once.  The backward also reads grad_out and writes the
    input gradient of every corner term and the offset / scalar gradients."""
    D, e = wl.C // wl.groups, wl.elem_bytes
    ho, wo = wl.out_hw
    n_s = wl.samples
    out_el = wl.N * ho * wo * wl.C
    b_fwd = n_s * (4 * D * e + 12) + out_el * out_bytes
    b_bwd = n_s * (4 * D * e + 12 + 4 * D * 4 + 12) + out_el * out_bytes
    return b_fwd, b_bwd


GRAPH_LAUNCH = "hip graph: one captured step (forward + backward), replayed"


def graph_step_seconds(step, warmup, steps):
    """Wall time per step of `steps` replays of one HIP graph holding a captured
    step (after a warm-up call on a side stream and `warmup` replays), between
    device synchronisations.  The library's calls only launch kernels, so the
    graph replays exactly their kernels."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    del graph
    return t


def graph_call_seconds(fn, calls, replays):
    """Time per call of `calls` back-to-back calls of fn captured in one HIP graph
    and replayed `replays` times (HIP events on the replaying stream): the calls'
    kernels alone, without the host's launch gaps of eager calls."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (calls * replays)
    del graph
    return t


def bench_dcn(args):
    """Deformable convolution (DCNv3 / DCNv4 operator): forward + backward on the
    shape the DCNv4 notes time (56x56x128, batch 64, 4 groups by default)."""
    import torch
    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd import workloads as W
    wl = W.DCN_WORKLOADS[args.workload]
    inp = W.make_dcn_inputs(wl)
    dev = torch.device("cuda:0")
    x = inp["input"]
    if x.dtype == np.uint16:
        x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        x = torch.from_numpy(x).to(dev)
    om = torch.from_numpy(inp["offset_mask"]).to(dev)
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.out_dtype]
    go = torch.from_numpy(inp["grad_out"]).to(dev).to(odt)
    conf = dict(groups=wl.groups, kernel=wl.kernel, stride=wl.stride, pad=wl.pad,
                dilation=wl.dilation)
    out = torch.empty(tuple(go.shape), device=dev, dtype=odt)
    gi = torch.empty(tuple(x.shape), device=dev, dtype=torch.float32)
    gom = torch.empty_like(om)
    nws = vdf.dcn_workspace_size(x, **conf, grad_out_dtype=odt)
    ws = torch.empty(nws, device=dev, dtype=torch.uint8) if nws else None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        vdf.dcn_forward(x, om, **conf, out=out)
        if ev is not None:
            ev[1].record()
        vdf.dcn_backward(x, om, go, **conf, grad_input=gi, grad_offset_mask=gom, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_all = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    b_all = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_fwd, t_bwd = float(f_all.mean()), float(b_all.mean())
    t_step = t_eager = wall / args.steps
    launch = "eager calls"
    if args.launch == "graph":
        t_step = graph_step_seconds(step, args.warmup, args.steps)
        launch = GRAPH_LAUNCH
    e_fwd, e_bwd = dcn_bytes(wl, out.element_size())
    # compulsory: input and offset_mask read once, out written once; the backward
    # also reads grad_out and writes grad_input (binary32) and grad_offset_mask
    n_in = x.numel() * x.element_size()
    n_om = om.numel() * om.element_size()
    n_out = out.numel() * out.element_size()
    b_fwd = n_in + n_om + n_out
    b_bwd = n_in + n_om + n_out + gi.numel() * 4 + gom.numel() * 4
    sc = wl.sample_channels
    vref = vector_memory_reference()

    def roof(b, eff, t, kernel):
        a = b / t / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel,
                "algorithmic_bytes": int(b),
                "algorithmic": "compulsory: each input read once, each output written once",
                "avg_launch_us": round(t * 1e6, 2),
                "effective": effective_entry(eff, t, vref)}

    ho, wo = wl.out_hw
    rec = {"metric": "deformable convolution: bilinear sample-channels/s, forward + backward",
           "value": sc / t_step, "unit": "sample-channels/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": ("f32" if wl.dtype == "f32" and args.out_dtype == "f32"
                     else f"{wl.dtype}-input/{args.out_dtype}-out/f32"),
           "data": "synthetic",
           "config": {"workload": f"{wl.name}: N={wl.N}, {wl.H}x{wl.W}x{wl.C}, groups={wl.groups}, "
                                  f"kernel {wl.kernel[0]}x{wl.kernel[1]}, out {ho}x{wo}",
                      "sample_channels_per_step": sc, "out_dtype": args.out_dtype,
                      "launch": launch},
           "eager_ms_per_step": t_eager * 1e3,
           "forward": {"avg_us": t_fwd * 1e6, "median_us": float(np.median(f_all)) * 1e6,
                       "value": sc / t_fwd, "unit": "sample-channels/s"},
           "backward": {"avg_us": t_bwd * 1e6, "median_us": float(np.median(b_all)) * 1e6,
                        "value": sc / t_bwd, "unit": "sample-channels/s"},
           "roofline": roof(b_bwd, e_bwd, t_bwd, "dcn_backward call: fill_zero_kernel, "
                                                 "dcn_bound_kernel, dcn_bwd_tile_kernel, "
                                                 "dcn_far_kernel"),
           "roofline_forward": roof(b_fwd, e_fwd, t_fwd, "dcn_forward_kernel"),
           "vector_memory_reference": vref}
    if args.launch == "graph":
        # the same calls' kernels back to back in one captured graph
        reps = max(2, args.steps // 8)
        rec["forward"]["graph_us"] = graph_call_seconds(
            lambda: vdf.dcn_forward(x, om, **conf, out=out), 8, reps) * 1e6
        rec["backward"]["graph_us"] = graph_call_seconds(
            lambda: vdf.dcn_backward(x, om, go, **conf, grad_input=gi, grad_offset_mask=gom,
                                     workspace=ws), 8, reps) * 1e6
    cref = copy_reference()
    rec["copy_reference"] = cref
    for key in ("roofline", "roofline_forward"):
        rec[key]["frac_of_copy"] = round(rec[key]["achieved"] / cref["achieved"], 4)
    if not args.no_cpu_baseline:
        import oracle
        sub = W.dcn_custom(wl.name + "_sample", N=1, H=wl.H, W=wl.W, C=wl.C, groups=wl.groups,
                           kernel=wl.kernel, stride=wl.stride, pad=wl.pad, dilation=wl.dilation,
                           dtype=wl.dtype, seed=wl.seed)
        si = W.make_dcn_inputs(sub)
        oracle.dcn_out_size(wl.H, wl.W, wl.kernel, wl.stride, wl.pad, wl.dilation)
        reps, c0 = 0, time.perf_counter()
        while True:
            oracle.dcn_forward(si["input"], si["offset_mask"], **conf)
            oracle.dcn_backward(si["input"], si["offset_mask"], si["grad_out"], **conf)
            reps += 1
            el = time.perf_counter() - c0
            if el >= args.cpu_seconds:
                break
        rec["cpu_baseline"] = {"value": sub.sample_channels * reps / el, "unit": "sample-channels/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"one image of {wl.name} (1 of {wl.N}), forward + backward, "
                                         f"{reps} passes in {el:.1f} s (fp64 C loop, one thread)",
                               "host": host_info()}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="nuscenes_bwd",
                    help="workload name (nuscenes_bwd is the headline one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    ap.add_argument("--out-dtype", default="f32", choices=("f32", "bf16", "f16"),
                    help="element type of out and grad_out (binary32 arithmetic throughout)")
    ap.add_argument("--deterministic", action="store_true",
                    help="run the backward in its deterministic (64-bit fixed-point) form")
    ap.add_argument("--backward", default="gather", choices=("gather", "atomic"),
                    help="gather: da_backward (row-sorted gather, the default); atomic: "
                         "da_backward_atomic, the page's scatter of every feature-gradient "
                         "term with a binary32 atomic")
    ap.add_argument("--launch", default="graph", choices=("graph", "eager"),
                    help="time the step as replays of one captured HIP graph (default) or as "
                         "eager calls; the per-call forward / backward times are eager either way")
    ap.add_argument("--cold", action="store_true",
                    help="also time each call after writing a 512 MiB buffer (L2 and MALL "
                         "hold none of the inputs)")
    ap.add_argument("--op", default="aggregate", choices=("aggregate", "pack", "dcn"),
                    help="aggregate: forward + backward step (the headline); pack: level "
                         "packing and unpacking of the workload's feature maps; dcn: the "
                         "deformable convolution (workload dcn_56, dcn_28, dcn_14, dcn_56_f16)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the op would shard).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.op == "pack":
        bench_pack(args)
        return
    if args.op == "dcn":
        if args.workload == "nuscenes_bwd":
            args.workload = "dcn_56"
        bench_dcn(args)
        return

    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    inp = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if inp["feat"].dtype == np.uint16:
        feat = torch.from_numpy(inp["feat"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        feat = torch.from_numpy(inp["feat"]).to(dev)           # float32 or float16
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.out_dtype]
    loc = torch.from_numpy(inp["loc"]).to(dev)
    w = torch.from_numpy(inp["weights"]).to(dev)
    go = torch.from_numpy(inp["grad_out"]).to(dev).to(odt)
    shape, start = inp["spatial_shape"], inp["scale_start_index"]
    out = torch.empty((wl.bs, wl.anchors, wl.C), device=dev, dtype=odt)
    gf = torch.empty(tuple(feat.shape), device=dev, dtype=torch.float32)
    gl = torch.empty(tuple(loc.shape), device=dev, dtype=torch.float32)
    gw = torch.empty(tuple(w.shape), device=dev, dtype=torch.float32)
    # caller-owned workspaces, allocated once, as a training loop would hold them
    fws_n = vdf.forward_workspace_size(feat, shape, loc, w)
    fws = torch.empty(fws_n, device=dev, dtype=torch.uint8) if fws_n else None
    det = args.deterministic
    atomic = args.backward == "atomic"
    if atomic and det:
        raise SystemExit("the atomic backward has no deterministic form")
    bws = None if atomic else torch.empty(vdf.workspace_size(feat, shape, loc, w, deterministic=det,
                                                             grad_out_dtype=odt),
                                          device=dev, dtype=torch.uint8)

    def backward():
        if atomic:
            vdf.da_backward_atomic(feat, shape, start, loc, w, go, grad_feat=gf, grad_loc=gl,
                                   grad_weights=gw)
        else:
            vdf.da_backward(feat, shape, start, loc, w, go, grad_feat=gf, grad_loc=gl,
                            grad_weights=gw, workspace=bws, deterministic=det)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        vdf.da_forward(feat, shape, start, loc, w, out=out, workspace=fws)
        if ev is not None:
            ev[1].record()
        backward()
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_fwd = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_bwd = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_step = wall / args.steps
    t_eager = t_step
    launch = "eager calls"
    if args.launch == "graph":
        t_step = graph_step_seconds(step, args.warmup, args.steps)
        launch = GRAPH_LAUNCH
    b_fwd, b_bwd = compulsory_bytes(wl, out.element_size())
    e_fwd, e_bwd = effective_bytes(wl, out.element_size())
    sc = wl.sample_channels
    fwd_s, bwd_s = float(t_fwd.mean()), float(t_bwd.mean())
    dominant = "backward" if bwd_s >= fwd_s else "forward"
    vref = vector_memory_reference()

    # counter totals are taken on the binary32-out configuration only
    traffic = measured_traffic(wl.name) if args.out_dtype == "f32" else None

    def roof(bytes_, eff, secs, kernel, direction):
        a = bytes_ / secs / 1e9
        t = None
        if traffic is not None and direction in traffic:
            t = int(traffic[direction]["fetch_bytes"] + traffic[direction]["write_bytes"])
        r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBS, 4), "traffic": t, "kernel": kernel,
             "algorithmic_bytes": int(bytes_),
             "algorithmic": "compulsory: each input read once, each output written once",
             "avg_launch_us": round(secs * 1e6, 2),
             "effective": effective_entry(eff, secs, vref)}
        if t is not None:
            # counter-measured bytes (FETCH_SIZE + WRITE_SIZE, beyond L2) of the same
            # call, taken from the committed profile, over this run's call time
            r["traffic_source"] = (f"{os.path.relpath(TRAFFIC_FILE, ROOT)}: rocprofv3 --pmc on "
                                   "the same kernel sources, not measured in this run")
            r["traffic_gbs"] = round(t / secs / 1e9, 1)
            r["traffic_frac"] = round(t / secs / 1e9 / HBM_PEAK_GBS, 4)
        return r

    rec = {
        "metric": "bilinear sample-channels/s, forward + backward (1 GPU)",
        "value": sc / t_step,
        "unit": "sample-channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32" if wl.feat_dtype == "f32" and args.out_dtype == "f32"
                  else f"{wl.feat_dtype}-features/{args.out_dtype}-out/f32"),
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: bs={wl.bs}, {wl.num_cams} cameras, scales "
                               + "/".join(f"{h}x{w_}" for h, w_ in wl.levels)
                               + f", C={wl.C}, groups={wl.groups}, anchors={wl.anchors}, "
                                 f"points={wl.pts}",
                   "sample_channels_per_step": sc, "out_dtype": args.out_dtype,
                   "backward_form": ("atomic scatter (da_backward_atomic)" if atomic else
                                     "deterministic" if det else "default"),
                   "launch": launch},
        "eager_ms_per_step": t_eager * 1e3,
        "forward": {"value": sc / fwd_s, "unit": "sample-channels/s", "avg_us": fwd_s * 1e6},
        "backward": {"avg_us": bwd_s * 1e6, "value": sc / bwd_s, "unit": "sample-channels/s"},
        "roofline": roof(b_bwd, e_bwd, bwd_s,
                         (BWD_ATOMIC_KERNELS if atomic else BWD_KERNELS)
                         + (" (prep_kernel also converts grad_out)"
                            if args.out_dtype != "f32" and not atomic else ""),
                         "backward_atomic" if atomic else "backward")
        if dominant == "backward" else roof(b_fwd, e_fwd, fwd_s, FWD_KERNELS, "forward"),
        "roofline_forward": roof(b_fwd, e_fwd, fwd_s, FWD_KERNELS, "forward"),
        "vector_memory_reference": vref,
    }
    rec["forward"]["median_us"] = float(np.median(t_fwd)) * 1e6
    rec["backward"]["median_us"] = float(np.median(t_bwd)) * 1e6
    if args.launch == "graph":
        # the same calls' kernels back to back in one captured graph
        reps = max(2, args.steps // 8)
        rec["forward"]["graph_us"] = graph_call_seconds(
            lambda: vdf.da_forward(feat, shape, start, loc, w, out=out, workspace=fws), 8, reps) * 1e6
        rec["backward"]["graph_us"] = graph_call_seconds(backward, 8, reps) * 1e6
    if args.cold:
        # a 512 MiB write between calls evicts the inputs from L2 and the MALL
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        cf, cb = [], []
        for _ in range(max(5, args.steps // 5)):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            flush.fill_(0.0)
            e[0].record()
            vdf.da_forward(feat, shape, start, loc, w, out=out, workspace=fws)
            e[1].record()
            flush.fill_(1.0)
            e[2].record()
            backward()
            e[3].record()
            torch.cuda.synchronize()
            cf.append(e[0].elapsed_time(e[1]) * 1e-3)
            cb.append(e[2].elapsed_time(e[3]) * 1e-3)
        del flush
        rec["cold"] = {"forward_median_us": float(np.median(cf)) * 1e6,
                       "backward_median_us": float(np.median(cb)) * 1e6,
                       "calls": len(cf), "flush_bytes": 512 << 20}
    cref = copy_reference()
    rec["copy_reference"] = cref
    for key in ("roofline", "roofline_forward"):
        rec[key]["frac_of_copy"] = round(rec[key]["achieved"] / cref["achieved"], 4)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        rec["cpu_baseline_forward_parallel"] = cpu_forward_parallel(wl, inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
