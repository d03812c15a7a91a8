#!/usr/bin/env python3
"""Throughput of the MSDeformAttn sampling core on one MI355X.

A step is one pass of the whole hot path over one batch: the forward
(msda_forward) and the backward (msda_backward: grad_attn/grad_loc kernel
beside the grad_value pipeline) at the Deformable-DETR encoder shape -- B=2,
four levels 100x167, 50x84, 25x42, 13x21 (Nv = 22,223), every pixel a query
(Nq = Nv), M=8 heads, D=32, K=4, fp32.  Inputs are seeded synthetic data
(workloads.make) resident in HBM before the timed region; their SHA-256s are
in the line.

Printed: one JSON line.  value = sampled points (B*Nq*M*L*K) per second of
fwd+bwd steps, timed with HIP events over `--steps` back-to-back steps.
"roofline" describes the dominant kernel: the one with the largest warm
duration in a per-kernel breakdown taken first (torch events around the
forward; the backward's own stage events, msda_backward_events, recorded on
the stream that runs each kernel, the side stream included).  Inside the
timed region that kernel, and only it, is bracketed by HIP events on its
stream in every step (an event record costs the stream a few microseconds);
its algorithmic bytes (each tensor it must touch read or written once) over
its average duration there give "achieved", against the 8 TB/s HBM peak.
"traffic" is the HBM byte count rocprofv3 measured for that kernel
(profiles/traffic.json) and "counters" its L2 hit rate and atomic requests
(profiles/counters.json), each when taken on the current 2-D kernel sources.
"roofline.alone" is the same kernel timed with the backward on one stream,
nothing beside it.  "roofline.forward" places the forward against both of its ceilings: the HBM
roofline (cold and warm) and the row-gather rate of the vector memory path,
measured here by the probe kernel of libmsda_probe.so ("gather_ceiling").
"stream_copy" is a streaming 16-byte copy, the achievable HBM bandwidth.
"decoder" and "train_bf16" are the other two configurations (forward and
backward each).  "cpu_baseline" times the CPU oracle on this host's cores
and on one core.  --extra adds the encoder backward in workspaces below its
one-pass size (grad_value in passes, and the no-allocation entry point), the
fused prologue at the encoder shape, the 3-D trilinear variant on a voxel
workload, and DAT's sampled-key attention (sampling and MFMA attention) at its
two configurations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20   # > the 256 MB Infinity Cache
CSRC = os.path.join(ROOT, "scale_deformable_attention_04_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f)
                  for f in ("common.h", "bins.h", "msda.hip", "msda3d.hip", "dat_attn.hip",
                            "probe.hip")]
# the sources the 2-D kernels are built from: the traffic counters of
# profiles/traffic.json hold while these are unchanged
ENCODER_SOURCES = [os.path.join(CSRC, f) for f in ("common.h", "bins.h", "msda.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")

# kernel names as rocprofv3 reports them, per stage of a step
KERNELS = {
    "forward": "msda_fwd_kernel<32, float, false, 1>",
    "clear_bins": "fill_zero_kernel",
    "count": "bin_count_kernel<false>",
    "dots": "bwd_dots_kernel<32, float>",
    "scan": "bin_scan_kernel<false>",
    "scatter": "bin_scatter_kernel<false>",
    "tiles": "grad_value_gather_kernel<32, false, 16>",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(files=None) -> str:
    files = KERNEL_SOURCES if files is None else files
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()[:16]


def byte_model(B, Nv, Nq, M, D, L, K, value_bytes=4):
    """Algorithmic bytes per kernel: every tensor it needs read or written once."""
    pts = B * Nq * M * L * K
    value = B * Nv * M * D * value_bytes
    loc, attn = pts * 2 * 4, pts * 4
    rows = B * Nq * M * D * 4           # out or grad_out
    gvalue = B * Nv * M * D * 4
    return {
        "points": pts,
        "forward": value + loc + attn + rows,
        "backward": value + loc + attn + rows + gvalue + loc + attn,
        "count": loc,
        "dots": value + loc + attn + rows + loc + attn,    # grad_loc, grad_attn written
        "scatter": loc + attn,
        "tiles": rows + gvalue,
    }


def to_device(w, torch, bf16=False):
    import numpy as np
    d = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    if bf16:
        value = torch.from_numpy(w.value_bf16.view(np.int16).copy()).view(torch.bfloat16).to(d)
    else:
        value = t(w.value)
    x = dict(value=value, spatial_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
             attn_weight=t(w.attn_weight))
    g = t(w.grad_out) if w.grad_out is not None else None
    return x, g


def time_forward(torch, fn, reps, flush):
    """Mean us of one call timed alone (events around it, synchronized after
    it); with `flush` a 512 MB fill runs before each call, evicting L2 and the
    Infinity Cache (cold)."""
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return statistics.mean(times)


def time_warm(torch, fn, reps):
    """Mean us per call of `reps` calls back to back on torch's stream (warm
    caches; the launch gaps of a steady stream of work, as in a training
    step and as the gather-ceiling probe is timed)."""
    return _time_launches(torch, fn, reps)


def time_backward_stages(torch, msda, x, g, bufs, reps):
    """Mean per-stage us of msda_backward with stage events (as in production:
    the side stream runs concurrently), warm."""
    sets = [msda.make_events() for _ in range(reps)]
    for ev in sets:
        msda.backward(**x, grad_out=g, **bufs, validate=False, events=ev)
    torch.cuda.synchronize()
    acc = [0.0] * len(msda.BWD_STAGES)
    for ev in sets:
        acc = [a + b for a, b in zip(acc, msda.stage_times(ev))]
    return {k: v / reps for k, v in zip(msda.BWD_STAGES, acc)}


def time_backward_total(torch, msda, x, g, bufs, reps):
    """Mean us of one whole msda_backward call (events on the caller's stream)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        msda.backward(**x, grad_out=g, **bufs, validate=False)
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def measure_config(torch, msda, w, bf16, reps, flush, label):
    x, g = to_device(w, torch, bf16)
    dims = w.dims
    bm = byte_model(dims["B"], dims["Nv"], dims["Nq"], dims["M"], dims["D"], dims["L"],
                    dims["K"], 2 if bf16 else 4)
    out = torch.empty(dims["B"], dims["Nq"], dims["M"] * dims["D"], device="cuda")
    res = {"points": bm["points"]}
    fwd = lambda: msda.forward(**x, out=out, validate=False)
    for _ in range(3):
        fwd()
    cold = time_forward(torch, fwd, reps, flush)
    warm = time_warm(torch, fwd, reps)
    res["forward"] = {"us_cold": cold, "us_warm": warm, "points_per_s": bm["points"] / cold * 1e6,
                      "algorithmic_GBps": bm["forward"] / cold / 1e3,
                      "algorithmic_bytes": bm["forward"]}
    if g is not None:
        bufs = dict(grad_value=torch.empty(x["value"].shape, dtype=torch.float32, device="cuda"),
                    grad_sampling_loc=torch.empty_like(x["sampling_loc"]),
                    grad_attn_weight=torch.empty_like(x["attn_weight"]))
        for _ in range(3):
            msda.backward(**x, grad_out=g, **bufs, validate=False)
        stages = time_backward_stages(torch, msda, x, g, bufs, reps)
        total = time_backward_total(torch, msda, x, g, bufs, reps)
        res["backward"] = {"us_warm": total, "stages_us_warm": stages,
                           "points_per_s": bm["points"] / total * 1e6,
                           "algorithmic_GBps": bm["backward"] / total / 1e3,
                           "algorithmic_bytes": bm["backward"]}
    log(f"{label}: {json.dumps(res)}")
    return res, x, g, bm


def measure_bounded(torch, msda, x, g, dims, reps):
    """The encoder backward with workspaces below the one-pass size (grad_value
    in passes, see msda_backward_workspace_min), and through the no-allocation
    entry point (its 64 MiB static scratch), back to back."""
    B, Nv, Nq, M, D, L, K = (dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    full = msda.workspace_size(B, Nv, Nq, M, D, L, K)
    bufs = dict(grad_value=torch.empty(x["value"].shape, dtype=torch.float32, device="cuda"),
                grad_sampling_loc=torch.empty_like(x["sampling_loc"]),
                grad_attn_weight=torch.empty_like(x["attn_weight"]))
    res = {"one_pass_bytes": full,
           "least_bytes": msda.workspace_min(B, Nv, Nq, M, D, L, K)}
    for label, nbytes in (("full", full), ("64MiB", 64 << 20), ("32MiB", 32 << 20)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        fn = lambda: msda.backward(**x, grad_out=g, **bufs, validate=False, workspace=ws)
        for _ in range(3):
            fn()
        res[label] = {"bytes": nbytes, "us_warm": time_warm(torch, fn, reps)}
        del ws
    fn = lambda: msda.backward_noalloc(**x, grad_out=g, side_stream="auto", **bufs)
    for _ in range(3):
        fn()
    res["noalloc"] = {"bytes": msda.NOALLOC_SCRATCH_BYTES, "us_warm": time_warm(torch, fn, reps)}
    log(f"bounded workspace: {json.dumps(res)}")
    return res


def measure_fused(torch, msda, reps, flush):
    """The fused prologue at the encoder shape (reference points, pixel
    offsets, logits): its forward and backward kernels, and one fwd+bwd
    autograd step of it against the same step with the prologue written in
    torch ops around the core entry points."""
    import workloads
    w = workloads.make_fused(3)
    d = torch.device("cuda")
    t = lambda a: torch.from_numpy(a).to(d)
    x = dict(value=t(w.value), spatial_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), reference_points=t(w.reference_points),
             sampling_offsets=t(w.sampling_offsets), attn_logits=t(w.attn_logits))
    g = t(w.grad_out)
    dims = w.dims
    B, Nq, M, L, K = dims["B"], dims["Nq"], dims["M"], dims["L"], dims["K"]
    out = torch.empty(B, Nq, M * dims["D"], device=d)
    fwd = lambda: msda.forward_fused(**x, out=out, validate=False)
    for _ in range(3):
        fwd()
    res = {"points": w.points, "forward": {"us_cold": time_forward(torch, fwd, reps, flush),
                                           "us_warm": time_warm(torch, fwd, reps)}}
    gv = torch.empty(tuple(w.value.shape), dtype=torch.float32, device=d)
    for _ in range(3):
        msda.backward_fused(**x, grad_out=g, grad_value=gv, validate=False)
    sets = [msda.make_events(fused=True) for _ in range(reps)]
    for ev in sets:
        msda.backward_fused(**x, grad_out=g, grad_value=gv, validate=False, events=ev)
    torch.cuda.synchronize()
    acc = [0.0] * len(msda.BWD_FUSED_STAGES)
    for ev in sets:
        acc = [a + b for a, b in zip(acc, msda.stage_times(ev))]
    stages = {k: v / reps for k, v in zip(msda.BWD_FUSED_STAGES, acc)}
    res["backward"] = {"us_warm": time_warm(
        torch, lambda: msda.backward_fused(**x, grad_out=g, grad_value=gv, validate=False),
        reps), "stages_us_warm": stages}
    # a training step: the forward stores the locations and weights, the
    # backward reads them instead of recomputing them
    saved = msda.forward_fused(**x, validate=False, save=True)[1:]
    res["forward_saving"] = {"us_warm": time_warm(
        torch, lambda: msda.forward_fused(**x, validate=False, save=True), reps)}
    res["backward_saved"] = {"us_warm": time_warm(
        torch, lambda: msda.backward_fused(**x, grad_out=g, grad_value=gv, validate=False,
                                           saved=saved), reps)}

    leaves = {k: x[k].clone().requires_grad_(True)
              for k in ("value", "reference_points", "sampling_offsets", "attn_logits")}
    wh = torch.tensor([[W, H] for H, W in w.spatial_shapes.tolist()], dtype=torch.float32,
                      device=d)

    def fused_step():
        o = msda.ms_deform_attn_fused(leaves["value"], x["spatial_shapes"],
                                      x["level_start_index"], leaves["reference_points"],
                                      leaves["sampling_offsets"], leaves["attn_logits"])
        o.backward(g)

    def unfused_step():
        loc = (leaves["reference_points"][:, :, None, :, None, :] +
               leaves["sampling_offsets"] / wh[None, None, None, :, None, :])
        a = torch.softmax(leaves["attn_logits"], dim=-1).view(B, Nq, M, L, K)
        o = msda.ms_deform_attn(leaves["value"], x["spatial_shapes"], x["level_start_index"],
                                loc, a)
        o.backward(g)

    for name, fn in (("autograd_step_fused_us", fused_step),
                     ("autograd_step_torch_prologue_us", unfused_step)):
        for _ in range(3):
            fn()
        res[name] = time_warm(torch, fn, reps)
    log(f"fused: {json.dumps(res)}")
    return res


def measure_volume(torch, msda, reps, flush):
    """The 3-D trilinear variant on the voxel workload (workloads.make_volume):
    forward cold/warm and backward warm, with algorithmic bytes."""
    import workloads
    w = workloads.make_volume()
    d = torch.device("cuda")
    t = lambda a: torch.from_numpy(a).to(d)
    x = dict(value=t(w.value), volume_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
             attn_weight=t(w.attn_weight))
    g = t(w.grad_out)
    dims = w.dims
    B, Nv, Nq, M, D, L, K = (dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    pts = w.points
    val, loc, attn, rows = B * Nv * M * D * 4, pts * 12, pts * 4, B * Nq * M * D * 4
    fwd_bytes = val + loc + attn + rows
    # backward: value, loc, attn, grad_out read; grad_loc, grad_attn written;
    # grad_value zero-filled and then written once per voxel
    bwd_bytes = val + loc + attn + rows + loc + attn + 2 * val
    out = torch.empty(B, Nq, M * D, device=d)
    fwd = lambda: msda.forward3d(**x, out=out, validate=False)
    for _ in range(3):
        fwd()
    gv = torch.empty(tuple(w.value.shape), dtype=torch.float32, device=d)
    bwd = lambda: msda.backward3d(**x, grad_out=g, grad_value=gv, validate=False)
    for _ in range(3):
        bwd()
    cold = time_forward(torch, fwd, reps, flush)
    warm = time_warm(torch, fwd, reps)
    bw = time_warm(torch, bwd, reps)
    res = {"points": pts, "workload": "voxel pyramid 4x128x128, 2x64x64, 1x32x32; Nq=16384, "
                                      "M=8, D=32, K=4, fp32",
           "forward": {"us_cold": cold, "us_warm": warm, "algorithmic_bytes": fwd_bytes,
                       "algorithmic_GBps": fwd_bytes / cold / 1e3},
           "backward": {"us_warm": bw, "algorithmic_bytes": bwd_bytes,
                        "algorithmic_GBps": bwd_bytes / bw / 1e3}}
    log(f"volume: {json.dumps(res)}")
    return res


MFMA_FP32_PEAK_TFLOPS = 157.3


def measure_dat(torch, msda, reps, flush):
    """DAT's sampled-key attention at both DAT configurations, without the
    optional bias: the sampling step (core with one level and point) forward
    and backward, and the MFMA attention forward and backward, with the
    attention's algorithmic flops (2 per multiply-add: QK^T and PV forward;
    S, dP recomputed twice, dQ, dK, dV backward) against the fp32 MFMA peak."""
    import workloads
    res = {}
    for name in ("dat_cls", "dat_det"):
        w = workloads.make_dat(name)
        dims = w.dims
        B, N, Ns, Hh, d = (dims[k] for k in ("B", "N", "Ns", "Hh", "d"))
        t = lambda a: torch.from_numpy(a).cuda()
        x, pos, gs = t(w.x), t(w.pos), t(w.grad_sampled)
        q, k, v, g = t(w.q), t(w.k), t(w.v), t(w.grad_out)
        smp = lambda: msda.dat_sample(x, w.hw, pos, validate=False)
        smp_b = lambda: msda.dat_sample_backward(x, w.hw, pos, gs, validate=False)
        out, lse = msda.dat_attention(q, k, v)
        att = lambda: msda.dat_attention(q, k, v)
        att_b = lambda: msda.dat_attention_backward(q, k, v, out, lse, g)
        for fn in (smp, smp_b, att, att_b):
            for _ in range(3):
                fn()
        mm = 2.0 * B * Hh * N * Ns * d            # flops of one N x Ns x d product
        r = {"B": B, "N": N, "Ns": Ns, "heads": Hh, "head_dim": d, "groups": dims["G"],
             "sample_fwd_us": time_warm(torch, smp, reps),
             "sample_bwd_us": time_warm(torch, smp_b, reps),
             "attn_fwd_us": time_forward(torch, att, reps, flush),
             "attn_bwd_us": time_warm(torch, att_b, reps)}
        # where the sampling backward's time goes (the core's stage events)
        ss, st = msda._binding._level_of(w.hw, x.device)
        ones = msda._binding._ones_of((B, Ns, dims["G"], 1, 1), x.device)
        loc = pos.reshape(B, Ns, dims["G"], 1, 1, 2)
        ev = msda.make_events()
        msda.backward(x, ss, st, loc, ones, gs, validate=False, align_corners=True, events=ev)
        torch.cuda.synchronize()
        r["sample_bwd_stages_us"] = dict(zip(msda.BWD_STAGES, msda.stage_times(ev)))
        r["attn_fwd_tflops"] = 2 * mm / r["attn_fwd_us"] / 1e6
        r["attn_bwd_tflops"] = 7 * mm / r["attn_bwd_us"] / 1e6
        r["attn_fwd_frac_of_fp32_mfma_peak"] = r["attn_fwd_tflops"] / MFMA_FP32_PEAK_TFLOPS
        res[name] = r
    log(f"dat: {json.dumps(res)}")
    return res


def cpu_info() -> dict:
    """The host the oracle runs on: model name, logical CPUs, the CPUs this
    process may use, and OMP_NUM_THREADS as set."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def _time_oracle(w, threads, min_seconds, max_runs):
    import oracle
    args = (w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc, w.attn_weight)
    times = []
    t_start = time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_start < min_seconds and len(times) < max_runs):
        t0 = time.perf_counter()
        oracle.forward(*args, threads=threads)
        oracle.backward(*args, w.grad_out, threads=threads)
        times.append(time.perf_counter() - t0)
    return statistics.median(times), len(times)


def cpu_baseline(w, min_seconds=10.0):
    """The oracle (fp64 accumulation, OpenMP over independent outputs) on the
    whole encoder workload, forward + backward: on every core this process
    may use, then on one core."""
    import oracle
    pts = w.points
    med, n = _time_oracle(w, 0, min_seconds, 10)
    cores = oracle.max_threads()
    med1, n1 = _time_oracle(w, 1, 0.0, 2)
    return {"value": pts / med, "unit": "points/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole encoder workload ({pts} points), forward + backward, "
                      f"{n} runs, median {med:.2f} s per step, fp64 accumulation",
            "single_core": {"value": pts / med1, "unit": "points/s", "cores": 1,
                            "sample": f"the same, {n1} runs on one thread, median "
                                      f"{med1:.2f} s per step"},
            **cpu_info()}


# ---------------------------------------------------------------------------
# ceilings: the row-gather rate and a streaming copy (libmsda_probe.so)
# ---------------------------------------------------------------------------
PROBE_GRID = 2048      # workgroups of 256 lanes per probe launch
PROBE_ITERS = 256      # rows per lane group per launch


def probe_lib():
    import ctypes
    import scale_deformable_attention_04_amd.build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    p, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
    lib.msda_probe_row_gather.argtypes = [p, u32, u32, u32, u32, u32, u32, p, p]
    lib.msda_probe_row_gather.restype = ctypes.c_int
    lib.msda_probe_copy.argtypes = [p, p, u64, p]
    lib.msda_probe_copy.restype = ctypes.c_int
    return lib


def _time_launches(torch, launch, reps):
    s = torch.cuda.current_stream()
    for _ in range(2):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        launch()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps  # us per launch


def gather_ceiling(torch, reps=10):
    """Rows per second the chip gathers with the sampling kernels' access
    pattern (lane groups reading whole pseudo-random rows, 16 or 8 bytes per
    lane, four rows in flight), from buffers resident in L1 (16 KiB), in one
    XCD's L2 (2 MiB), in the Infinity Cache (64 MiB) and beyond it (1 GiB)."""
    import ctypes
    lib = probe_lib()
    dev = torch.device("cuda")
    sink = torch.empty(PROBE_GRID * 256, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {"method": f"{PROBE_GRID} workgroups x 256 lanes, {PROBE_ITERS} rows per lane group "
                     "per launch, 4 rows in flight, buffer-load instructions as in the kernels"}
    cases = (("rows_128B_16B_lanes", 128, 16, ("16KiB", "2MiB", "64MiB", "1GiB")),
             ("rows_64B_8B_lanes", 64, 8, ("2MiB",)))
    size = {"16KiB": 16 << 10, "2MiB": 2 << 20, "64MiB": 64 << 20, "1GiB": 1 << 30}
    for name, row_bytes, lane_bytes, bufs in cases:
        res = {}
        for b in bufs:
            buf = torch.randint(0, 1 << 30, (size[b] // 4,), dtype=torch.int32, device=dev)
            rows = size[b] // row_bytes
            groups = PROBE_GRID * 256 // (row_bytes // lane_bytes)

            def launch():
                rc = lib.msda_probe_row_gather(ctypes.c_void_p(buf.data_ptr()), rows, row_bytes,
                                               lane_bytes, PROBE_ITERS, PROBE_GRID, 12345,
                                               ctypes.c_void_p(sink.data_ptr()), stream)
                if rc != 0:
                    raise RuntimeError(f"msda_probe_row_gather: hipError_t {rc}")
            us = _time_launches(torch, launch, reps)
            rate = groups * PROBE_ITERS / us * 1e6
            res[b] = {"rows_per_s": rate, "bytes_per_s": rate * row_bytes, "us_per_launch": us}
            del buf
        out[name] = res
    log(f"gather ceiling: {json.dumps(out)}")
    return out


def stream_copy(torch, nbytes=1 << 30, reps=10):
    """A streaming copy of nbytes with 16-byte loads and stores: bytes read +
    written per second, the achievable counterpart of the 8 TB/s peak."""
    import ctypes
    lib = probe_lib()
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.msda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 nbytes, stream)
        if rc != 0:
            raise RuntimeError(f"msda_probe_copy: hipError_t {rc}")
    us = _time_launches(torch, launch, reps)
    res = {"bytes_per_copy": 2 * nbytes, "us": us, "GBps": 2 * nbytes / us / 1e3,
           "frac_of_peak": 2 * nbytes / us / 1e3 / HBM_PEAK_GBS}
    log(f"stream copy: {json.dumps(res)}")
    return res


def forward_roofline(enc_fwd, pts, ceiling):
    """The forward against the HBM roofline (cold and warm) and against the
    L2-resident row-gather ceiling: it must gather 4 rows per point."""
    rows = 4 * pts
    rate = ceiling["rows_128B_16B_lanes"]["2MiB"]["rows_per_s"]
    ceil_us = rows / rate * 1e6
    b = enc_fwd["algorithmic_bytes"]
    cold, warm = enc_fwd["us_cold"], enc_fwd["us_warm"]
    return {"kernel": KERNELS["forward"], "algorithmic_bytes": b, "us_cold": cold,
            "us_warm": warm, "hbm_frac_cold": b / cold / 1e3 / HBM_PEAK_GBS,
            "hbm_frac_warm": b / warm / 1e3 / HBM_PEAK_GBS, "rows_gathered": rows,
            "rows_per_s_warm": rows / warm * 1e6, "gather_ceiling_rows_per_s": rate,
            "gather_ceiling_us": ceil_us, "frac_of_gather_ceiling_warm": ceil_us / warm,
            "frac_of_gather_ceiling_cold": ceil_us / cold,
            "hbm_frac_at_gather_ceiling": b / ceil_us / 1e3 / HBM_PEAK_GBS}


def _profile_for(path, kernel_name):
    """The entry of a profiles/ summary for this kernel, when it was taken on
    the current 2-D kernel sources."""
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_sha(ENCODER_SOURCES):
        return None
    return t.get("kernels", {}).get(kernel_name)


def traffic_for(kernel_name: str):
    """HBM bytes per launch measured by rocprofv3 for this kernel on this source."""
    k = _profile_for(TRAFFIC_FILE, kernel_name)
    return int(k["fetch_bytes"] + k["write_bytes"]) if k else None


def counters_for(kernel_name: str):
    """L2 hit rate and atomic requests per launch (rocprofv3) for this kernel."""
    return _profile_for(COUNTERS_FILE, kernel_name)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=30, help="launches per kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true",
                    help="also measure the fused prologue, the 3-D variant and DAT")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the sampling core shards over (batch, head) with no communication, "
              "so a multi-GPU figure is not produced here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import scale_deformable_attention_04_amd as msda
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msda.load()
    log(f"device {torch.cuda.get_device_name(0)}")

    w = workloads.make(3)   # encoder shapes with grad_out
    dims = w.dims
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    enc, x, g, bm = measure_config(torch, msda, w, False, args.reps, flush, "encoder")

    # ---- timed region: K whole steps (fwd + bwd) -------------------------------------
    out = torch.empty(dims["B"], dims["Nq"], dims["M"] * dims["D"], device="cuda")
    gv = torch.empty(x["value"].shape, dtype=torch.float32, device="cuda")
    gl = torch.empty_like(x["sampling_loc"])
    ga = torch.empty_like(x["attn_weight"])

    # The dominant kernel is the one with the largest warm duration in the
    # breakdown above; in the timed region only it is bracketed by events
    # (each event record costs the stream a few microseconds).
    warm = {"forward": enc["forward"]["us_warm"], **enc["backward"]["stages_us_warm"]}
    dom = max((k for k in warm if k in bm), key=lambda k: warm[k])
    ev_sets = []
    for _ in range(args.steps):
        if dom == "forward":
            ev_sets.append((torch.cuda.Event(enable_timing=True),
                            torch.cuda.Event(enable_timing=True)))
        else:
            ev_sets.append(msda.make_events(dom))

    def step(i=None):
        cur = torch.cuda.current_stream()
        fe = ev_sets[i] if (i is not None and dom == "forward") else None
        be = ev_sets[i] if (i is not None and dom != "forward") else None
        if fe:
            fe[0].record(cur)
        msda.forward(**x, out=out, validate=False)
        if fe:
            fe[1].record(cur)
        msda.backward(**x, grad_out=g, grad_value=gv, grad_sampling_loc=gl,
                      grad_attn_weight=ga, validate=False, events=be)

    for _ in range(args.warmup):
        step()
    for ev in ev_sets:  # create the events before the timed region
        for e in ev:
            if e is not None:
                e.record()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for i in range(args.steps):
        step(i)
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    log(f"timed {args.steps} steps: {step_s * 1e6:.1f} us/step (events), wall {wall:.3f} s")

    # average duration of the dominant kernel inside the timed region
    if dom == "forward":
        us = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev_sets)
    else:
        k = msda.BWD_STAGES.index(dom)
        us = statistics.mean(msda.stage_times(ev)[k] for ev in ev_sets)
    log(f"dominant kernel {KERNELS[dom]}: {us:.2f} us per launch in the timed region")
    achieved = bm[dom] / us / 1e3
    # the ceilings: row-gather rate and a streaming copy
    ceiling = gather_ceiling(torch)
    copy = stream_copy(torch)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(KERNELS[dom]), "kernel": KERNELS[dom],
                "algorithmic_bytes_per_launch": bm[dom], "avg_launch_us": round(us, 2),
                "counters": counters_for(KERNELS[dom]),
                "achievable_copy_GBps": round(copy["GBps"], 1),
                "forward": forward_roofline(enc["forward"], bm["points"], ceiling)}
    roofline["forward"]["counters"] = counters_for(KERNELS["forward"])
    # the same kernel with nothing beside it: the backward on one stream (in
    # the step the grad_attn/grad_loc kernel shares the chip with the grad_value
    # kernels, and its duration there depends on how the two share it)
    if dom == "forward":
        us_alone = us
    else:
        sets = [msda.make_events(dom) for _ in range(20)]
        for ev in sets:
            msda.backward(**x, grad_out=g, grad_value=gv, grad_sampling_loc=gl,
                          grad_attn_weight=ga, validate=False, events=ev, side_stream=None)
        torch.cuda.synchronize()
        us_alone = statistics.mean(msda.stage_times(ev)[k] for ev in sets)
    roofline["alone"] = {"avg_launch_us": round(us_alone, 2),
                         "achieved": round(bm[dom] / us_alone / 1e3, 1),
                         "frac": round(bm[dom] / us_alone / 1e3 / HBM_PEAK_GBS, 4)}

    # the other two configurations: the decoder and the bf16 training shape
    dec_w = workloads.make(2)
    dec, _, _, _ = measure_config(torch, msda, dec_w, False, args.reps, flush, "decoder")
    trn_w = workloads.make(4)
    trn, _, _, _ = measure_config(torch, msda, trn_w, True, max(5, args.reps // 3), flush,
                                  "train_bf16")
    inputs_sha = {"encoder": w.sha256(), "decoder": dec_w.sha256(), "train_bf16": trn_w.sha256()}
    del trn_w

    extra = {}
    if args.extra:
        extra["encoder_bounded_workspace"] = measure_bounded(torch, msda, x, g, dims,
                                                             max(5, args.reps // 3))
        extra["fused_encoder"] = measure_fused(torch, msda, args.reps, flush)
        extra["volume"] = measure_volume(torch, msda, args.reps, flush)
        extra["dat"] = measure_dat(torch, msda, args.reps, flush)

    result = {
        "metric": "sampled points/s (fwd+bwd) at the DETR encoder shape",
        "value": bm["points"] / step_s,
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "deformable-detr encoder self-attention sampling core, fwd+bwd",
                   "B": dims["B"], "levels_hw": [list(map(int, r)) for r in w.spatial_shapes],
                   "Nv": dims["Nv"], "Nq": dims["Nq"], "M": dims["M"], "D": dims["D"],
                   "L": dims["L"], "K": dims["K"], "value_dtype": "fp32",
                   "points_per_step": bm["points"]},
        "roofline": roofline,
        "encoder": enc,
        "decoder": dict(dec, config="B=2, Nq=300 object queries over the encoder's 4-level "
                                    "value, M=8, D=32, K=4, fp32"),
        "train_bf16": dict(trn, config="B=4, Nq=Nv=22223, M=8, D=32, L=4, K=8, bf16 value, "
                                       "fp32 locations, weights, accumulation and gradients"),
        "gather_ceiling": ceiling,
        "stream_copy": copy,
        "inputs_sha256": inputs_sha,
        "kernel_source_sha": source_sha(),
        **extra,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(w)
        # the GPU step rate over the oracle's, on all cores and on one
        cpu["gpu_over_oracle"] = result["value"] / cpu["value"]
        if "single_core" in cpu:
            cpu["single_core"]["gpu_over_oracle"] = result["value"] / cpu["single_core"]["value"]
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
