#!/usr/bin/env python3
"""rocprofv3 driver and summarizer for the sampling-core kernels.

Modes:

  python3 profile_kernels.py run
      The workload the two counter passes are pointed at: the encoder-shape
      forward and backward (3 calls each), then an elementwise multiply that
      reads 256 MiB and writes 256 MiB, used to calibrate the FETCH_SIZE /
      WRITE_SIZE counters (bytes known / counter reading).

  python3 profile_kernels.py run-fused
      The same for the fused prologue at the encoder shape: forward storing
      the locations and weights + backward reading them (5 each), backward
      recomputing them (5), then the calibration multiply.

  python3 profile_kernels.py run-volume
      The 3-D trilinear variant on the voxel workload: forward and backward
      (5 each), then the calibration multiply.

  python3 profile_kernels.py run-dat
      DAT's sampled-key attention at its detection configuration (B=2, 4096
      tokens, 256 keys, 12 heads of 32, 6 groups): sampling forward/backward
      and attention forward/backward (5 each), then the calibration multiply.

  python3 profile_kernels.py summarize --stats DIR --fetch DIR --write DIR
      Reads the CSV output of three rocprofv3 runs (kernel trace of the bench
      command itself; --pmc FETCH_SIZE and --pmc WRITE_SIZE of `run`) and
      writes profiles/encoder_kernels.txt (per-kernel durations, one line per
      kernel and grid size: the bench also runs the decoder and bf16 shapes,
      whose launches of the same kernels have other grids) and
      profiles/traffic.json (HBM bytes per launch of each kernel, scaled by
      the multiply's calibration, tagged with the kernel source hash).

  python3 profile_kernels.py summarize-counters --hit DIR --atomic DIR
      Reads two --pmc runs of `run` (L2 hits and misses; L2 atomics, atomics
      sent beyond L2, atomic requests from the vector L1) and writes
      profiles/counters.json: per kernel and launch, the L2 hit rate and the
      atomic counts, tagged with the kernel source hash.

  python3 profile_kernels.py summarize-fused --stats DIR --fetch DIR --write DIR
      The same from the three runs of `run-fused`: profiles/fused_encoder_kernels.txt
      and profiles/fused_traffic.json.

  python3 profile_kernels.py summarize-volume --stats DIR --fetch DIR --write DIR
      The same from the three runs of `run-volume`: profiles/volume_kernels.txt and
      profiles/volume_traffic.json.

  python3 profile_kernels.py summarize-dat --stats DIR --fetch DIR --write DIR
      The same from the three runs of `run-dat`: profiles/dat_kernels.txt and
      profiles/dat_traffic.json.

The GPU commands (run from /tmp with TMPDIR=/tmp; OUT is any output directory):
  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/stats -o run -- python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- python3 profile_kernels.py run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- python3 profile_kernels.py run
  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/fstats -o run -- python3 profile_kernels.py run-fused
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/ffetch -o run -- python3 profile_kernels.py run-fused
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/fwrite -o run -- python3 profile_kernels.py run-fused
  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/vstats -o run -- python3 profile_kernels.py run-volume
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/vfetch -o run -- python3 profile_kernels.py run-volume
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/vwrite -o run -- python3 profile_kernels.py run-volume
  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/dstats -o run -- python3 profile_kernels.py run-dat
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/dfetch -o run -- python3 profile_kernels.py run-dat
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/dwrite -o run -- python3 profile_kernels.py run-dat
  rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d OUT/hit -o run -- python3 profile_kernels.py run
  rocprofv3 --pmc TCC_ATOMIC_sum TCC_EA0_ATOMIC_sum TCP_TCC_ATOMIC_WITH_RET_REQ_sum TCP_TCC_ATOMIC_WITHOUT_RET_REQ_sum --output-format csv -d OUT/atomic -o run -- python3 profile_kernels.py run
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "scale_deformable_attention_04_amd", "csrc")
# per profile family, the sources its kernels are built from (the summaries
# are tagged with their hash, so a change elsewhere leaves them valid)
FAMILY_SOURCES = {
    "encoder": ("common.h", "bins.h", "msda.hip"),
    "fused_encoder": ("common.h", "bins.h", "msda.hip"),
    "volume": ("common.h", "bins.h", "msda3d.hip"),
    "dat": ("common.h", "bins.h", "msda.hip", "dat_attn.hip"),
}
COPY_BYTES = 256 << 20


def source_sha(name: str = "encoder") -> str:
    files = [os.path.join(CSRC, f) for f in FAMILY_SOURCES[name]]
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0].strip()


def run():
    import torch
    import scale_deformable_attention_04_amd as msda
    import workloads
    w = workloads.make(3)
    d = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(d)
    x = dict(value=t(w.value), spatial_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
             attn_weight=t(w.attn_weight))
    g = t(w.grad_out)
    for _ in range(3):
        msda.forward(**x, validate=False)
        msda.backward(**x, grad_out=g, validate=False)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=d)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print("profile workload done", flush=True)


def run_fused():
    import torch
    import scale_deformable_attention_04_amd as msda
    import workloads
    w = workloads.make_fused(3)
    d = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(d)
    x = dict(value=t(w.value), spatial_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), reference_points=t(w.reference_points),
             sampling_offsets=t(w.sampling_offsets), attn_logits=t(w.attn_logits))
    g = t(w.grad_out)
    for _ in range(5):
        out, loc, attn = msda.forward_fused(**x, validate=False, save=True)
        msda.backward_fused(**x, grad_out=g, validate=False, saved=(loc, attn))
    for _ in range(5):
        msda.backward_fused(**x, grad_out=g, validate=False)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=d)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print("profile workload done", flush=True)


def run_volume():
    import torch
    import scale_deformable_attention_04_amd as msda
    import workloads
    w = workloads.make_volume()
    d = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(d)
    x = dict(value=t(w.value), volume_shapes=t(w.spatial_shapes),
             level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
             attn_weight=t(w.attn_weight))
    g = t(w.grad_out)
    for _ in range(5):
        msda.forward3d(**x, validate=False)
        msda.backward3d(**x, grad_out=g, validate=False)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=d)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print("profile workload done", flush=True)


def run_dat():
    import torch
    import scale_deformable_attention_04_amd as msda
    import workloads
    w = workloads.make_dat("dat_det")
    t = lambda a: torch.from_numpy(a).cuda()
    x, pos, gs = t(w.x), t(w.pos), t(w.grad_sampled)
    q, k, v, g = t(w.q), t(w.k), t(w.v), t(w.grad_out)
    for _ in range(5):
        msda.dat_sample(x, w.hw, pos, validate=False)
        msda.dat_sample_backward(x, w.hw, pos, gs, validate=False)
        out, lse = msda.dat_attention(q, k, v)
        msda.dat_attention_backward(q, k, v, out, lse, g)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print("profile workload done", flush=True)


def _rows(path_glob):
    rows = []
    for f in sorted(glob.glob(path_glob, recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    return rows


def _counter_means(dirpath, counter, scale=1024.0):
    """Mean per launch of a counter, by kernel (FETCH_SIZE / WRITE_SIZE read
    in KiB: scale 1024 gives bytes)."""
    per = collections.defaultdict(list)
    for r in _rows(os.path.join(dirpath, "**", "*counter_collection.csv")):
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]) * scale)
    return {k: sum(v) / len(v) for k, v in per.items()}


def _trace_stats(dirpath):
    """Per (kernel, workgroups) launch statistics from a kernel trace."""
    per = collections.defaultdict(list)
    for r in _rows(os.path.join(dirpath, "**", "*kernel_trace.csv")):
        wgs = 1
        for ax in "XYZ":  # workgroups over all three grid dimensions
            wgs *= int(r.get(f"Grid_Size_{ax}") or 1) // max(1, int(r.get(f"Workgroup_Size_{ax}") or 1))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per[(short_name(r["Kernel_Name"]), wgs)].append(dur)
    total = sum(sum(v) for v in per.values()) or 1.0
    out = [(k, len(v), sum(v) / len(v), min(v), max(v), 100.0 * sum(v) / total)
           for k, v in per.items()]
    return sorted(out, key=lambda e: -e[1] * e[2])


HEADERS = {
    "encoder": ["# rocprofv3 --kernel-trace --stats of bench.py: encoder workload (B=2, Nq=Nv=22223,",
                "# M=8, D=32, L=4, K=4, fp32), forward and backward (its grad_attn/grad_loc kernel on",
                "# a side stream, concurrent with the grad_value kernels)"],
    "fused_encoder": ["# rocprofv3 --kernel-trace --stats of profile_kernels.py run-fused: the fused",
                      "# prologue at the encoder shape (B=2, Nq=Nv=22223, M=8, D=32, L=4, K=4, fp32;",
                      "# reference points + pixel offsets + logits): 5 x (forward storing the",
                      "# locations and weights, backward reading them), 5 x backward recomputing",
                      "# them (prologue kernel), then the 256 MiB calibration multiply"],
    "volume": ["# rocprofv3 --kernel-trace --stats of profile_kernels.py run-volume: the 3-D",
               "# trilinear variant on the voxel workload (pyramid 4x128x128, 2x64x64, 1x32x32;",
               "# Nq=16384, M=8, D=32, K=4, fp32): 5 x (forward, backward with its grad_value",
               "# zero-fill), then the 256 MiB calibration multiply"],
    "dat": ["# rocprofv3 --kernel-trace --stats of profile_kernels.py run-dat: DAT's",
            "# sampled-key attention at the detection configuration (B=2, 64x64 tokens, 16x16",
            "# = 256 sampled keys, 12 heads of 32, 6 offset groups of 64 channels, fp32): 5 x",
            "# (sampling forward and backward through the core, attention forward and",
            "# backward), then the 256 MiB calibration multiply"],
}


def summarize(stats_dir, fetch_dir, write_dir, commands, name="encoder"):
    head = list(HEADERS[name])
    head[-1] += "; kernel source sha " + source_sha(name)
    lines = head + ["# command: " + commands["stats"], "",
                    f"{'kernel':46s} {'wgs':>7s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
                    f"{'max_us':>10s} {'pct':>6s}"]
    for (k, wgs), calls, avg, mn, mx, pct in _trace_stats(stats_dir):
        lines.append(f"{k[:46]:46s} {wgs:7d} {calls:6d} {avg:10.2f} {mn:10.2f} {mx:10.2f} "
                     f"{pct:6.2f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"{name}_kernels.txt"), "w").write("\n".join(lines) + "\n")

    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    copy_name = next((k for k in fetch if "MulFunctor" in k), None)
    f_scale = COPY_BYTES / fetch[copy_name] if copy_name and fetch.get(copy_name) else 1.0
    w_scale = COPY_BYTES / write[copy_name] if copy_name and write.get(copy_name) else 1.0
    out = {"source_sha": source_sha(name), "sources": list(FAMILY_SOURCES[name]),
           "calibration_kernel": copy_name,
           "calibration_bytes": COPY_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
           "commands": commands, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if k == copy_name:
            continue
        out["kernels"][k] = {"fetch_bytes": fetch.get(k, 0.0) * f_scale,
                             "write_bytes": write.get(k, 0.0) * w_scale}
    tname = "traffic.json" if name == "encoder" else f"{name.split('_')[0]}_traffic.json"
    json.dump(out, open(os.path.join(ROOT, "profiles", tname), "w"), indent=1)
    print("\n".join(lines))
    print(json.dumps(out, indent=1))


COUNTERS = {  # output key: rocprofv3 counter
    "l2_hit": "TCC_HIT_sum", "l2_miss": "TCC_MISS_sum", "l2_atomic": "TCC_ATOMIC_sum",
    "atomic_beyond_l2": "TCC_EA0_ATOMIC_sum",
    "l1_atomic_with_return": "TCP_TCC_ATOMIC_WITH_RET_REQ_sum",
    "l1_atomic_without_return": "TCP_TCC_ATOMIC_WITHOUT_RET_REQ_sum"}


def summarize_counters(hit_dir, atomic_dir, commands, name="encoder"):
    vals = {}
    for key, counter in COUNTERS.items():
        d = hit_dir if key in ("l2_hit", "l2_miss") else atomic_dir
        vals[key] = _counter_means(d, counter, scale=1.0)
    kernels = sorted(set().union(*[set(v) for v in vals.values()]))
    out = {"source_sha": source_sha(name), "sources": list(FAMILY_SOURCES[name]),
           "counters": COUNTERS, "commands": commands,
           "note": "per launch means; l2_hit_rate = l2_hit / (l2_hit + l2_miss)", "kernels": {}}
    for k in kernels:
        e = {key: vals[key].get(k) for key in COUNTERS}
        h, m = e.get("l2_hit"), e.get("l2_miss")
        e["l2_hit_rate"] = h / (h + m) if h is not None and m is not None and h + m > 0 else None
        out["kernels"][k] = e
    json.dump(out, open(os.path.join(ROOT, "profiles", "counters.json"), "w"), indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    sub.add_parser("run")
    sub.add_parser("run-fused")
    sub.add_parser("run-volume")
    sub.add_parser("run-dat")
    for mode in ("summarize", "summarize-fused", "summarize-volume", "summarize-dat"):
        s = sub.add_parser(mode)
        s.add_argument("--stats", required=True)
        s.add_argument("--fetch", required=True)
        s.add_argument("--write", required=True)
    c = sub.add_parser("summarize-counters")
    c.add_argument("--hit", required=True)
    c.add_argument("--atomic", required=True)
    a = ap.parse_args()
    if a.mode == "run":
        run()
    elif a.mode == "run-fused":
        run_fused()
    elif a.mode == "run-volume":
        run_volume()
    elif a.mode == "run-dat":
        run_dat()
    else:
        doc = __doc__.split("The GPU commands")[1].splitlines()[1:15]
        cmds = [c.strip() for c in doc]
        if a.mode == "summarize-counters":
            summarize_counters(a.hit, a.atomic, {"hit": cmds[12], "atomic": cmds[13]})
        elif a.mode == "summarize":
            summarize(a.stats, a.fetch, a.write,
                      {"stats": cmds[0], "fetch": cmds[1], "write": cmds[2]})
        elif a.mode == "summarize-fused":
            summarize(a.stats, a.fetch, a.write,
                      {"stats": cmds[3], "fetch": cmds[4], "write": cmds[5]}, "fused_encoder")
        elif a.mode == "summarize-volume":
            summarize(a.stats, a.fetch, a.write,
                      {"stats": cmds[6], "fetch": cmds[7], "write": cmds[8]}, "volume")
        else:
            summarize(a.stats, a.fetch, a.write,
                      {"stats": cmds[9], "fetch": cmds[10], "write": cmds[11]}, "dat")


if __name__ == "__main__":
    main()
