#!/usr/bin/env python
"""Benchmark: mixer tokens/s of the exact online causal long convolution.

One step = one full pass of the hot path over one batch: fi_run_closed_loop
on the Hyena-like mixer workload (B=1, D=1024, L=16384, fp32, closed-loop tanh
feedback, decaying-Gaussian filters with log-uniform tau in [64, 8192]) with
the inputs already resident in HBM.  Protocol of the pages: warm-ups, then
the mean over timed runs (here 20 and 20 by default).  Prints ONE JSON line.

Also reported:
  roofline      the persistent kernel (k_run, the only kernel of a step):
                algorithmic bytes of the method (per-tile x block read, accumulator
                read+write, filter taps or spectrum, per-step reads/writes) divided
                by its mean duration from HIP events on its stream, against
                MI355X's 8 TB/s HBM peak; ``traffic`` comes from the committed
                rocprofv3 counter summary when it was taken on the current kernel
                source, else null.
  cpu_baseline  the CPU oracle (fp64 brute force) timed on a channel subset of
                the same workload, scaled to the whole workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mixer tokens/sec (B·L/s) at D=1024, L=16K; % HBM roofline"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_run_hyena-d1024-l16k_traffic.json")
KERNEL_SOURCES = ["exact_online_amd/csrc/fi_kernels.hip", "exact_online_amd/csrc/fi_device.hpp",
                  "exact_online_amd/csrc/fi_internal.h"]


def progress(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(B, D, L, s_x, s_h, T, closed, fed=None) -> int:
    """Bytes the method moves: every tile of side U reads its x block (U s_x)
    and reads+writes U accumulators (2U*4) per channel, plus the filter data
    per filter channel (taps h[1..2U) for direct tiles, the (U+1)-point complex
    spectrum for FFT tiles); every step reads the accumulator and x, writes y,
    and writes x where it is fed back (``fed`` positions: all of them in
    closed loop, none in open loop, those after the prompt in a prompted run)."""
    P = (L - 1).bit_length()
    tot = 0
    for q in range(P):
        U = 1 << q
        n = L // (2 * U)
        Fq = (2 * U - 1) * s_h if U <= T else (U + 1) * 8
        tot += n * (B * D * (U * s_x + 2 * U * 4) + D * Fq)
    if fed is None:
        fed = L if closed else 0
    tot += B * D * L * (4 + s_x + 4) + B * D * fed * s_x
    return tot


def load_traffic(sha: str, workload: str, mode: str):
    """The committed counter summary's HBM bytes per launch, when it was taken
    on this kernel source, workload and mode; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != sha or t.get("workload") != workload or t.get("mode", mode) != mode:
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_rows(path: str, kernel_regex: str):
    """Per-dispatch counter values (summed over counters named in the file) of
    the kernels whose name matches kernel_regex, from a rocprofv3 --pmc csv
    output directory (or one *counter_collection.csv file)."""
    import csv
    import glob
    import re
    files = [path] if path.endswith(".csv") else \
        sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    per = {}
    pat = re.compile(kernel_regex)
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if pat.search(r["Kernel_Name"]):
                    key = (fn, r.get("Dispatch_Id") or r.get("Correlation_Id"))
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {kernel_regex!r} in {path}")
    return list(per.values())


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, command):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, in KiB per
    dispatch, of k_run and of a plain copy of copy_mib MiB) into HBM bytes per
    k_run launch, each counter scaled by what it reads for the copy."""
    mean = lambda v: sum(v) / len(v)
    nbytes = copy_mib * (1 << 20)
    kf = mean(_counter_rows(fetch_dir, r"k_run"))
    kw = mean(_counter_rows(write_dir, r"k_run"))
    cf = mean(_counter_rows(copy_fetch_dir, r"neg"))
    cw = mean(_counter_rows(copy_write_dir, r"neg"))
    f_scale = nbytes / (cf * 1024.0)
    w_scale = nbytes / (cw * 1024.0)
    out = {"kernel": "k_run", "workload": "hyena-d1024-l16k", "mode": "closed-loop tanh",
           "kernel_source_sha": kernel_source_sha(),
           "fetch_kib_per_launch": kf, "write_kib_per_launch": kw,
           "copy_bytes": nbytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": round(kf * 1024.0 * f_scale),
           "hbm_write_bytes_per_launch": round(kw * 1024.0 * w_scale),
           "command": command}
    out["hbm_bytes_per_launch"] = out["hbm_read_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def copy_probe(mib: int, reps: int = 5) -> int:
    """A plain elementwise copy (y = -x) of mib MiB: the known-size kernel the
    counter runs are calibrated against."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "reps": reps}), flush=True)
    return 0


def cpu_baseline(w, h, x0, nch: int, prompt=None):
    import oracle
    orc = oracle.default()
    nch = min(nch, w.D)
    t0 = time.perf_counter()
    if prompt is None:
        orc.conv_closed(h[:, :nch], x0[:, :nch])
        kind = "closed loop"
    else:
        orc.conv_prompted(h[:, :nch], prompt[:, :, :nch])
        kind = f"prompt of {prompt.shape[1]}, then closed loop"
    dt = time.perf_counter() - t0
    scale = (w.B * w.D) / (x0.shape[0] * nch)
    return {"value": w.B * w.L / (dt * scale), "unit": "tokens/s", "cores": orc.threads,
            "kind": "oracle",
            "sample": f"{nch} of {w.D} channels, all {w.L} positions, {kind}, fp64; "
                      f"{dt:.2f} s measured, scaled x{scale:g} (channels are independent)"}


def per_token(args, w, fi, torch) -> int:
    """The online interface one position per call: fi_step (the red cell and
    read-out, then the tile that position completes) on the workload's
    open-loop inputs.  Reports the GPU time of every call (events on the
    stream around it) and the host wall time per call."""
    import numpy as np

    import workloads
    T = args.small_tile_max or fi.FI_DEFAULT_SMALL_TILE_MAX
    stream = torch.cuda.current_stream()
    io = fi.FI_BF16 if w.dtype == "bf16" else fi.FI_F32

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(workloads.to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    hd = dev(workloads.make_filter(w))
    xt = dev(np.ascontiguousarray(workloads.make_x(w).transpose(1, 0, 2)))   # [L][B][D]
    yt = torch.empty((w.L, w.B, w.D), dtype=torch.float32, device="cuda")
    m = fi.Mixer(w.B, w.D, w.L, hd, io, args.small_tile_max, stream)
    for _ in range(max(1, args.warmup // 10)):
        m.reset()
        for t in range(w.L):
            m.step(xt[t], yt[t])
    torch.cuda.synchronize()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(w.L)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(w.L)]
    m.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(w.L):
        e0[t].record(stream)
        m.step(xt[t], yt[t])
        e1[t].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(e0, e1)])
    m.close()
    pos = np.arange(1, w.L + 1)
    U = pos & -pos
    U[-1] = 0   # the last position completes no tile
    by_u = {}
    for u in np.unique(U):
        sel = us[U == u]
        by_u[str(int(u))] = {"count": int(sel.size), "mean_us": round(float(sel.mean()), 2)}
    out = {"metric": "fi_step GPU time per token", "unit": "us", "workload": w.name,
           "B": w.B, "D": w.D, "L": w.L, "io_dtype": w.dtype, "small_tile_max": T,
           "mean_us": round(float(us.mean()), 2), "median_us": round(float(np.median(us)), 2),
           "p99_us": round(float(np.percentile(us, 99)), 2), "max_us": round(float(us.max()), 2),
           "wall_us_per_token": round(wall / w.L * 1e6, 2),
           "by_tile_side": by_u}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the card's clock settles over the first ten or so passes of a fresh
    # process (a pass at D=1024, L=16K falls from 0.80 to 0.73 ms), so the
    # default warm-up is longer than the pages' two runs
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="hyena-d1024-l16k")
    ap.add_argument("--small-tile-max", type=int, default=0)
    ap.add_argument("--cpu-channels", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-token", action="store_true",
                    help="time the online interface fi_step one position per call instead")
    ap.add_argument("--prompt", type=int, default=0, metavar="P",
                    help="generation from a prompt: the workload's first P open-loop inputs are "
                         "given (fi_run_prompted), later ones fed back")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=5,
                    metavar=("K_FETCH", "K_WRITE", "COPY_FETCH", "COPY_WRITE", "COPY_MIB"),
                    help="host only: rocprofv3 --pmc output dirs -> the traffic summary")
    ap.add_argument("--traffic-command", default="", help="recorded with --write-traffic")
    args = ap.parse_args()
    if args.write_traffic:
        a = args.write_traffic
        return write_traffic(a[0], a[1], a[2], a[3], int(a[4]), args.traffic_command)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the path shards "
              "over channels with no per-step communication, so a multi-GPU figure is not produced here.",
              file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe)

    import numpy as np
    import torch

    import exact_online_amd as fi
    import workloads

    w = workloads.get(args.workload)
    if args.per_token:
        torch.cuda.set_device(0)
        return per_token(args, w, fi, torch)
    T = args.small_tile_max or fi.FI_DEFAULT_SMALL_TILE_MAX
    closed = "closed" in w.modes[0]
    progress(f"bench: workload {w.name} B={w.B} D={w.D} L={w.L} {w.dtype} closed={closed}")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    h = workloads.make_filter(w)
    x0 = workloads.make_x0(w)
    io = fi.FI_BF16 if w.dtype == "bf16" else fi.FI_F32

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(workloads.to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    hd = dev(h)
    P = args.prompt
    prompt = None
    if P:
        if not 1 <= P <= w.L:
            print(f"--prompt must lie in [1, {w.L}]", file=sys.stderr)
            return 2
        prompt = np.ascontiguousarray(workloads.make_x(w)[:, :P, :])
        xin = dev(prompt)
    else:
        xin = dev(x0) if closed else dev(workloads.make_x(w))
    y = torch.empty((w.B, w.L, w.D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    m = fi.Mixer(w.B, w.D, w.L, hd, io, args.small_tile_max, stream)
    create_ms = (time.perf_counter() - t0) * 1e3
    fb = fi.FI_FEEDBACK_TANH if closed else fi.FI_FEEDBACK_NONE

    def one():
        m.reset()
        if P:
            m.run_prompted(xin, P, y)
        else:
            m.run(xin, fb, y)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    progress(f"bench: create {create_ms:.1f} ms, {args.warmup} warm-up passes done")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        evs[k][0].record(stream)
        one()
        evs[k][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per = [a.elapsed_time(b) for a, b in evs]
    ms_step = total_ms / args.steps
    kern_ms = sum(per) / len(per)
    assert torch.isfinite(y).all().item(), "non-finite output"
    progress(f"bench: {args.steps} timed passes, {ms_step:.4f} ms/pass, per-pass {['%.4f' % p for p in per]}")

    s_x = 2 if w.dtype == "bf16" else 4
    fed = w.L - P if P else None
    ab = algorithmic_bytes(w.B, w.D, w.L, s_x, s_x, 128, closed, fed)
    mode = (f"prompt of {P}, then closed-loop tanh" if P else
            "closed-loop tanh" if closed else "open loop")
    achieved = ab / (kern_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(sha, w.name, mode),
                "kernel": "k_run", "algorithmic_bytes": ab, "kernel_ms": round(kern_ms, 4),
                "kernel_source_sha": sha}
    cpu = None
    if not args.no_cpu_baseline:
        progress(f"bench: timing the CPU oracle on {args.cpu_channels} channels")
        cpu = cpu_baseline(w, h, x0, args.cpu_channels, prompt)
    m.close()
    value = w.B * w.L / (ms_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "D": w.D, "L": w.L, "io_dtype": w.dtype,
                   "mode": mode, "small_tile_max": T,
                   "create_ms": round(create_ms, 1)},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
