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
def traffic_file(workload: str) -> str:
    """The committed counter summary of k_run on one workload."""
    return os.path.join(ROOT, "profiles", f"k_run_{workload}_traffic.json")
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
        with open(traffic_file(workload)) as f:
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


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, command, workload, mode):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, in KiB per
    dispatch, of k_run and of a plain copy of copy_mib MiB) into HBM bytes per
    k_run launch on `workload` in `mode`, each counter scaled by what it reads
    for the copy."""
    mean = lambda v: sum(v) / len(v)
    nbytes = copy_mib * (1 << 20)
    kf = mean(_counter_rows(fetch_dir, r"k_run"))
    kw = mean(_counter_rows(write_dir, r"k_run"))
    cf = mean(_counter_rows(copy_fetch_dir, r"neg"))
    cw = mean(_counter_rows(copy_write_dir, r"neg"))
    f_scale = nbytes / (cf * 1024.0)
    w_scale = nbytes / (cw * 1024.0)
    out = {"kernel": "k_run", "workload": workload, "mode": mode,
           "kernel_source_sha": kernel_source_sha(),
           "fetch_kib_per_launch": kf, "write_kib_per_launch": kw,
           "copy_bytes": nbytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": round(kf * 1024.0 * f_scale),
           "hbm_write_bytes_per_launch": round(kw * 1024.0 * w_scale),
           "command": command}
    out["hbm_bytes_per_launch"] = out["hbm_read_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def run_mode(closed: bool, prompt: int) -> str:
    return (f"prompt of {prompt}, then closed-loop tanh" if prompt else
            "closed-loop tanh" if closed else "open loop")


def cpu_points(w, h, x, n: int, seed: int = 5):
    """The oracle on n sampled (b, c, t) outputs of an open-loop run (each
    costs t + 1 multiply-adds), single-threaded: the check the parity tests
    make at full size."""
    import numpy as np

    import oracle
    r = np.random.default_rng(seed)
    bs = r.integers(0, w.B, n)
    cs = r.integers(0, w.D, n)
    ts = r.integers(0, w.L, n)
    orc = oracle.Oracle(threads=1)
    t0 = time.perf_counter()
    for b, c, t in zip(bs, cs, ts):
        orc.conv_points(np.ascontiguousarray(h[:, c]), np.ascontiguousarray(x[b, :, c]), [int(t)])
    dt = time.perf_counter() - t0
    return {"pairs": n, "seconds": round(dt, 3), "us_per_pair": round(dt / n * 1e6, 1), "threads": 1,
            "sample": f"{n} uniform (b, c, t) outputs, seed {seed}, fp64, one thread (each pays its "
                      f"channel's column copies, L = {w.L})"}


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


def host_cpu():
    """(threads the oracle may use, CPUs this process may run on, CPU model)."""
    cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = cpus
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        threads = min(threads, int(env))   # the host's share for this job, where one is set
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, cpus, model


ORACLE_BUDGET_MACS = 1.4e11   # about 10-30 s of the fp64 brute force on 16 host threads


def oracle_sample(C: int, L: int, threads: int, budget: float = ORACLE_BUDGET_MACS):
    """(channels, prefix length) of the oracle's timed sample: the whole
    workload when it fits the budget, else as many channels as keep every
    thread busy (the oracle hands out channels in blocks of 16) over the
    longest power-of-two prefix that fits.  The brute force costs
    Lp (Lp + 1) / 2 multiply-adds per channel, so the time extrapolates
    exactly in channels and in L (L + 1)."""
    cost = lambda n, l: n * l * (l + 1) / 2.0
    if cost(C, L) <= budget:
        return C, L
    n_min = min(C, 16 * threads)
    if cost(n_min, L) <= budget:
        n = int(budget // cost(1, L)) // n_min * n_min
        return max(n_min, min(n, C)), L
    lp = L
    while lp > 1 and cost(n_min, lp) > budget:
        lp //= 2
    return n_min, lp


def cpu_baseline(w, h, x_in, closed: bool, prompt=None, nch: int = 0, budget: float = ORACLE_BUDGET_MACS):
    """The oracle (fp64 brute force), in the GPU run's mode, timed on a bounded
    sample of the workload (``oracle_sample``; ``nch`` forces a channel count)
    and extrapolated to the whole workload."""
    import numpy as np

    import oracle
    threads, cpus, model = host_cpu()
    orc = oracle.Oracle(threads=threads)
    n, lp = oracle_sample(w.B * w.D, w.L, threads, budget)
    if nch:
        n, lp = min(nch, w.B * w.D), w.L
    # channels (b, c) in row-major order: whole batch rows where they fit
    nb = max(1, min(w.B, n // w.D))
    nd = min(w.D, n) if n < w.D else w.D
    nsamp = nb * nd
    hs = np.ascontiguousarray(h[:lp, :nd])
    t0 = time.perf_counter()
    if prompt is not None:
        p = min(prompt.shape[1], lp)
        orc.conv_prompted(hs, np.ascontiguousarray(prompt[:nb, :p, :nd]), L=lp)
        kind = f"prompt of {prompt.shape[1]}, then closed loop"
    elif closed:
        orc.conv_closed(hs, np.ascontiguousarray(x_in[:nb, :nd]), L=lp)
        kind = "closed loop"
    else:
        orc.conv_open(hs, np.ascontiguousarray(x_in[:nb, :lp, :nd]))
        kind = "open loop"
    dt = time.perf_counter() - t0
    scale = (w.B * w.D) / nsamp * (w.L * (w.L + 1)) / (lp * (lp + 1))
    used = min(threads, -(-nd // 16) * nb)
    full_s = dt * scale
    return {"value": w.B * w.L / full_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "seconds": round(full_s, 3), "host_cpus": cpus, "threads_allowed": threads, "cpu_model": model,
            "sample": f"{nsamp} of {w.B * w.D} channels ({nb} x {nd}), positions [0, {lp}) of {w.L}, {kind}, "
                      f"fp64; {dt:.2f} s measured, scaled x{scale:.4g} (channels are independent; "
                      f"the brute force costs L(L+1)/2 per channel)"}


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
    # the method's bytes for the whole sequence (every red cell and tile, open
    # loop, at this T) over the calls' summed GPU time
    s_x = 2 if w.dtype == "bf16" else 4
    ab = algorithmic_bytes(w.B, w.D, w.L, s_x, s_x, T, False)
    gbs = ab / (us.sum() * 1e-6) / 1e9
    out = {"metric": "fi_step GPU time per token", "unit": "us", "workload": w.name,
           "B": w.B, "D": w.D, "L": w.L, "io_dtype": w.dtype, "small_tile_max": T,
           "mean_us": round(float(us.mean()), 2), "median_us": round(float(np.median(us)), 2),
           "p99_us": round(float(np.percentile(us, 99)), 2), "max_us": round(float(us.max()), 2),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 5), "algorithmic_bytes": ab,
                        "note": "launch-bound: one or two launches per position"},
           "wall_us_per_token": round(wall / w.L * 1e6, 2),
           "by_tile_side": by_u}
    print(json.dumps(out), flush=True)
    return 0


def phases(args, w, fi, torch) -> int:
    """The phase-timing build (libfi_prof.so): one pass after the warm-ups,
    then the per-team cycle sums of the chain wavefront's phases (chain
    segments, the rest of its block work, the barrier after the chain, the
    block-boundary tiles by side, the stores), and the cumulative time at the
    start of every block of the first channel (the per-token response of the
    pages' Figure 2c, at the granularity of a block of 256 positions)."""
    import numpy as np

    import workloads
    closed = (args.mode or w.modes[0]) == "closed"
    stream = torch.cuda.current_stream()
    io = fi.FI_BF16 if w.dtype == "bf16" else fi.FI_F32

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(workloads.to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    hd = dev(workloads.make_filter(w))
    xin = dev(workloads.make_x0(w) if closed else workloads.make_x(w))
    y = torch.empty((w.B, w.L, w.D), dtype=torch.float32, device="cuda")
    m = fi.Mixer(w.B, w.D, w.L, hd, io, args.small_tile_max, stream)
    fb = fi.FI_FEEDBACK_TANH if closed else fi.FI_FEEDBACK_NONE
    for _ in range(max(1, args.warmup)):
        m.reset()
        m.run(xin, fb, y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m.reset()
    torch.cuda.synchronize()
    e0.record(stream)
    m.run(xin, fb, y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rec = np.array(fi.fi_profile_read(m.handle), dtype=np.float64)
    m.close()
    G, S, N = int(rec[0]), int(rec[1]), int(rec[2])
    teams = rec[4:4 + G * S].reshape(G, S)
    mean = teams.mean(axis=0)
    total = mean[0]
    blocks = mean[9]
    mhz = teams[:, 0].max() / (ms * 1e3)   # the slowest team spans the pass
    out = {"metric": "k_run phase breakdown (phase-timing build)", "workload": w.name,
           "mode": "closed-loop tanh" if closed else "open loop", "teams": G,
           "pass_ms": round(ms, 4), "clock_mhz_est": round(mhz, 1),
           "cycles_per_team": round(total),
           "share": {}, "chain_cycles_per_position": {}, "tile_cycles_each": {}}
    names = {1: "setup", 6: "chain_rest", 7: "barrier_after_chain", 8: "stores"}
    out["chain_rest_parts"] = {"prologue": round(mean[11] / total, 4), "epilogue": round(mean[12] / total, 4),
                               "of_which_load_wait": round(mean[13] / total, 4)}
    for k in range(4):
        names[2 + k] = f"chain_segment_{k}"
    for k, nm in names.items():
        out["share"][nm] = round(mean[k] / total, 4)
    tiles = 0.0
    for q in range(24):
        n = mean[40 + q]
        if n > 0:
            tiles += mean[16 + q]
            out["share"][f"tile_{1 << q}"] = round(mean[16 + q] / total, 4)
            out["tile_cycles_each"][str(1 << q)] = round(mean[16 + q] / n)
    out["share"]["unaccounted"] = round(1.0 - sum(mean[k] for k in names) / total - tiles / total, 4)
    if blocks > 0:
        for k in range(4):
            out["chain_cycles_per_position"][str(k)] = round(mean[2 + k] / (blocks * 64), 2)
    # where the teams' wavefronts ran (XCC id << 32 | HW_ID: SIMD in bits
    # 4-5, CU in 8-11, shader array 12, shader engine 13-15)
    from collections import Counter

    def where(v):
        v = int(v)
        hw = v & 0xFFFFFFFF
        return (v >> 32, (hw >> 13) & 7, (hw >> 12) & 1, (hw >> 8) & 15), (hw >> 4) & 3
    if S > 15 and teams[:, 14].any():
        wc = [where(v) for v in teams[:, 14]]
        wh = [where(v) for v in teams[:, 15]]
        chains = Counter(wc)
        waves = Counter(wc + wh)
        out["placement"] = {
            "cus": len({c for c, _ in wc + wh}),
            "teams_per_cu": dict(Counter(Counter(c for c, _ in wc).values())),
            "chain_wavefronts_per_simd_holding_one": dict(Counter(chains.values())),
            "wavefronts_per_simd": dict(Counter(waves.values())),
            "teams_with_both_wavefronts_on_one_simd": int(sum(a == b for a, b in zip(wc, wh))),
            "chain_simd_index": dict(Counter(sd for _, sd in wc)),
            "helper_simd_index": dict(Counter(sd for _, sd in wh)),
        }
        # pairs: the team whose second wavefront shares this team's chain
        # SIMD has its chain on this team's second wavefront's SIMD
        helper_at = {v: k for k, v in enumerate(wh)}
        sym = sum(1 for k in range(len(wc)) if wc[k] in helper_at and wc[helper_at[wc[k]]] == wh[k])
        out["placement"]["teams_in_symmetric_pairs"] = int(sym)
        out["placement"]["chain_simd_parity_vs_helper"] = dict(Counter(f"{a[1] % 2}{b[1] % 2}" for a, b in zip(wc, wh)))
    ser = rec[4 + G * S:4 + G * S + 8 * N].reshape(N, 8)
    if N and ser[0, 0] > 0:
        t_us = (ser[:, 0] - ser[0, 0]) / mhz
        out["cumulative_us_at_block_start"] = [round(v, 2) for v in t_us.tolist()]
        out["block"] = 256
        # the first channel's blocks, by the side of the tile at their end:
        # mean cycles of each part of the block's timeline
        parts = ("prologue", "chain", "epilogue_to_load_wait", "rest_of_epilogue", "barrier", "tile", "stores")
        by = {}
        for n in range(N):
            r = ser[n]
            i = (n + 1) * 256
            key = str(i & -i) if i < w.L else "last"
            if r[1] > 0:
                d = [r[1] - r[0], r[2] - r[1], r[3] - r[2], r[4] - r[3], r[5] - r[4], r[6] - r[5], r[7] - r[6]]
            else:   # no chain (open loop): everything before the barrier is the block's own work
                d = [0.0, r[4] - r[0], 0.0, 0.0, r[5] - r[4], r[6] - r[5], r[7] - r[6]]
            by.setdefault(key, []).append(d)
        out["first_channel_block_cycles_by_tile"] = {
            k: dict(zip(parts, [round(float(v)) for v in np.mean(np.array(v), axis=0)])) | {"blocks": len(v)}
            for k, v in by.items()}
    print(json.dumps(out), flush=True)
    return 0


def stack_bench(args, fi, torch) -> int:
    """The layer stack (fi_stack_run): M mixers with MLP + GELU blocks and the
    sampler feeding noise back, one position per step over the whole
    sequence.  Reports generated tokens/s (B L per pass), the time per
    position, and the oracle's stack on a prefix of the same workload."""
    import numpy as np

    import workloads
    w = workloads.get_stack(args.stack)
    progress(f"bench: stack {w.name} B={w.B} D={w.D} L={w.L} M={w.M}")
    stream = torch.cuda.current_stream()
    rho = workloads.make_stack_filters(w)
    w1, w2 = workloads.make_stack_weights(w)
    x0 = workloads.make_stack_x0(w)
    nz = workloads.make_stack_noise(w)
    dv = [torch.from_numpy(a).cuda() for a in (rho, w1, w2, x0, nz)]
    y = torch.empty((w.B, w.L, w.D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s = fi.Stack(w.B, w.D, w.L, w.M, dv[0], dv[1], dv[2], fi.FI_ACT_GELU, args.small_tile_max, stream)
    create_ms = (time.perf_counter() - t0) * 1e3
    for k in range(args.warmup):
        s.run(dv[3], y, None, dv[4], w.sigma)
    torch.cuda.synchronize()
    progress(f"bench: stack create {create_ms:.1f} ms, {args.warmup} warm-up passes done")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        s.run(dv[3], y, None, dv[4], w.sigma)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    per = [a.elapsed_time(b) for a, b in evs]
    ms = sum(per) / len(per)
    assert torch.isfinite(y).all().item(), "non-finite output"
    s.close()
    progress(f"bench: stack {args.steps} timed passes, {ms:.3f} ms/pass")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the oracle's stack is O(M D t) per position t: time a prefix of
        # about 10-30 s and report its positions per second
        P = min(w.L, 1024)
        orc = oracle.default()
        t1 = time.perf_counter()
        orc.conv_stack(rho[:, :P], w1, w2, x0, noise=nz[:, :P], sigma=np.float32(w.sigma), act="gelu")
        sec = time.perf_counter() - t1
        _, cpus, model = host_cpu()
        cpu = {"value": round(w.B * P / sec, 2), "unit": "tokens/s", "cores": min(w.B, orc.threads),
               "kind": "oracle", "host_cpus": cpus, "cpu_model": model,
               "sample": f"the first {P} of {w.L} positions, all {w.B} batch rows and {w.M} layers, "
                         f"{sec:.1f} s (one thread per batch row; later positions cost more, "
                         f"so the full sequence runs slower than this rate)"}
        progress(f"bench: oracle {cpu['sample']}")
    out = {"metric": "stack tokens/sec (B·L/s), M mixers + MLP/GELU blocks + sampler", "value":
           round(w.B * w.L / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "D": w.D, "L": w.L, "M": w.M, "act": "gelu",
                      "sigma": w.sigma, "us_per_position": round(ms * 1e3 / w.L, 2),
                      "host_wall_ms_per_pass": round(wall * 1e3, 2), "create_ms": round(create_ms, 1)},
           "cpu_baseline": cpu}
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
    ap.add_argument("--mode", choices=("open", "closed"), default=None,
                    help="open or closed loop (default: the workload's first mode)")
    ap.add_argument("--cpu-channels", type=int, default=0,
                    help="time the oracle on this many channels at all positions (default: a sample "
                         "sized to about 10-30 s, see oracle_sample)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-points", type=int, default=0, metavar="N",
                    help="also time the oracle on N sampled outputs (open loop)")
    ap.add_argument("--per-token", action="store_true",
                    help="time the online interface fi_step one position per call instead")
    ap.add_argument("--prompt", type=int, default=0, metavar="P",
                    help="generation from a prompt: the workload's first P open-loop inputs are "
                         "given (fi_run_prompted), later ones fed back")
    ap.add_argument("--phases", action="store_true",
                    help="phase breakdown of one pass from the phase-timing build "
                         "(python exact_online_amd/build.py --profile)")
    ap.add_argument("--stack", default="", metavar="NAME",
                    help="time the layer stack workload NAME (e.g. stack-m18-d256-l32k) instead")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=5,
                    metavar=("K_FETCH", "K_WRITE", "COPY_FETCH", "COPY_WRITE", "COPY_MIB"),
                    help="host only: rocprofv3 --pmc output dirs -> the traffic summary")
    ap.add_argument("--traffic-command", default="", help="recorded with --write-traffic")
    args = ap.parse_args()
    if args.write_traffic:
        import workloads
        a = args.write_traffic
        w = workloads.get(args.workload)
        closed = (args.mode or w.modes[0]) == "closed"
        return write_traffic(a[0], a[1], a[2], a[3], int(a[4]), args.traffic_command, w.name,
                             run_mode(closed, args.prompt))
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the path shards "
              "over channels with no per-step communication, so a multi-GPU figure is not produced here.",
              file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe)

    if args.phases:
        prof = os.path.join(ROOT, "exact_online_amd", "libfi_prof.so")
        if not os.path.exists(prof):
            print("--phases needs the phase-timing build: python exact_online_amd/build.py --profile",
                  file=sys.stderr)
            return 2
        os.environ["EXACT_ONLINE_AMD_LIB"] = prof
    import numpy as np
    import torch

    import exact_online_amd as fi
    import workloads

    if args.stack:
        torch.cuda.set_device(0)
        return stack_bench(args, fi, torch)
    w = workloads.get(args.workload)
    if args.phases:
        torch.cuda.set_device(0)
        return phases(args, w, fi, torch)
    if args.per_token:
        torch.cuda.set_device(0)
        return per_token(args, w, fi, torch)
    T = args.small_tile_max or fi.FI_DEFAULT_SMALL_TILE_MAX
    mode_name = args.mode or w.modes[0]
    if mode_name not in ("open", "closed"):
        print(f"--mode must be open or closed", file=sys.stderr)
        return 2
    closed = mode_name == "closed"
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
        xh = x0 if closed else workloads.make_x(w)
        xin = dev(xh)
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
    mode = run_mode(closed, P)
    achieved = ab / (kern_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(sha, w.name, mode),
                "kernel": "k_run", "algorithmic_bytes": ab, "kernel_ms": round(kern_ms, 4),
                "kernel_source_sha": sha}
    m.close()
    cpu = None
    if not args.no_cpu_baseline:
        progress("bench: timing the CPU oracle on a sample of the workload")
        cpu = cpu_baseline(w, h, None if P else xh, closed, prompt, args.cpu_channels)
        progress(f"bench: oracle {cpu['sample']}")
        if args.cpu_points and not closed and not P:
            cpu["points"] = cpu_points(w, h, xh, args.cpu_points)
            progress(f"bench: oracle on sampled outputs {cpu['points']}")
    value = w.B * w.L / (ms_step * 1e-3)
    out = {
        "metric": METRIC if w.name == "hyena-d1024-l16k" else "mixer tokens/sec (B·L/s); % HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "D": w.D, "L": w.L, "io_dtype": w.dtype,
                   "acc_dtype": "f32", "mode": mode, "small_tile_max": T,
                   "create_ms": round(create_ms, 1)},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
