"""Test helpers: upload seeded inputs, drive the library through its C ABI,
and compare with the CPU oracle.  Test infrastructure only."""
from __future__ import annotations

import math
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import workloads


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray, dtype: str):
    """float32 numpy array (values representable in ``dtype``) -> CUDA tensor."""
    t = torch()
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(a).view(np.int16)
        return t.from_numpy(bits).cuda().view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def io_torch_dtype(dtype: str):
    t = torch()
    return t.bfloat16 if dtype == "bf16" else t.float32


def gpu_run(h_dev, B, D, L, dtype, x_in_dev, closed: bool, T: int = 0, want_x=True):
    """One fi_run_closed_loop over a fresh handle; returns (y, x_out) CUDA tensors."""
    import exact_online_amd as fi
    t = torch()
    io = fi.FI_BF16 if dtype == "bf16" else fi.FI_F32
    y = t.empty((B, L, D), dtype=t.float32, device="cuda")
    xo = t.empty((B, L, D), dtype=io_torch_dtype(dtype), device="cuda") if want_x else None
    with fi.Mixer(B, D, L, h_dev, io, T, t.cuda.current_stream()) as m:
        m.run(x_in_dev, fi.FI_FEEDBACK_TANH if closed else fi.FI_FEEDBACK_NONE, y, xo)
        t.cuda.synchronize()
        assert m.position == L
    return y, xo


def gpu_prompted(h_dev, B, D, L, dtype, prompt_dev, p: int, T: int = 0):
    """One fi_run_prompted (prompt of p given inputs, then tanh feedback) over
    a fresh handle; returns (y, x_out) CUDA tensors."""
    import exact_online_amd as fi
    t = torch()
    io = fi.FI_BF16 if dtype == "bf16" else fi.FI_F32
    y = t.empty((B, L, D), dtype=t.float32, device="cuda")
    xo = t.empty((B, L, D), dtype=io_torch_dtype(dtype), device="cuda")
    with fi.Mixer(B, D, L, h_dev, io, T, t.cuda.current_stream()) as m:
        m.run_prompted(prompt_dev, p, y, xo)
        t.cuda.synchronize()
        assert m.position == L
    return y, xo


def gpu_steps(h_dev, B, D, L, dtype, x_dev, T: int = 0):
    """Open loop through fi_step, one position per call."""
    import exact_online_amd as fi
    t = torch()
    io = fi.FI_BF16 if dtype == "bf16" else fi.FI_F32
    y = t.empty((B, L, D), dtype=t.float32, device="cuda")
    xt = t.empty((B, D), dtype=io_torch_dtype(dtype), device="cuda")
    yt = t.empty((B, D), dtype=t.float32, device="cuda")
    with fi.Mixer(B, D, L, h_dev, io, T, t.cuda.current_stream()) as m:
        if B == 1:
            # x[0, s, :] and y[0, s, :] are contiguous rows: pass them directly
            for s in range(L):
                m.step(x_dev[0, s], y[0, s])
        else:
            for s in range(L):
                xt.copy_(x_dev[:, s, :])
                m.step(xt, yt)
                y[:, s, :].copy_(yt)
        t.cuda.synchronize()
        assert m.position == L
    return y


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def host(tn) -> np.ndarray:
    t = torch()
    if tn.dtype == t.bfloat16:
        return tn.float().cpu().numpy()
    return tn.cpu().numpy()


def columns(tn, chans) -> np.ndarray:
    """[B][L][D] CUDA tensor -> host [len(chans)][L] fp64 for (b, c) pairs."""
    t = torch()
    bs = t.tensor([b for b, _ in chans], device=tn.device)
    cs = t.tensor([c for _, c in chans], device=tn.device)
    cols = tn[bs, :, cs]          # [n][L]
    return cols.float().cpu().numpy().astype(np.float64)


def oracle_points_parallel(h_cols, x_cols, ts_list, threads=None):
    """Teacher-forced oracle values, one channel per task (the oracle call
    releases the GIL)."""
    threads = threads or oracle.default_threads()
    orc = oracle.Oracle(threads=1)

    def one(k):
        return orc.conv_points(h_cols[k], x_cols[k], ts_list[k])
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(one, range(len(h_cols))))


def chaos_horizon(h, x0, L, bf16=False, eps=1e-7, tol=1e-4) -> int:
    """First position where two oracle runs, from x0 and x0*(1+eps), differ by
    more than ``tol`` (L if never): beyond it the free-running closed loop has
    no unique answer at the fp32 level and only step-wise validity is checked."""
    orc = oracle.default()
    y1, _ = orc.conv_closed(h[:L], x0, L=L, bf16=bf16)
    y2, _ = orc.conv_closed(h[:L], x0 * (1.0 + eps), L=L, bf16=bf16)
    d = np.abs(y1 - y2).max(axis=(0, 2))
    bad = np.nonzero(d > tol)[0]
    return int(bad[0]) if bad.size else L


def boundary_positions(L: int, T: int = 128, extra: int = 0, seed: int = 0) -> np.ndarray:
    """Positions around every tile boundary of the schedule: 2^k - 1, 2^k, and
    for every tile of side > T: i-1, i, i+U-1, min(i+U, L-1); plus ``extra``
    uniform ones."""
    s = {0, L - 1}
    k = 1
    while k < L:
        s.update({k - 1, k})
        k <<= 1
    U = 1
    while U < L:
        if U > T:
            for i in range(U, L, 2 * U):
                s.update({i - 1, i, min(i + U - 1, L - 1), min(i + U, L - 1)})
        U <<= 1
    if extra:
        r = np.random.default_rng(seed)
        s.update(r.integers(0, L, size=extra).tolist())
    return np.array(sorted(p for p in s if 0 <= p < L), dtype=np.int64)
