"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default small_tile_max, one fi_run_closed_loop per pass).

The oracle cannot run whole workloads of this size, so each test checks
 * sampled channels against the oracle, at every position or at sampled
   positions around every tile boundary (the oracle computes y[t] one by one);
 * properties that hold at any size on every output: in closed loop the
   recorded feedback x[t+1] equals tanh(y[t]) (fp64 tanh of the GPU's own y)
   within 1e-6 (plus half a bf16 ulp for bf16 storage), and x[0] is the given
   start.
Tolerances (fp32 arithmetic): open loop relative L2 error <= 1e-5 over the
checked entries; closed loop max abs error <= 1e-3, teacher-forced (the
oracle fed the GPU's recorded inputs).  The free-running closed loop is
compared where it is well posed: on the prefix before the chaos horizon
(two oracle runs from x0 and x0 (1 + 1e-7) agree to 1e-4).
"""
import numpy as np
import pytest

import oracle
import workloads
from fi_harness import (boundary_positions, chaos_horizon, columns, gpu_prompted, gpu_run, log,
                        oracle_points_parallel, rel_l2, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import exact_online_amd as fi  # noqa: E402  (fails loudly if libfi.so is missing)

NSAMP = 16


def sample_channels(w, n, seed=11):
    """(b, c) pairs: the corners and the first/last channel of every row, then
    uniform ones."""
    s = [(0, 0), (w.B - 1, w.D - 1), (0, w.D - 1), (w.B - 1, 0)]
    r = np.random.default_rng(seed)
    while len(set(s)) < min(n, w.C):
        s.append((int(r.integers(w.B)), int(r.integers(w.D))))
    out = []
    for p in s:
        if p not in out:
            out.append(p)
    return out[:n]


def feedback_check(y, xo, x0d, bf16):
    """Every recorded feedback against tanh of the GPU's own output."""
    B, L, D = y.shape
    assert torch.equal(xo[:, 0, :], x0d)
    worst = 0.0
    chunk = max(1, (1 << 26) // D)
    for b in range(B):
        for l0 in range(0, L - 1, chunk):
            l1 = min(L - 1, l0 + chunk)
            want = torch.tanh(y[b, l0:l1].double())
            got = xo[b, l0 + 1:l1 + 1].double()
            err = (got - want).abs()
            if bf16:
                err = err - 2.0 ** -8 * want.abs()
            worst = max(worst, err.max().item())
    log("feedback worst excess", worst)
    assert worst <= 1e-6


def full_columns(h, chans, x_cols):
    ts = np.arange(x_cols.shape[1], dtype=np.int64)
    h_cols = [h[:, c] for _, c in chans]
    return np.stack(oracle_points_parallel(h_cols, list(x_cols), [ts] * len(chans)))


def open_full(name, n=NSAMP):
    w = workloads.get(name)
    log("case", name, "open loop: generating inputs")
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    hd, xd = to_dev(h, w.dtype), to_dev(x, w.dtype)
    log("case", name, "open loop: GPU pass")
    y, _ = gpu_run(hd, w.B, w.D, w.L, w.dtype, xd, closed=False, want_x=False)
    del hd, xd
    assert torch.isfinite(y).all().item()
    chans = sample_channels(w, n)
    yg = columns(y, chans)
    del y
    torch.cuda.empty_cache()
    xc = np.stack([x[b, :, c] for b, c in chans]).astype(np.float64)
    log("case", name, "open loop: oracle on", len(chans), "channels")
    ref = full_columns(h, chans, xc)
    err = rel_l2(yg, ref)
    per = [rel_l2(yg[k], ref[k]) for k in range(len(chans))]
    log("rel l2", err, "worst channel", max(per))
    assert err <= 1e-5
    assert max(per) <= 1e-5          # an error confined to one channel shows here
    return w, h, x


def closed_full(name, n=NSAMP, free_prefix=4096, free_chans=4):
    w = workloads.get(name)
    bf16 = w.dtype == "bf16"
    log("case", name, "closed loop: generating inputs")
    h = workloads.make_filter(w)
    x0 = workloads.make_x0(w)
    hd, x0d = to_dev(h, w.dtype), to_dev(x0, w.dtype)
    log("case", name, "closed loop: GPU pass")
    y, xo = gpu_run(hd, w.B, w.D, w.L, w.dtype, x0d, closed=True)
    assert torch.isfinite(y).all().item()
    feedback_check(y, xo, x0d, bf16)
    chans = sample_channels(w, n)
    yg, xg = columns(y, chans), columns(xo, chans)
    del y, xo, hd
    torch.cuda.empty_cache()
    # teacher-forced: the oracle fed the GPU's recorded inputs
    log("case", name, "closed loop: teacher-forced oracle on", len(chans), "channels")
    ref = full_columns(h, chans, xg)
    err = np.abs(yg - ref).max()
    log("teacher-forced max abs", err)
    assert err <= 1e-3
    # free-running, on the prefix where the trajectory is unique at fp32 level
    fc = chans[:free_chans]
    P = min(free_prefix, w.L)
    hs = np.stack([h[:P, c] for _, c in fc], axis=1)
    x0s = np.array([[x0[b, c] for b, c in fc]])
    hor = chaos_horizon(hs, x0s, P, bf16=bf16)
    yr, _ = oracle.default().conv_closed(hs, x0s, L=P, bf16=bf16)
    free = np.abs(yg[:free_chans, :hor] - yr[0, :hor, :].T).max() if hor > 0 else 0.0
    log("chaos horizon", hor, "of prefix", P, "free-running max abs", free)
    assert hor >= min(P, 256)
    assert free <= 1e-3
    return w


def prompted_full(name, P, n=NSAMP):
    """A prompt of the workload's first P open-loop inputs, then the feedback
    (fi_run_prompted): the recorded inputs hold the prompt unchanged and
    tanh(y[t-1]) from P on, everywhere; sampled channels teacher-forced."""
    w = workloads.get(name)
    bf16 = w.dtype == "bf16"
    log("case", name, "prompt", P, ": generating inputs")
    h = workloads.make_filter(w)
    prompt = np.ascontiguousarray(workloads.make_x(w)[:, :P, :])
    hd, pd = to_dev(h, w.dtype), to_dev(prompt, w.dtype)
    log("case", name, "prompt", P, ": GPU pass")
    y, xo = gpu_prompted(hd, w.B, w.D, w.L, w.dtype, pd, P)
    assert torch.isfinite(y).all().item()
    assert torch.equal(xo[:, :P, :], pd)
    worst = 0.0
    chunk = max(1, (1 << 26) // w.D)
    for b in range(w.B):
        for l0 in range(P - 1, w.L - 1, chunk):
            l1 = min(w.L - 1, l0 + chunk)
            want = torch.tanh(y[b, l0:l1].double())
            err = (xo[b, l0 + 1:l1 + 1].double() - want).abs()
            if bf16:
                err = err - 2.0 ** -8 * want.abs()
            worst = max(worst, err.max().item())
    log("feedback worst excess", worst)
    assert worst <= 1e-6
    chans = sample_channels(w, n)
    yg, xg = columns(y, chans), columns(xo, chans)
    del y, xo, hd, pd
    torch.cuda.empty_cache()
    log("case", name, "prompt", P, ": teacher-forced oracle on", len(chans), "channels")
    ref = full_columns(h, chans, xg)
    err = np.abs(yg - ref).max()
    log("teacher-forced max abs", err, "prompt part rel l2", rel_l2(yg[:, :P], ref[:, :P]))
    assert err <= 1e-3
    assert rel_l2(yg[:, :P], ref[:, :P]) <= 1e-5     # the prompt's outputs are open loop


# ------------------------------------------------------------------ D=1024
def test_hyena_d1024_l16k_prompt_8192():
    prompted_full("hyena-d1024-l16k", 8192, n=32)


def test_hyena_d1024_l16k_closed():
    closed_full("hyena-d1024-l16k", n=32)


def test_hyena_d1024_l16k_open():
    open_full("hyena-d1024-l16k", n=32)


# ------------------------------------------------------------------ B=8, L=64K
def test_b8_d2048_l64k_open():
    open_full("b8-d2048-l64k")


def test_b8_d2048_l64k_closed():
    closed_full("b8-d2048-l64k", free_prefix=2048)


def test_b8_d2048_l64k_prompt_32768():
    prompted_full("b8-d2048-l64k", 32768)


# ------------------------------------------------------------------ bf16, L=128K
def test_b4_d4096_l128k_bf16_open_sampled():
    """256 sampled (b, c, t): uniform ones plus t in {0, L-1} and the
    power-of-two boundaries; relative L2 over the samples; two whole channels."""
    w = workloads.get("b4-d4096-l128k-bf16")
    log("case", w.name, "generating inputs")
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    hd, xd = to_dev(h, w.dtype), to_dev(x, w.dtype)
    log("case", w.name, "GPU pass")
    y, _ = gpu_run(hd, w.B, w.D, w.L, w.dtype, xd, closed=False, want_x=False)
    del hd, xd
    assert torch.isfinite(y).all().item()
    r = np.random.default_rng(3)
    fixed = [0, w.L - 1] + [p for k in range(1, 17) for p in ((1 << k) - 1, 1 << k)]
    ts = np.array(fixed + r.integers(0, w.L, size=256 - len(fixed)).tolist(), dtype=np.int64)
    bs = r.integers(0, w.B, size=256)
    cs = r.integers(0, w.D, size=256)
    bs[:4], cs[:4] = [0, w.B - 1, 0, w.B - 1], [0, w.D - 1, w.D - 1, 0]
    yg = y[torch.from_numpy(bs).cuda(), torch.from_numpy(ts).cuda(), torch.from_numpy(cs).cuda()]
    yg = yg.double().cpu().numpy()
    whole = [(0, 0), (w.B - 1, w.D - 1)]
    yw = columns(y, whole)
    del y
    torch.cuda.empty_cache()
    log("case", w.name, "oracle on 256 samples and 2 channels")
    refs = oracle_points_parallel([h[:, c] for c in cs], [x[b, :, c] for b, c in zip(bs, cs)],
                                  [np.array([t]) for t in ts])
    ref = np.array([v[0] for v in refs])
    err = rel_l2(yg, ref)
    # per sample: 1e-5 of the Cauchy-Schwarz bound on |y[t]|, the norms of the
    # filter prefix and of the inputs that reach position t
    scale = np.array([np.linalg.norm(h[:t + 1, c].astype(np.float64)) *
                      np.linalg.norm(x[b, :t + 1, c].astype(np.float64)) for b, c, t in zip(bs, cs, ts)])
    worst = float(np.max(np.abs(yg - ref) / np.maximum(scale, 1e-30)))
    log("samples rel l2", err, "worst sample / its bound scale", worst)
    assert err <= 1e-5
    assert worst <= 1e-5
    xw = np.stack([x[b, :, c] for b, c in whole]).astype(np.float64)
    refw = full_columns(h, whole, xw)
    errw = rel_l2(yw, refw)
    perw = [rel_l2(yw[k], refw[k]) for k in range(len(whole))]
    log("whole channels rel l2", errw, "per channel", perw)
    assert errw <= 1e-5
    assert max(perw) <= 1e-5


# ------------------------------------------------------------------ L=1M power law
def test_d768_l1m_powerlaw_closed_boundaries():
    """Closed loop at L = 2^20: feedback checked everywhere; teacher-forced at
    every tile boundary of the schedule (i-1, i, i+U-1, i+U for every FFT
    tile, 2^k-1 and 2^k) on 8 channels and at the power-of-two boundaries on
    8 more; free-running on the prefix before the chaos horizon."""
    w = workloads.get("d768-l1m-powerlaw")
    log("case", w.name, "generating inputs")
    h = workloads.make_filter(w)
    x0 = workloads.make_x0(w)
    hd, x0d = to_dev(h, w.dtype), to_dev(x0, w.dtype)
    log("case", w.name, "GPU pass")
    y, xo = gpu_run(hd, w.B, w.D, w.L, w.dtype, x0d, closed=True)
    assert torch.isfinite(y).all().item()
    feedback_check(y, xo, x0d, False)
    chans = sample_channels(w, 16)
    yg, xg = columns(y, chans), columns(xo, chans)
    del y, xo, hd
    torch.cuda.empty_cache()
    tiles = boundary_positions(w.L, T=fi.FI_DEFAULT_SMALL_TILE_MAX, extra=256, seed=4)
    pow2 = boundary_positions(w.L, T=w.L, extra=64, seed=5)
    ts = [tiles] * 8 + [pow2] * 8
    log("case", w.name, "teacher-forced oracle at", len(tiles), "positions x 8 and", len(pow2), "x 8")
    refs = oracle_points_parallel([h[:, c] for _, c in chans], list(xg), ts)
    err = max(np.abs(yg[k][ts[k]] - refs[k]).max() for k in range(len(chans)))
    log("teacher-forced max abs", err)
    assert err <= 1e-3
    P = 1 << 14
    fc = chans[:4]
    hs = np.stack([h[:P, c] for _, c in fc], axis=1)
    x0s = np.array([[x0[b, c] for b, c in fc]])
    hor = chaos_horizon(hs, x0s, P)
    yr, _ = oracle.default().conv_closed(hs, x0s, L=P)
    free = np.abs(yg[:4, :hor] - yr[0, :hor, :].T).max()
    log("chaos horizon", hor, "of prefix", P, "free-running max abs", free)
    assert hor >= 256
    assert free <= 1e-3
