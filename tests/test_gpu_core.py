"""GPU parity at small sizes: the HIP library (through its C ABI) against the
CPU oracle on the same seeded inputs, element by element.

Tolerances (BASELINE north-star, fp32 arithmetic): open loop relative L2
error <= 1e-5; closed loop max abs error <= 1e-3 on y; closed-loop feedback
consistency |x[t+1] - tanh(y[t])| <= 1e-6 (fp64 tanh of the GPU's own y; for
bf16 storage half a bf16 ulp more).  Cases with only direct tiles and integer
data are compared bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from fi_harness import (boundary_positions, chaos_horizon, columns, gpu_prompted, gpu_run, gpu_steps,
                        host, log, rel_l2, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import exact_online_amd as fi  # noqa: E402  (fails loudly if libfi.so is missing)

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.default()
    return ORC


def small(name="mixer-d16-l1k", **kw):
    return workloads.get(name).with_(**kw)


def _open_case(w, T=0, via_steps=False):
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    hd, xd = to_dev(h, w.dtype), to_dev(x, w.dtype)
    if via_steps:
        y = gpu_steps(hd, w.B, w.D, w.L, w.dtype, xd, T)
    else:
        y, xo = gpu_run(hd, w.B, w.D, w.L, w.dtype, xd, closed=False, T=T)
        assert torch.equal(xo, xd)
    ref = orc().conv_open(h, x)
    return host(y), ref


# ---------------------------------------------------------------- open loop
@pytest.mark.parametrize("T", [0, 64, 256])
def test_small_mixer_open_run(T):
    w = small()
    log("case small mixer open run T", T)
    y, ref = _open_case(w, T)
    err = rel_l2(y, ref)
    log("rel l2", err)
    assert err <= 1e-5


def test_small_mixer_open_steps():
    w = small()
    log("case small mixer open via fi_step")
    y, ref = _open_case(w, 0, via_steps=True)
    assert rel_l2(y, ref) <= 1e-5


@pytest.mark.parametrize("L,T", [(1, 64), (2, 64), (5, 64), (63, 64), (64, 64), (65, 64), (100, 64),
                                 (129, 64), (257, 64), (300, 0), (511, 64), (513, 64), (1000, 64),
                                 (3000, 128), (5000, 64)])
def test_ragged_lengths_open(L, T):
    w = small(B=2, D=3, L=L, seed=L)
    log("case ragged open L", L, "T", T)
    y, ref = _open_case(w, T)
    assert rel_l2(y, ref) <= 1e-5
    if L <= 300:
        ys, _ = _open_case(w, T, via_steps=True)
        assert rel_l2(ys, ref) <= 1e-5


@pytest.mark.parametrize("T", [64, 128, 256])
def test_delta_filters_hit_every_level(T):
    """h = delta_k gives y[t] = x[t-k]; one k per channel, chosen on and
    around every tile side, so every level's kernel moves data exactly once."""
    L = 16384
    ks = [1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 1023, 1024,
          2047, 2048, 4095, 4096, 4097, 8191, 8192, 12345, 16383]
    D = len(ks)
    h = np.zeros((L, D), np.float32)
    for c, k in enumerate(ks):
        h[k, c] = 1.0
    x = np.random.default_rng(5).standard_normal((1, L, D)).astype(np.float32)
    log("case delta filters T", T)
    y, _ = gpu_run(to_dev(h, "f32"), 1, D, L, "f32", to_dev(x, "f32"), closed=False, T=T, want_x=False)
    y = host(y)
    for c, k in enumerate(ks):
        ref = np.zeros(L)
        ref[k:] = x[0, :L - k, c]
        err = np.abs(y[0, :, c] - ref).max()
        assert err <= 2e-5, (k, err)
        if T >= 256:
            # below the first FFT tile (side 512) only direct fp32 tiles of a
            # single nonzero tap: exact
            assert np.array_equal(y[0, :512, c], ref[:512].astype(np.float32)), k
        else:
            # below 1024 every contribution is a matrix-core block product of
            # fp16 halves (the open block's own triangle, the tiles of side
            # 256 and 512): x = hi + lo + r with |r| <= 2^-22 |x| plus, where
            # lo is an fp16 subnormal, an absolute 2^-24 of the scaled block
            # (2^-37 of the block's largest |x|), and exactly 0 where the
            # single tap meets no input
            bound = 2.0 ** -21 * np.abs(ref[:1024]) + 2.0 ** -30 * np.abs(x[0, :1024, c]).max()
            assert (np.abs(y[0, :1024, c] - ref[:1024]) <= bound).all(), k


@pytest.mark.parametrize("T", [64, 128])
def test_delta_filters_through_steps(T):
    """fi_step one position per call (the red cell fused with the small direct
    tiles, separate launches for the others): h = delta_k gives y[t] =
    x[t-k], exactly before the first FFT tile (side 2T)."""
    L = 2048
    ks = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 2047]
    D = len(ks)
    h = np.zeros((L, D), np.float32)
    for c, k in enumerate(ks):
        h[k, c] = 1.0
    x = np.random.default_rng(6).standard_normal((1, L, D)).astype(np.float32)
    log("case delta filters through fi_step T", T)
    y = host(gpu_steps(to_dev(h, "f32"), 1, D, L, "f32", to_dev(x, "f32"), T))
    for c, k in enumerate(ks):
        ref = np.zeros(L)
        ref[k:] = x[0, :L - k, c]
        assert np.abs(y[0, :, c] - ref).max() <= 2e-5, k
        assert np.array_equal(y[0, :2 * T, c], ref[:2 * T].astype(np.float32)), k


def test_bf16_through_steps():
    w = small(dtype="bf16", B=2, D=5, L=700)
    log("case bf16 open through fi_step")
    y, ref = _open_case(w, 0, via_steps=True)
    assert rel_l2(y, ref) <= 1e-5


@pytest.mark.parametrize("L,T", [(8192, 128), (8192, 0), (512, 256)])
def test_integer_data(L, T):
    """x, h in {-3..3}: direct tiles are exact; FFT tiles round to the exact
    integer (|y| < 2^24).  Positions below 512 see no FFT tile (the tiles of
    side 256 are direct products), so they are exact too."""
    D, B = 4, 2
    r = np.random.default_rng(9)
    h = r.integers(-3, 4, size=(L, D)).astype(np.float32)
    x = r.integers(-3, 4, size=(B, L, D)).astype(np.float32)
    log("case integer data T", T)
    y, _ = gpu_run(to_dev(h, "f32"), B, D, L, "f32", to_dev(x, "f32"), closed=False, T=T, want_x=False)
    y = host(y).astype(np.float64)
    ref = orc().conv_open(h, x)
    assert np.array_equal(np.rint(y), ref)
    assert np.abs(y - ref).max() < 0.05
    assert np.array_equal(y[:, :512], ref[:, :512])
    if L <= 2 * T:   # every tile direct (the largest tile side is L/2)
        assert np.array_equal(y, ref)


def test_large_fft_tiles_global_path():
    """L = 2^15: tiles of side 8192 and 16384 exceed LDS and run through the
    global-scratch passes."""
    w = workloads.get("hyena-d1024-l16k").with_(D=6, L=1 << 15, B=2)
    log("case global-path fft L=32768")
    y, ref = _open_case(w)
    assert rel_l2(y, ref) <= 1e-5


# -------------------------------------------------------------- closed loop
def _closed_case(w, T=0):
    h = workloads.make_filter(w)
    x0 = workloads.make_x0(w)
    y, xo = gpu_run(to_dev(h, w.dtype), w.B, w.D, w.L, w.dtype, to_dev(x0, w.dtype), closed=True, T=T)
    return h, x0, host(y).astype(np.float64), host(xo).astype(np.float64)


def _check_feedback(y, xo, x0, bf16):
    assert np.array_equal(xo[:, 0, :], x0.astype(np.float64))
    want = np.tanh(y[:, :-1, :])
    tol = 1e-6
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(want)   # half a bf16 ulp is at most 2^-8 of the value
    assert np.all(np.abs(xo[:, 1:, :] - want) <= tol)


@pytest.mark.parametrize("T", [0, 64])
def test_small_mixer_closed(T):
    w = small()
    log("case small mixer closed T", T)
    h, x0, y, xo = _closed_case(w, T)
    _check_feedback(y, xo, x0, False)
    assert chaos_horizon(h, x0, w.L) == w.L        # well-posed over the whole run
    yr, _ = orc().conv_closed(h, x0)
    assert np.abs(y - yr).max() <= 1e-3
    ytf = orc().conv_open(h, xo)                    # step-wise validity
    assert np.abs(y - ytf).max() <= 1e-4


@pytest.mark.parametrize("L", [1, 3, 64, 65, 300, 511, 700, 3000])
def test_ragged_closed(L):
    w = small(B=2, D=3, L=L, seed=L + 1)
    log("case ragged closed L", L)
    h, x0, y, xo = _closed_case(w, 64)
    _check_feedback(y, xo, x0, False)
    yr, _ = orc().conv_closed(h, x0)
    assert np.abs(y - yr).max() <= 1e-3


def test_bf16_open_and_closed():
    w = small(dtype="bf16", B=2, D=8, L=4096)
    log("case bf16 open")
    y, ref = _open_case(w)
    assert rel_l2(y, ref) <= 1e-5
    log("case bf16 closed")
    h, x0, y, xo = _closed_case(w)
    _check_feedback(y, xo, x0, True)
    assert np.array_equal(orc().round_bf16(xo), xo)     # stored on the bf16 grid
    ytf = orc().conv_open(h, xo)
    assert np.abs(y - ytf).max() <= 1e-4


# ----------------------------------------------------------------- prompted
# A prompt of p given inputs, then x[t+1] = tanh(y[t]) from position p on
# (fi_run_prompted).  The prompt is the first p inputs of the workload's
# open-loop series.
def _prompted_case(w, p, T=0):
    h = workloads.make_filter(w)
    prompt = np.ascontiguousarray(workloads.make_x(w)[:, :p, :])
    y, xo = gpu_prompted(to_dev(h, w.dtype), w.B, w.D, w.L, w.dtype, to_dev(prompt, w.dtype), p, T)
    return h, prompt, host(y).astype(np.float64), host(xo).astype(np.float64)


def _check_prompted(h, prompt, y, xo, bf16):
    p = prompt.shape[1]
    assert np.array_equal(xo[:, :p, :], prompt.astype(np.float64))   # the prompt, unchanged
    want = np.tanh(y[:, p - 1:-1, :])
    tol = 1e-6
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    assert np.all(np.abs(xo[:, p:, :] - want) <= tol)
    # each output from the inputs that were realised, to the closed-loop bound
    # (|y| reaches ~10^2 in the long-filter family, so fp32 rounding alone is
    # ~1e-4 there)
    ytf = orc().conv_open(h, xo)
    assert np.abs(y - ytf).max() <= 1e-3


@pytest.mark.parametrize("p,T", [(2, 0), (100, 0), (255, 0), (256, 0), (257, 0), (300, 64), (511, 0),
                                 (512, 0), (700, 0), (1023, 0), (300, 256), (768, 256)])
def test_prompted_small_mixer(p, T):
    w = small(B=2, D=5, seed=p)
    log("case prompted small mixer p", p, "T", T)
    h, prompt, y, xo = _prompted_case(w, p, T)
    _check_prompted(h, prompt, y, xo, False)
    yr, _ = orc().conv_prompted(h, prompt)         # free-running: this family is not chaotic
    assert np.abs(y - yr).max() <= 1e-3


@pytest.mark.parametrize("L,p", [(300, 299), (300, 257), (700, 513), (700, 650), (700, 699), (1000, 768)])
def test_prompted_ragged(L, p):
    w = small(B=2, D=3, L=L, seed=L + p)
    log("case prompted ragged L", L, "p", p)
    h, prompt, y, xo = _prompted_case(w, p)
    _check_prompted(h, prompt, y, xo, False)
    yr, _ = orc().conv_prompted(h, prompt)
    assert np.abs(y - yr).max() <= 1e-3


def test_prompted_extremes_are_closed_and_open_loop():
    w = small(B=2, D=4, L=700)
    hd = to_dev(workloads.make_filter(w), "f32")
    x = workloads.make_x(w)
    log("case prompted p=1 and p=L")
    y1, x1 = gpu_prompted(hd, w.B, w.D, w.L, "f32", to_dev(np.ascontiguousarray(x[:, :1]), "f32"), 1)
    yc, xc = gpu_run(hd, w.B, w.D, w.L, "f32", to_dev(np.ascontiguousarray(x[:, 0]), "f32"), closed=True)
    assert torch.equal(y1, yc) and torch.equal(x1, xc)
    yl, xl = gpu_prompted(hd, w.B, w.D, w.L, "f32", to_dev(x, "f32"), w.L)
    yo, _ = gpu_run(hd, w.B, w.D, w.L, "f32", to_dev(x, "f32"), closed=False)
    assert torch.equal(yl, yo)


@pytest.mark.parametrize("L,p", [(16384, 5000), (16384, 8192), (1 << 15, 12345)])
def test_prompted_long(L, p):
    # FFT tiles in LDS and (L = 2^15) through global scratch; this family is
    # chaotic in closed loop, so the check is per step against the realised inputs
    w = workloads.get("hyena-d1024-l16k").with_(D=4, L=L, B=1, seed=p)
    log("case prompted long L", L, "p", p)
    h, prompt, y, xo = _prompted_case(w, p)
    _check_prompted(h, prompt, y, xo, False)


def test_prompted_bf16():
    w = small(dtype="bf16", B=2, D=8, L=4096)
    log("case prompted bf16 p 1500")
    h, prompt, y, xo = _prompted_case(w, 1500)
    _check_prompted(h, prompt, y, xo, True)
    assert np.array_equal(orc().round_bf16(xo), xo)


def test_prompted_errors():
    w = small(D=4, L=256)
    h = to_dev(workloads.make_filter(w), "f32")
    x = to_dev(workloads.make_x(w), "f32")
    y = torch.empty((1, 256, 4), device="cuda")
    with fi.Mixer(1, 4, 256, h, stream=torch.cuda.current_stream()) as m:
        for p in (0, -1, 257):
            with pytest.raises(fi.FiError) as e:
                m.run_prompted(x, p, y)
            assert e.value.status == fi.FI_ERR_INVALID
        with pytest.raises(fi.FiError) as e:
            m.run_prompted(0, 10, y)
        assert e.value.status == fi.FI_ERR_INVALID
        m.run_prompted(x, 10, y)
        with pytest.raises(fi.FiError) as e:
            m.run_prompted(x, 10, y)
        assert e.value.status == fi.FI_ERR_STATE
        torch.cuda.synchronize()


# ------------------------------------------------------------- HIP graphs
def test_persistent_pass_replays_from_a_captured_graph():
    """One fi_run_closed_loop / fi_run_prompted / open-loop launch captured on
    the handle's stream and replayed several times, with eager work and
    synchronisation between the replays: every replay equals the eager run
    (the pass clears the rows it owns itself, so it needs no host-side
    reset between replays)."""
    w = small(B=2, D=8, L=2048)
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    hd = to_dev(h, "f32")
    x0d = to_dev(np.ascontiguousarray(x[:, 0]), "f32")
    xd = to_dev(x, "f32")
    pd = to_dev(np.ascontiguousarray(x[:, :700]), "f32")
    st = torch.cuda.Stream()
    cases = [("closed", lambda m, y, xo: m.run(x0d, fi.FI_FEEDBACK_TANH, y, xo)),
             ("open", lambda m, y, xo: m.run(xd, fi.FI_FEEDBACK_NONE, y, xo)),
             ("prompted", lambda m, y, xo: m.run_prompted(pd, 700, y, xo))]
    for name, call in cases:
        log("case graph replay", name)
        with fi.Mixer(w.B, w.D, w.L, hd, stream=st) as m:
            y_ref = torch.empty((w.B, w.L, w.D), device="cuda")
            x_ref = torch.empty_like(y_ref)
            with torch.cuda.stream(st):
                call(m, y_ref, x_ref)
            torch.cuda.synchronize()
            m.reset()
            y = torch.empty_like(y_ref)
            xo = torch.empty_like(y_ref)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                call(m, y, xo)
            for _ in range(3):
                y.fill_(float("nan"))
                xo.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(y, y_ref) and torch.equal(xo, x_ref)
            del g


def test_distinct_handles_are_independent():
    """Two handles with different filters and sizes, their passes interleaved
    on one stream, give what each gives alone."""
    wa = small(B=1, D=6, L=1500, seed=3)
    wb = small(B=2, D=4, L=900, seed=4)
    st = torch.cuda.current_stream()
    ha, hb = to_dev(workloads.make_filter(wa), "f32"), to_dev(workloads.make_filter(wb), "f32")
    xa, xb = to_dev(workloads.make_x(wa), "f32"), to_dev(workloads.make_x(wb), "f32")
    ya1 = torch.empty((wa.B, wa.L, wa.D), device="cuda")
    yb1 = torch.empty((wb.B, wb.L, wb.D), device="cuda")
    with fi.Mixer(wa.B, wa.D, wa.L, ha, stream=st) as ma:
        ma.run(xa, fi.FI_FEEDBACK_NONE, ya1)
    with fi.Mixer(wb.B, wb.D, wb.L, hb, stream=st) as mb:
        mb.run(xb, fi.FI_FEEDBACK_NONE, yb1)
    ya2, yb2 = torch.empty_like(ya1), torch.empty_like(yb1)
    log("case two handles interleaved")
    with fi.Mixer(wa.B, wa.D, wa.L, ha, stream=st) as ma, fi.Mixer(wb.B, wb.D, wb.L, hb, stream=st) as mb:
        ma.run(xa, fi.FI_FEEDBACK_NONE, ya2)
        mb.run(xb, fi.FI_FEEDBACK_NONE, yb2)
        ma.reset()
        mb.reset()
        ma.run(xa, fi.FI_FEEDBACK_NONE, ya2)
        mb.run(xb, fi.FI_FEEDBACK_NONE, yb2)
        torch.cuda.synchronize()
    assert torch.equal(ya1, ya2) and torch.equal(yb1, yb2)


# ------------------------------------------------------------------- state
def test_state_machine_and_determinism():
    w = small(D=4, L=256)
    h = to_dev(workloads.make_filter(w), "f32")
    x = to_dev(workloads.make_x(w), "f32")
    y1 = torch.empty((1, 256, 4), device="cuda")
    y2 = torch.empty_like(y1)
    xt = torch.zeros((1, 4), device="cuda")
    yt = torch.zeros((1, 4), device="cuda")
    with fi.Mixer(1, 4, 256, h, stream=torch.cuda.current_stream()) as m:
        m.run(x, fi.FI_FEEDBACK_NONE, y1)
        with pytest.raises(fi.FiError) as e:
            m.step(xt, yt)
        assert e.value.status == fi.FI_ERR_STATE
        with pytest.raises(fi.FiError) as e:
            m.run(x, fi.FI_FEEDBACK_NONE, y2)
        assert e.value.status == fi.FI_ERR_STATE
        m.reset()
        m.step(xt, yt)
        with pytest.raises(fi.FiError) as e:
            m.run(x, fi.FI_FEEDBACK_NONE, y2)
        assert e.value.status == fi.FI_ERR_STATE
        m.reset()
        m.run(x, fi.FI_FEEDBACK_NONE, y2)
        torch.cuda.synchronize()
    assert torch.equal(y1, y2)
