"""Pins for the CPU oracle, independent of the oracle itself.

The oracle computes the plain definition of the page "Flash Inference:
Inferenza in Tempo Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga
e Oltre", section "Definizione del Compito": per channel,
y[t] = sum_{s<=t} h[t-s] x[s] (0-indexed, lag 0 included), and in closed loop
x[t+1] = tanh(y[t]).  The pages print no worked example, so these tests pin it
to what mathematics fixes: a textbook routine (numpy.convolve,
scipy.signal.lfilter), closed forms, exact integer arithmetic, invariants and
pure-Python brute force on tiny inputs.  ``test_mutants_are_caught`` plants
each of the oracle's mutation hooks and checks that some pin fails.
"""
import math
import random

import numpy as np
import pytest
import scipy.signal

import oracle as oracle_mod
import workloads


def _np_conv(h, x):
    """numpy.convolve per channel, truncated to the causal window."""
    L, D = h.shape
    x3 = x if x.ndim == 3 else x[None]
    out = np.empty(x3.shape, dtype=np.float64)
    for b in range(x3.shape[0]):
        for c in range(D):
            out[b, :, c] = np.convolve(x3[b, :, c].astype(np.float64),
                                       h[:, c].astype(np.float64))[:L]
    return out if x.ndim == 3 else out[0]


def _rng(seed=1):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ textbook routine
def test_matches_numpy_convolve_small_mixer(orc):
    w = workloads.get("mixer-d16-l1k")
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    y = orc.conv_open(h, x)
    ref = _np_conv(h, x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,L,D", [(1, 1, 1), (2, 2, 3), (1, 3, 17), (2, 7, 5),
                                   (3, 16, 2), (1, 100, 33), (2, 257, 4)])
def test_matches_numpy_convolve_shapes(orc, B, L, D):
    r = _rng(B * 1000 + L * 10 + D)
    h = r.standard_normal((L, D))
    x = r.standard_normal((B, L, D))
    np.testing.assert_allclose(orc.conv_open(h, x), _np_conv(h, x), rtol=1e-12, atol=1e-12)


def test_points_match_numpy_convolve(orc):
    r = _rng(7)
    L = 3000
    h = r.standard_normal(L)
    x = r.standard_normal(L)
    ts = np.array([0, 1, 2, 63, 64, 65, 1023, 1024, 2047, 2999])
    ref = np.convolve(x, h)[:L][ts]
    np.testing.assert_allclose(orc.conv_points(h, x, ts), ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- closed forms, open loop
def test_delta0_is_identity(orc):
    r = _rng(2)
    L, D = 300, 5
    h = np.zeros((L, D)); h[0] = 1.0
    x = r.standard_normal((2, L, D))
    assert np.array_equal(orc.conv_open(h, x), x)


@pytest.mark.parametrize("k", [1, 2, 3, 127, 255, 299])
def test_delta_k_is_shift(orc, k):
    r = _rng(3 + k)
    L, D = 300, 3
    h = np.zeros((L, D)); h[k] = 1.0
    x = r.standard_normal((1, L, D))
    y = orc.conv_open(h, x)
    ref = np.zeros_like(x)
    ref[:, k:, :] = x[:, :L - k, :]
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("a", [0.5, -0.9, math.exp(-1 / 64.0), math.exp(-1 / 8192.0)])
def test_geometric_filter_is_first_order_recurrence(orc, a):
    r = _rng(4)
    L, D = 2048, 2
    j = np.arange(L, dtype=np.float64)
    h = np.repeat((a ** j)[:, None], D, axis=1)
    x = r.standard_normal((L, D))
    y = orc.conv_open(h, x)
    for c in range(D):
        ref = scipy.signal.lfilter([1.0], [1.0, -a], x[:, c])
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-9, atol=1e-9)


def test_constant_input_gives_prefix_sums(orc):
    r = _rng(5)
    L, D = 500, 4
    h = r.standard_normal((L, D))
    y = orc.conv_open(h, np.ones((L, D)))
    np.testing.assert_allclose(y, np.cumsum(h, axis=0), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ closed forms, closed loop
def test_closed_delta0_iterates_tanh(orc):
    L, D = 200, 3
    h = np.zeros((L, D)); h[0] = 1.0
    x0 = np.array([[0.3, -2.0, 1.5]])
    y, x = orc.conv_closed(h, x0)
    for c in range(D):
        v = x0[0, c]
        for t in range(L):
            assert y[0, t, c] == v
            v = math.tanh(v)


@pytest.mark.parametrize("k", [1, 3, 17])
def test_closed_delta_k(orc, k):
    L, D = 120, 2
    h = np.zeros((L, D)); h[k] = 1.0
    x0 = np.array([[0.7, -1.1]])
    y, x = orc.conv_closed(h, x0)
    for c in range(D):
        xs = [x0[0, c]] + [0.0] * (L - 1)
        for t in range(L - 1):
            xs[t + 1] = math.tanh(xs[t - k]) if t >= k else 0.0
        ys = [xs[t - k] if t >= k else 0.0 for t in range(L)]
        np.testing.assert_array_equal(x[0, :, c], xs)
        np.testing.assert_array_equal(y[0, :, c], ys)


@pytest.mark.parametrize("a", [0.5, math.exp(-1 / 64.0)])
def test_closed_geometric_recurrence(orc, a):
    L, D = 1500, 2
    j = np.arange(L, dtype=np.float64)
    h = np.repeat((a ** j)[:, None], D, axis=1)
    x0 = np.array([[0.4, -1.3]])
    y, _ = orc.conv_closed(h, x0)
    for c in range(D):
        ref = np.empty(L)
        ref[0] = x0[0, c]
        for t in range(1, L):
            ref[t] = a * ref[t - 1] + math.tanh(ref[t - 1])
        np.testing.assert_allclose(y[0, :, c], ref, rtol=1e-10, atol=1e-10)


# ------------------------------------------------ closed forms, prompted runs
# The generation task starts from a prompt x_0 .. x_{p-1}; the feedback
# x_{t+1} = tanh(y_t) takes over from position p.
@pytest.mark.parametrize("p", [1, 2, 7, 64])
def test_prompted_delta0(orc, p):
    L, D = 150, 2
    h = np.zeros((L, D)); h[0] = 1.0
    prompt = _rng(31).standard_normal((1, p, D))
    y, x = orc.conv_prompted(h, prompt)
    for c in range(D):
        for t in range(p):
            assert y[0, t, c] == prompt[0, t, c] and x[0, t, c] == prompt[0, t, c]
        v = prompt[0, p - 1, c]
        for t in range(p, L):
            v = math.tanh(v)
            assert y[0, t, c] == v


@pytest.mark.parametrize("p,k", [(5, 1), (9, 3), (40, 17)])
def test_prompted_delta_k(orc, p, k):
    L, D = 130, 2
    h = np.zeros((L, D)); h[k] = 1.0
    prompt = _rng(32).standard_normal((1, p, D))
    y, x = orc.conv_prompted(h, prompt)
    for c in range(D):
        xs = list(prompt[0, :, c]) + [0.0] * (L - p)
        for t in range(p - 1, L - 1):
            xs[t + 1] = math.tanh(xs[t - k]) if t >= k else 0.0
        ys = [xs[t - k] if t >= k else 0.0 for t in range(L)]
        np.testing.assert_array_equal(x[0, :, c], xs)
        np.testing.assert_array_equal(y[0, :, c], ys)


@pytest.mark.parametrize("p", [1, 3, 100])
def test_prompted_geometric_recurrence(orc, p):
    L, D, a = 700, 2, math.exp(-1 / 32.0)
    h = np.repeat((a ** np.arange(L, dtype=np.float64))[:, None], D, axis=1)
    prompt = _rng(33).standard_normal((1, p, D))
    y, _ = orc.conv_prompted(h, prompt)
    for c in range(D):
        ref = np.empty(L)
        for t in range(L):
            xt = prompt[0, t, c] if t < p else math.tanh(ref[t - 1])
            ref[t] = (a * ref[t - 1] if t else 0.0) + xt
        np.testing.assert_allclose(y[0, :, c], ref, rtol=1e-10, atol=1e-10)


def test_prompted_full_prompt_is_open_loop(orc):
    L, D = 300, 3
    r = _rng(34)
    h = r.standard_normal((L, D)); x = r.standard_normal((2, L, D))
    y, xo = orc.conv_prompted(h, x)
    np.testing.assert_array_equal(xo, x)
    np.testing.assert_allclose(y, _np_conv(h, x), rtol=1e-12, atol=1e-12)


def test_prompted_prefix_is_causal(orc):
    # the prompt's outputs are the open-loop convolution of the prompt alone
    L, D, p = 400, 2, 123
    r = _rng(35)
    h = r.standard_normal((L, D)) * 0.05
    prompt = r.standard_normal((1, p, D))
    y, _ = orc.conv_prompted(h, prompt)
    np.testing.assert_allclose(y[0, :p], _np_conv(h[:p], prompt[0]), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- exact arithmetic
def test_integer_inputs_are_exact(orc):
    r = random.Random(11)
    B, L, D = 2, 257, 3
    h = [[r.randint(-3, 3) for _ in range(D)] for _ in range(L)]
    x = [[[r.randint(-3, 3) for _ in range(D)] for _ in range(L)] for _ in range(B)]
    y = orc.conv_open(np.array(h, float), np.array(x, float))
    for b in range(B):
        for t in range(L):
            for c in range(D):
                ref = sum(h[t - s][c] * x[b][s][c] for s in range(t + 1))
                assert y[b, t, c] == ref


def test_tiny_brute_force_bitwise(orc):
    r = _rng(12)
    for L in range(1, 17):
        h = r.standard_normal((L, 2))
        x = r.standard_normal((2, L, 2))
        y = orc.conv_open(h, x)
        for b in range(2):
            for t in range(L):
                for c in range(2):
                    acc = 0.0
                    for s in range(t + 1):
                        acc += float(h[t - s, c]) * float(x[b, s, c])
                    assert y[b, t, c] == acc


# ------------------------------------------------------------------ invariants
def test_linearity_shift_and_batch_independence(orc):
    r = _rng(13)
    L, D = 400, 5
    h = r.standard_normal((L, D))
    x1 = r.standard_normal((1, L, D))
    x2 = r.standard_normal((1, L, D))
    np.testing.assert_allclose(orc.conv_open(h, 2.0 * x1 - 3.0 * x2),
                               2.0 * orc.conv_open(h, x1) - 3.0 * orc.conv_open(h, x2),
                               rtol=1e-10, atol=1e-10)
    k = 37
    xs = np.zeros_like(x1); xs[:, k:] = x1[:, :L - k]
    np.testing.assert_allclose(orc.conv_open(h, xs)[:, k:], orc.conv_open(h, x1)[:, :L - k],
                               rtol=0, atol=0)
    xb = np.concatenate([x1, x2], axis=0)
    yb = orc.conv_open(h, xb)
    yr = orc.conv_open(h, xb[::-1].copy())
    assert np.array_equal(yb[::-1], yr)


# ---------------------------------------------------------------- bf16 storage
def test_bf16_rounding_ties_and_library(orc):
    cases = {
        1.0: 1.0,
        1.0 + 2 ** -8: 1.0,                       # tie -> even (1.0)
        1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6,         # tie -> even
        1.0 + 2 ** -8 + 2 ** -30: 1.0 + 2 ** -7,  # just above the tie
        -(1.0 + 2 ** -8 + 2 ** -30): -(1.0 + 2 ** -7),
        0.0: 0.0,
        2 ** -130: 2 ** -130,                     # bf16 subnormal, exact
        0.7615941559557649: 0.76171875,           # tanh(1)
    }
    for v, want in cases.items():
        assert orc.round_bf16(v) == want, v
    import torch
    r = _rng(14)
    v32 = (r.standard_normal(20000) * np.exp(r.uniform(-20, 5, 20000))).astype(np.float32)
    lib = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_bf16(v32.astype(np.float64)), lib)
    # the input module's own rounding agrees with both
    np.testing.assert_array_equal(workloads.round_to_bf16(v32).astype(np.float64), lib)


def test_closed_loop_bf16_feedback_on_grid(orc):
    L, D = 300, 4
    w = workloads.get("mixer-d16-l1k").with_(dtype="bf16", D=D, L=L)
    h = workloads.make_filter(w)
    x0 = workloads.make_x0(w)
    _, x = orc.conv_closed(h, x0, bf16=True)
    np.testing.assert_array_equal(orc.round_bf16(x), x)
    _, xf = orc.conv_closed(h, x0, bf16=False)
    assert not np.array_equal(orc.round_bf16(xf), xf)


# --------------------------------------------------------------- mutation tests
def _pin_battery(o) -> list:
    """Compact subset of the pins above; returns the names that fail."""
    fails = []
    r = _rng(21)
    L, D = 64, 3
    h = r.standard_normal((L, D)); x = r.standard_normal((2, L, D))
    if not np.allclose(o.conv_open(h, x), _np_conv(h, x), rtol=1e-12, atol=1e-12):
        fails.append("numpy_convolve")
    hd = np.zeros((L, D)); hd[0] = 1
    if not np.array_equal(o.conv_open(hd, x), x):
        fails.append("delta0")
    hk = np.zeros((L, D)); hk[5] = 1
    ref = np.zeros_like(x); ref[:, 5:] = x[:, :-5]
    if not np.array_equal(o.conv_open(hk, x), ref):
        fails.append("delta5")
    a = 0.5
    hg = np.repeat((a ** np.arange(L))[:, None], D, axis=1)
    y, _ = o.conv_closed(hg, x[:, 0, :])
    rec = np.empty((2, L, D)); rec[:, 0] = x[:, 0]
    for t in range(1, L):
        rec[:, t] = a * rec[:, t - 1] + np.tanh(rec[:, t - 1])
    if not np.allclose(y, rec, rtol=1e-10, atol=1e-10):
        fails.append("closed_geometric")
    if o.round_bf16(1.0 + 3 * 2 ** -8) != 1.0 + 2 ** -6:
        fails.append("bf16_tie")
    p = 5
    y, _ = o.conv_prompted(hg, x[:, :p, :])
    rec = np.empty((2, L, D))
    for t in range(L):
        xt = x[:, t] if t < p else np.tanh(rec[:, t - 1])
        rec[:, t] = (a * rec[:, t - 1] if t else 0.0) + xt
    if not np.allclose(y, rec, rtol=1e-10, atol=1e-10):
        fails.append("prompted_geometric")
    return fails


def test_unmutated_oracle_passes_battery(orc):
    assert _pin_battery(orc) == []


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6, 7])
def test_mutants_are_caught(tmp_path, mutant):
    path = oracle_mod.build(tmp_path / f"libfio_m{mutant}.so", mutant=mutant)
    o = oracle_mod.Oracle(oracle_mod.load(path), threads=2)
    assert o.mutant == mutant
    assert _pin_battery(o), f"mutant {mutant} survived every pin"
