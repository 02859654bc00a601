"""Pins of the oracle's multi-layer stack (page "Flash Inference: Inferenza in
Tempo Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga e Oltre",
sections "Algoritmo di Inferenza LCSM (Algoritmo 2)", "Architettura del
Modello" and "Configurazione Sperimentale"), against facts that do not come
from the oracle:

* a linear stack (identity activation and identity weights) is the
  composition of its layers' convolutions: numpy.convolve applied layer by
  layer;
* one tanh layer with identity weights is the single-mixer closed loop
  (``conv_closed``, itself pinned in test_oracle_pins.py): the same realised
  inputs, and the stack's output is tanh of the mixer's;
* delta_0 filters make every mixer the identity, so each position runs the
  blocks alone: W2 GELU(W1 v) evaluated with numpy and scipy's erf;
* a tiny stack evaluated by brute force in another form (each layer's mixer
  as an explicit lower-triangular Toeplitz matrix over the whole prefix);
* the sampler alone (identity layer) accumulates the noise: x[t] = x[0] +
  sigma * sum_{s<t} noise[s].

Each planted mistake in the stack (mutants 8..12) fails at least one of these.
"""
import numpy as np
import pytest
from scipy.special import erf

import oracle as oracle_mod


def _rng(k):
    return np.random.default_rng(1000 + k)


def _gelu(v):
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def _eye(M, D):
    return np.repeat(np.eye(D)[None], M, axis=0)


def _decaying(r, M, L, D, tau=6.0):
    return r.standard_normal((M, L, D)) * np.exp(-np.arange(L) / tau)[None, :, None] / 2.0


def _linear_chain(rho, x):
    """Per channel, numpy.convolve through every layer, truncated to L."""
    M, L, D = rho.shape
    y = x.copy()
    for l in range(M):
        out = np.empty_like(y)
        for b in range(y.shape[0]):
            for c in range(D):
                out[b, :, c] = np.convolve(y[b, :, c], rho[l, :, c])[:L]
        y = out
    return y


def _blocks_only(w1, w2, x, act=_gelu):
    """delta_0 filters: a^{l+1}_t = W2 act(W1 a^l_t) at every position."""
    a = x.copy()
    for l in range(w1.shape[0]):
        a = np.einsum("jk,btk->btj", w2[l], act(np.einsum("jk,btk->btj", w1[l], a)))
    return a


def _toeplitz_stack(rho, w1, w2, x0, noise, sigma):
    """Free-running stack by brute force: at every position the mixers are
    evaluated as full lower-triangular Toeplitz matrix products over the
    prefix of each layer's input sequence."""
    M, L, D = rho.shape
    B = x0.shape[0]
    A = np.zeros((M + 1, B, L, D))
    A[0, :, 0] = x0
    y = np.zeros((B, L, D))
    T = np.zeros((M, D, L, L))
    for l in range(M):
        for c in range(D):
            for t in range(L):
                for s in range(t + 1):
                    T[l, c, t, s] = rho[l, t - s, c]
    for t in range(L):
        for l in range(M):
            z = np.stack([(T[l, c, :t + 1, :t + 1] @ A[l, :, :t + 1, c].T)[t] for c in range(D)], axis=-1)
            A[l + 1, :, t] = (w2[l] @ _gelu(w1[l] @ z.T)).T
        y[:, t] = A[M, :, t]
        if t + 1 < L:
            A[0, :, t + 1] = A[M, :, t] + sigma * noise[:, t]
    return y, A[0]


def _stack_battery(o):
    fails = []
    r = _rng(1)
    # linear chain
    M, L, D, B = 3, 40, 3, 2
    rho = _decaying(r, M, L, D)
    x = r.standard_normal((B, L, D))
    y, _ = o.conv_stack(rho, _eye(M, D), _eye(M, D), x, act="identity", teacher_forced=True)
    if not np.allclose(y, _linear_chain(rho, x), rtol=1e-11, atol=1e-11):
        fails.append("linear_chain")
    # one tanh layer = the single-mixer closed loop
    rho1 = _decaying(r, 1, L, D, tau=10.0) * 2.0
    x0 = r.standard_normal((B, D))
    y, xs = o.conv_stack(rho1, _eye(1, D), _eye(1, D), x0, act="tanh")
    yc, xc = o.conv_closed(rho1[0], x0)   # its y is the mixer output, the stack's y = tanh of it
    if not (np.allclose(y, np.tanh(yc), rtol=1e-12, atol=1e-12) and np.allclose(xs, xc, rtol=1e-12, atol=1e-12)):
        fails.append("single_mixer")
    # delta_0 filters: the blocks alone
    rho0 = np.zeros((M, L, D)); rho0[:, 0, :] = 1.0
    w1 = r.standard_normal((M, D, D)) / np.sqrt(D)
    w2 = r.standard_normal((M, D, D)) / np.sqrt(D)
    y, _ = o.conv_stack(rho0, w1, w2, x, act="gelu", teacher_forced=True)
    if not np.allclose(y, _blocks_only(w1, w2, x), rtol=1e-12, atol=1e-12):
        fails.append("blocks_only")
    # brute force, free-running with noise
    Mb, Lb, Db = 2, 9, 2
    rhob = _decaying(r, Mb, Lb, Db, tau=3.0)
    w1b = r.standard_normal((Mb, Db, Db))
    w2b = r.standard_normal((Mb, Db, Db))
    x0b = r.standard_normal((2, Db))
    nz = r.standard_normal((2, Lb, Db))
    y, xs = o.conv_stack(rhob, w1b, w2b, x0b, noise=nz, sigma=0.3, act="gelu")
    yb, xb = _toeplitz_stack(rhob, w1b, w2b, x0b, nz, 0.3)
    if not (np.allclose(y, yb, rtol=1e-11, atol=1e-11) and np.allclose(xs, xb, rtol=1e-11, atol=1e-11)):
        fails.append("toeplitz_brute_force")
    # the sampler alone
    rhod = np.zeros((1, L, D)); rhod[0, 0, :] = 1.0
    nz = r.standard_normal((B, L, D))
    y, xs = o.conv_stack(rhod, _eye(1, D), _eye(1, D), x0, noise=nz, sigma=0.5, act="identity")
    want = x0[:, None, :] + 0.5 * np.concatenate([np.zeros((B, 1, D)), np.cumsum(nz[:, :-1], axis=1)], axis=1)
    if not (np.allclose(xs, want, rtol=1e-12, atol=1e-12) and np.allclose(y, want, rtol=1e-12, atol=1e-12)):
        fails.append("sampler")
    return fails


def test_stack_pins(orc):
    assert _stack_battery(orc) == []


def test_stack_m1_identity_weights_reduce_to_the_open_loop(orc):
    """One identity layer, teacher-forced: exactly the single mixer's open loop."""
    r = _rng(2)
    L, D = 200, 5
    rho = _decaying(r, 1, L, D, tau=30.0)
    x = r.standard_normal((3, L, D))
    y, _ = orc.conv_stack(rho, _eye(1, D), _eye(1, D), x, act="identity", teacher_forced=True)
    np.testing.assert_allclose(y, orc.conv_open(rho[0], x), rtol=1e-12, atol=1e-12)


def test_stack_batch_rows_are_independent(orc):
    r = _rng(3)
    M, L, D = 2, 50, 4
    rho = _decaying(r, M, L, D)
    w1 = r.standard_normal((M, D, D)) / 2
    w2 = r.standard_normal((M, D, D)) / 2
    x0 = r.standard_normal((3, D))
    y, _ = orc.conv_stack(rho, w1, w2, x0)
    y2, _ = orc.conv_stack(rho, w1, w2, x0[::-1].copy())
    np.testing.assert_array_equal(y2, y[::-1])


@pytest.mark.parametrize("mutant", [8, 9, 10, 11, 12])
def test_stack_mutants_are_caught(tmp_path, mutant):
    path = oracle_mod.build(tmp_path / f"libfio_m{mutant}.so", mutant=mutant)
    o = oracle_mod.Oracle(oracle_mod.load(path), threads=2)
    assert o.mutant == mutant
    assert _stack_battery(o), f"mutant {mutant} survived every stack pin"
