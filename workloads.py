"""Seeded synthetic workloads for the online causal long convolution.

This module draws filters and inputs and nothing else: it holds none of the
convolution's arithmetic, so both the CPU oracle (``oracle/``) and the GPU
library take their inputs from here and share no other code.

The workloads follow the filter families of the Flash Inference setting
(per-channel long filters rho in R^{L x D}, page "Flash Inference: Inferenza in
Tempo Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga e Oltre",
section "Definizione Specifica di LCSM"): decaying Gaussian filters
``h[j, c] = N(0,1) * env(j, c)`` with either an exponential envelope
``exp(-j / tau_c)`` (tau_c fixed or log-uniform per channel) or a power law
``(1 + j) ** -0.6``.  Inputs are i.i.d. N(0,1).

Recipe (fixed here, used by tests and the benchmark alike):

* filter stream ``numpy.random.default_rng([seed, 0])`` (PCG64): first the
  per-channel ``tau`` (float64, only for the log-uniform family), then
  ``g = standard_normal((L, D), float32)`` drawn in row chunks (numpy fills
  arrays in C order, so chunking does not change the values);
  ``h = float32(float64(g) * env)``; for bf16 storage ``h`` is then rounded
  once, fp32 -> bf16 round-to-nearest-even.
* open-loop inputs ``x`` from ``default_rng([seed, 1])``:
  ``standard_normal((B, L, D), float32)`` in batch/row chunks, rounded the
  same way for bf16 storage.
* closed-loop start ``x0`` from ``default_rng([seed, 2])``:
  ``standard_normal((B, D), float32)``.

Arrays are returned as float32 whose values are exactly representable in the
storage dtype; :func:`to_bf16_bits` gives the uint16 bit patterns to upload.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "make_filter", "make_x", "make_x0",
    "round_to_bf16", "to_bf16_bits", "from_bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    D: int
    L: int
    dtype: str                 # storage of x and h: "f32" or "bf16"; y is always f32
    family: str                # "exp_fixed" | "exp_loguniform" | "powerlaw"
    tau: tuple = (256.0, 256.0)  # fixed tau or [lo, hi] of the log-uniform draw
    scale: float = 1.0         # extra factor on the filter (1/sqrt(64) for the small mixer)
    power: float = 0.6         # power-law exponent
    modes: tuple = ("closed",)
    seed: int = 0

    @property
    def C(self) -> int:
        return self.B * self.D

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Single small mixer: every output checkable against the full oracle in seconds.
    "mixer-d16-l1k": Workload("mixer-d16-l1k", 1, 16, 1024, "f32", "exp_fixed",
                              tau=(256.0, 256.0), scale=1.0 / math.sqrt(64.0),
                              modes=("open", "closed")),
    # Hyena-like mixer: the throughput workload.
    "hyena-d1024-l16k": Workload("hyena-d1024-l16k", 1, 1024, 16384, "f32", "exp_loguniform",
                                 tau=(64.0, 8192.0), modes=("closed", "open")),
    "b8-d2048-l64k": Workload("b8-d2048-l64k", 8, 2048, 65536, "f32", "exp_loguniform",
                              tau=(64.0, 8192.0), modes=("open", "closed")),
    "b4-d4096-l128k-bf16": Workload("b4-d4096-l128k-bf16", 4, 4096, 131072, "bf16",
                                    "exp_loguniform", tau=(128.0, 32768.0), modes=("open",)),
    "d768-l1m-powerlaw": Workload("d768-l1m-powerlaw", 1, 768, 1 << 20, "f32", "powerlaw",
                                  modes=("closed",)),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------- bf16 storage
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    return from_bf16_bits(to_bf16_bits(a))


# ---------------------------------------------------------------- generators
_ROWS = 1 << 14   # row chunk for large draws


def _taus(w: Workload, rng: np.random.Generator, D: int) -> np.ndarray:
    lo, hi = w.tau
    if w.family == "exp_loguniform":
        return np.exp(rng.uniform(math.log(lo), math.log(hi), size=D))
    return np.full(D, float(lo))


def _env(w: Workload, j: np.ndarray, taus: np.ndarray) -> np.ndarray:
    if w.family == "powerlaw":
        return ((1.0 + j) ** (-w.power))[:, None] * w.scale
    return np.exp(-j[:, None] / taus[None, :]) * w.scale


def make_filter(w: Workload, L: int | None = None, D: int | None = None) -> np.ndarray:
    """Filter h[L][D] (float32 values exactly representable in ``w.dtype``)."""
    L = w.L if L is None else L
    D = w.D if D is None else D
    rng = np.random.default_rng([w.seed, 0])
    taus = _taus(w, rng, D) if w.family != "powerlaw" else None
    h = np.empty((L, D), dtype=np.float32)
    for r0 in range(0, L, _ROWS):
        r1 = min(L, r0 + _ROWS)
        g = rng.standard_normal((r1 - r0, D), dtype=np.float32)
        j = np.arange(r0, r1, dtype=np.float64)
        h[r0:r1] = (g.astype(np.float64) * _env(w, j, taus)).astype(np.float32)
    if w.dtype == "bf16":
        for r0 in range(0, L, _ROWS):
            h[r0:r0 + _ROWS] = round_to_bf16(h[r0:r0 + _ROWS])
    return h


def make_x(w: Workload, B: int | None = None, L: int | None = None,
           D: int | None = None) -> np.ndarray:
    """Open-loop inputs x[B][L][D] (float32, representable in ``w.dtype``)."""
    B = w.B if B is None else B
    L = w.L if L is None else L
    D = w.D if D is None else D
    rng = np.random.default_rng([w.seed, 1])
    x = np.empty((B, L, D), dtype=np.float32)
    for b in range(B):
        for r0 in range(0, L, _ROWS):
            r1 = min(L, r0 + _ROWS)
            blk = rng.standard_normal((r1 - r0, D), dtype=np.float32)
            x[b, r0:r1] = round_to_bf16(blk) if w.dtype == "bf16" else blk
    return x


def make_x0(w: Workload, B: int | None = None, D: int | None = None) -> np.ndarray:
    """Closed-loop start x0[B][D] (float32, representable in ``w.dtype``)."""
    B = w.B if B is None else B
    D = w.D if D is None else D
    rng = np.random.default_rng([w.seed, 2])
    x0 = rng.standard_normal((B, D), dtype=np.float32)
    return round_to_bf16(x0) if w.dtype == "bf16" else x0


# ---------------------------------------------------------------- the stack
@dataclasses.dataclass(frozen=True)
class StackWorkload:
    """The multi-layer synthetic LCSM of the page's experiments (M layers,
    each a long-convolution mixer followed by an MLP + GELU block, and a
    sampler that adds noise).  Recipe, fixed here:

    * layer l's filter ``rho[l][j][c] = N(0,1) exp(-j / tau_c) / sqrt(S_c)``
      with tau_c log-uniform in ``tau`` per layer and channel and
      ``S_c = sum_j exp(-2 j / tau_c)`` (so a white input keeps unit
      variance through the mixer), from ``default_rng([seed, 10, l])``: tau
      first, then the Gaussians in row chunks;
    * ``W1[l], W2[l]`` (D x D, row j = output j) ``N(0, 1/D)`` from
      ``default_rng([seed, 11])`` and ``([seed, 12])``, layer by layer.  The
      blocks have no normalisation, so the fed-back loop is stable only
      when a block shrinks its input: at N(0, 2/D) the loop resonates at
      the filters' peak frequencies and grows without bound (|y| ~ 1e5 by
      t = 3000 at M = 2); at N(0, 1/D) it stays bounded, and a deep stack
      (M = 18) damps the signal to ~1e-7, leaving the sampler's noise;
    * ``x0[B][D] ~ N(0,1)`` from ``([seed, 13])``; the sampler's noise
      ``noise[B][L][D] ~ N(0,1)`` from ``([seed, 14])``, scaled by ``sigma``.
    All arrays float32."""
    name: str
    B: int
    D: int
    L: int
    M: int
    tau: tuple = (16.0, 4096.0)
    sigma: float = 0.1
    seed: int = 0

    def with_(self, **kw) -> "StackWorkload":
        return dataclasses.replace(self, **kw)


STACKS = {
    # small: every output checkable against the full oracle in seconds
    "stack-m3-d32-l1k": StackWorkload("stack-m3-d32-l1k", 2, 32, 1024, 3),
    # the smallest point of the pages' Hyena sweep (M = 18, D = 256, L = 2^15)
    "stack-m18-d256-l32k": StackWorkload("stack-m18-d256-l32k", 1, 256, 32768, 18),
}


def get_stack(name: str) -> StackWorkload:
    return STACKS[name]


def make_stack_filters(w: StackWorkload) -> np.ndarray:
    """rho[M][L][D] (float32)."""
    rho = np.empty((w.M, w.L, w.D), dtype=np.float32)
    lo, hi = w.tau
    j_all = np.arange(w.L, dtype=np.float64)
    for l in range(w.M):
        rng = np.random.default_rng([w.seed, 10, l])
        taus = np.exp(rng.uniform(math.log(lo), math.log(hi), size=w.D))
        norm = 1.0 / np.sqrt(np.sum(np.exp(-2.0 * j_all[:, None] / taus[None, :]), axis=0))
        for r0 in range(0, w.L, _ROWS):
            r1 = min(w.L, r0 + _ROWS)
            g = rng.standard_normal((r1 - r0, w.D), dtype=np.float32)
            env = np.exp(-j_all[r0:r1, None] / taus[None, :]) * norm[None, :]
            rho[l, r0:r1] = (g.astype(np.float64) * env).astype(np.float32)
    return rho


def make_stack_weights(w: StackWorkload):
    """(W1[M][D][D], W2[M][D][D]) float32, N(0, 1/D)."""
    out = []
    for k in (11, 12):
        rng = np.random.default_rng([w.seed, k])
        W = np.empty((w.M, w.D, w.D), dtype=np.float32)
        for l in range(w.M):
            W[l] = (rng.standard_normal((w.D, w.D), dtype=np.float32).astype(np.float64)
                    * math.sqrt(1.0 / w.D)).astype(np.float32)
        out.append(W)
    return out[0], out[1]


def make_stack_x0(w: StackWorkload) -> np.ndarray:
    return np.random.default_rng([w.seed, 13]).standard_normal((w.B, w.D), dtype=np.float32)


def make_stack_noise(w: StackWorkload) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 14])
    nz = np.empty((w.B, w.L, w.D), dtype=np.float32)
    for b in range(w.B):
        for r0 in range(0, w.L, _ROWS):
            r1 = min(w.L, r0 + _ROWS)
            nz[b, r0:r1] = rng.standard_normal((r1 - r0, w.D), dtype=np.float32)
    return nz
