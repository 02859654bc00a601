"""CPU oracle for the exact online causal long convolution (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product package never imports
it.  The arithmetic lives in ``fi_oracle.c`` (plain fp64 brute force, OpenMP
over channels); this module only builds it with gcc and marshals numpy arrays.

Every function is the plain definition of the page "Flash Inference:
Inferenza in Tempo Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga
e Oltre", section "Definizione del Compito" (z_t = sum_{i<=t} y_i rho_{t-i}),
restated 0-indexed as y[t] = sum_{s<=t} h[t-s] x[s], per channel.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "fi_oracle.c"
_LIB = _HERE / "libfi_oracle.so"
_lib = None


def build(out: Path | None = None, mutant: int = 0, quiet: bool = True) -> Path:
    """Compile fi_oracle.c with gcc (-fopenmp).  ``mutant`` plants a mistake
    (only for the oracle's own mutation tests)."""
    out = Path(out) if out is not None else _LIB
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           f"-DFIO_MUTANT={int(mutant)}", "-o", str(out), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    return out


def _bind(lib):
    i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_int
    lib.fio_open.argtypes = [i64, i64, i64, dp, dp, dp, ip]
    lib.fio_open.restype = None
    lib.fio_closed.argtypes = [i64, i64, i64, dp, dp, dp, ip, ip]
    lib.fio_closed.restype = None
    lib.fio_prompted.argtypes = [i64, i64, i64, i64, dp, dp, dp, ip, ip]
    lib.fio_prompted.restype = None
    lib.fio_points.argtypes = [i64, dp, dp, i64, ctypes.POINTER(ctypes.c_int64), dp]
    lib.fio_points.restype = None
    lib.fio_round_bf16.argtypes = [ctypes.c_double]
    lib.fio_round_bf16.restype = ctypes.c_double
    lib.fio_stack.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, dp, ctypes.c_double, ip, ip, dp, dp, ip]
    lib.fio_stack.restype = None
    lib.fio_mutant.argtypes = []
    lib.fio_mutant.restype = ctypes.c_int
    return lib


def load(path: Path | None = None):
    """Load the oracle library (building it when missing or older than its source)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(str(path)))
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        _lib = _bind(ctypes.CDLL(str(_LIB)))
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """Thin numpy front end over one loaded oracle library."""

    def __init__(self, lib=None, threads: int | None = None):
        self.lib = lib if lib is not None else load()
        self.threads = default_threads() if threads is None else int(threads)

    def conv_open(self, h, x) -> np.ndarray:
        """h[L][D], x[B][L][D] (or x[L][D]) -> y, same shape as x, fp64."""
        h = _f64(h)
        x = _f64(x)
        squeeze = x.ndim == 2
        if squeeze:
            x = x[None]
        B, L, D = x.shape
        assert h.shape == (L, D), (h.shape, x.shape)
        y = np.empty_like(x)
        self.lib.fio_open(B, D, L, _p(h), _p(x), _p(y), self.threads)
        return y[0] if squeeze else y

    def conv_closed(self, h, x0, L: int | None = None, bf16: bool = False):
        """Free-running closed loop x_{t+1} = tanh(y_t).  h[L][D], x0[B][D]
        -> (y[B][L][D], x[B][L][D]) in fp64; ``bf16`` rounds the fed-back x."""
        h = _f64(h)
        L = h.shape[0] if L is None else int(L)
        h = np.ascontiguousarray(h[:L])
        x0 = _f64(x0)
        squeeze = x0.ndim == 1
        if squeeze:
            x0 = x0[None]
        B, D = x0.shape
        assert h.shape == (L, D)
        x = np.zeros((B, L, D), dtype=np.float64)
        x[:, 0, :] = x0
        y = np.empty_like(x)
        self.lib.fio_closed(B, D, L, _p(h), _p(x), _p(y), int(bool(bf16)), self.threads)
        if squeeze:
            return y[0], x[0]
        return y, x

    def conv_prompted(self, h, prompt, L: int | None = None, bf16: bool = False):
        """Prompt, then free-running: x[s] = prompt[s] for s < p, x_{t+1} =
        tanh(y_t) from position p on.  h[L][D], prompt[B][p][D] -> (y[B][L][D],
        x[B][L][D]) in fp64; ``bf16`` rounds the fed-back x."""
        h = _f64(h)
        L = h.shape[0] if L is None else int(L)
        h = np.ascontiguousarray(h[:L])
        prompt = _f64(prompt)
        squeeze = prompt.ndim == 2
        if squeeze:
            prompt = prompt[None]
        B, P, D = prompt.shape
        assert h.shape == (L, D) and 1 <= P <= L
        x = np.zeros((B, L, D), dtype=np.float64)
        x[:, :P, :] = prompt
        y = np.empty_like(x)
        self.lib.fio_prompted(B, D, L, P, _p(h), _p(x), _p(y), int(bool(bf16)), self.threads)
        if squeeze:
            return y[0], x[0]
        return y, x

    def conv_points(self, h_col, x_col, ts) -> np.ndarray:
        """One channel: y at positions ``ts`` from its filter and input series."""
        h_col = _f64(h_col)
        x_col = _f64(x_col)
        assert h_col.shape == x_col.shape and h_col.ndim == 1
        ts = np.ascontiguousarray(ts, dtype=np.int64)
        y = np.empty(ts.shape[0], dtype=np.float64)
        self.lib.fio_points(h_col.shape[0], _p(h_col), _p(x_col), ts.shape[0],
                            ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(y))
        return y

    ACTS = {"gelu": 0, "tanh": 1, "identity": 2}

    def conv_stack(self, rho, w1, w2, x, noise=None, sigma: float = 0.0, act: str = "gelu",
                   teacher_forced: bool = False):
        """The multi-layer stack (page "Flash Inference: Inferenza in Tempo
        Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga e Oltre",
        sections "Algoritmo di Inferenza LCSM (Algoritmo 2)" and
        "Configurazione Sperimentale": MLP + GELU blocks, a sampler adding
        noise).  rho[M][L][D], w1 and w2 [M][D][D] (row j = output j).
        teacher_forced: x[B][L][D] is the whole input sequence; otherwise
        x[B][D] (or x[B][L][D] with only x[:, 0] read) starts the feedback
        x[t+1] = a^M[t] + sigma noise[t].  Returns (y = a^M [B][L][D], x
        [B][L][D]) in fp64."""
        rho = _f64(rho)
        w1 = _f64(w1)
        w2 = _f64(w2)
        M, L, D = rho.shape
        assert w1.shape == (M, D, D) and w2.shape == (M, D, D)
        x = _f64(x)
        if x.ndim == 2:
            B = x.shape[0]
            xx = np.zeros((B, L, D))
            xx[:, 0, :] = x
        else:
            B = x.shape[0]
            assert x.shape == (B, L, D)
            xx = x.copy()
        nz = None
        if noise is not None:
            nz = _f64(noise)
            assert nz.shape == (B, L, D)
        y = np.empty((B, L, D))
        work = np.empty(B * ((M + 1) * L * D + 2 * D))
        self.lib.fio_stack(B, D, L, M, _p(rho), _p(w1), _p(w2), _p(xx),
                           _p(nz) if nz is not None else None, float(sigma), self.ACTS[act],
                           int(bool(teacher_forced)), _p(y), _p(work), self.threads)
        return y, xx

    def round_bf16(self, v) -> np.ndarray:
        v = np.asarray(v, dtype=np.float64)
        return np.vectorize(self.lib.fio_round_bf16, otypes=[np.float64])(v)

    @property
    def mutant(self) -> int:
        return int(self.lib.fio_mutant())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def conv_open(h, x):
    return default().conv_open(h, x)


def conv_closed(h, x0, L=None, bf16=False):
    return default().conv_closed(h, x0, L=L, bf16=bf16)


def conv_prompted(h, prompt, L=None, bf16=False):
    return default().conv_prompted(h, prompt, L=L, bf16=bf16)


def conv_points(h_col, x_col, ts):
    return default().conv_points(h_col, x_col, ts)


def round_bf16(v):
    return default().round_bf16(v)


def conv_stack(rho, w1, w2, x, noise=None, sigma=0.0, act="gelu", teacher_forced=False):
    return default().conv_stack(rho, w1, w2, x, noise, sigma, act, teacher_forced)
