"""exact_online_amd -- exact online causal long convolution on AMD MI355X.

Thin ctypes binding over the C ABI of ``include/fi.h`` (``libfi.so``, HIP for
gfx950).  The functions keep the C names and only marshal arguments: device
pointers may be given as integers or as torch CUDA tensors, streams as
integers (hipStream_t) or torch streams.  Every step of the computation runs
in the library's HIP kernels; if ``libfi.so`` is missing this module raises at
import (build it with ``python exact_online_amd/build.py`` or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

__all__ = [
    "FI_F32", "FI_BF16", "FI_FEEDBACK_NONE", "FI_FEEDBACK_TANH",
    "FI_OK", "FI_ERR_INVALID", "FI_ERR_NOMEM", "FI_ERR_HIP", "FI_ERR_STATE", "FI_ERR_UNSUPPORTED",
    "FiError", "fi_config", "fi_tile", "fi_create", "fi_step", "fi_run_closed_loop", "fi_reset",
    "fi_destroy", "fi_position", "fi_strerror", "fi_tile_at", "fi_run_prompted", "fi_conv_static", "Mixer",
    "fi_stack_config", "fi_stack_create", "fi_stack_run", "fi_stack_destroy", "Stack", "EXPORTS", "lib",
    "LIB_PATH",
]

FI_F32, FI_BF16 = 0, 1
FI_FEEDBACK_NONE, FI_FEEDBACK_TANH = 0, 1
FI_DEFAULT_SMALL_TILE_MAX = 64
FI_MAX_L = 1 << 25
FI_OK, FI_ERR_INVALID, FI_ERR_NOMEM, FI_ERR_HIP, FI_ERR_STATE, FI_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5

# EXACT_ONLINE_AMD_LIB may name another build of the same library (the
# phase-timing build libfi_prof.so, for bench.py --phases)
LIB_PATH = Path(os.environ.get("EXACT_ONLINE_AMD_LIB") or Path(__file__).resolve().parent / "libfi.so")
if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is not built: run `python exact_online_amd/build.py` "
                      "(hipcc, gfx950) before using exact_online_amd")

# PyTorch, when installed, carries its own HIP runtime (same soname as the
# system one this library links).  Loaded first, torch's runtime is the one
# the library binds to, so the process has one runtime; the other order
# loads two, and whichever owns the device leaves the other without it.
try:
    import torch  # noqa: F401
except ImportError:
    pass

lib = ctypes.CDLL(str(LIB_PATH))

# every symbol include/fi.h declares
EXPORTS = ("fi_create", "fi_step", "fi_run_closed_loop", "fi_run_prompted", "fi_reset", "fi_destroy",
           "fi_position", "fi_strerror", "fi_tile_at", "fi_conv_static", "fi_stack_create", "fi_stack_run",
           "fi_stack_destroy")
FI_ACT_GELU, FI_ACT_TANH, FI_ACT_IDENTITY = 0, 1, 2
FI_STATIC_WORKSPACE_BYTES = 64 << 20


class fi_config(ctypes.Structure):
    # io_dtype is the C enum fi_dtype (int-sized)
    _fields_ = [("B", ctypes.c_int64), ("D", ctypes.c_int64), ("L", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("stream", ctypes.c_void_p),
                ("small_tile_max", ctypes.c_int32)]


class fi_stack_config(ctypes.Structure):
    # act is the C enum fi_activation (int-sized)
    _fields_ = [("B", ctypes.c_int64), ("D", ctypes.c_int64), ("L", ctypes.c_int64), ("M", ctypes.c_int64),
                ("act", ctypes.c_int32), ("stream", ctypes.c_void_p), ("small_tile_max", ctypes.c_int32)]


class fi_tile(ctypes.Structure):
    _fields_ = [("U", ctypes.c_int64), ("in_lo", ctypes.c_int64), ("in_hi", ctypes.c_int64),
                ("out_lo", ctypes.c_int64), ("out_hi", ctypes.c_int64)]


_H = ctypes.c_void_p
lib.fi_create.argtypes = [ctypes.POINTER(fi_config), ctypes.c_void_p, ctypes.POINTER(_H)]
lib.fi_create.restype = ctypes.c_int
lib.fi_step.argtypes = [_H, ctypes.c_void_p, ctypes.c_void_p]
lib.fi_step.restype = ctypes.c_int
lib.fi_run_closed_loop.argtypes = [_H, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
lib.fi_run_closed_loop.restype = ctypes.c_int
lib.fi_run_prompted.argtypes = [_H, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
lib.fi_run_prompted.restype = ctypes.c_int
lib.fi_reset.argtypes = [_H]
lib.fi_reset.restype = ctypes.c_int
lib.fi_destroy.argtypes = [_H]
lib.fi_destroy.restype = None
lib.fi_position.argtypes = [_H]
lib.fi_position.restype = ctypes.c_int64
lib.fi_strerror.argtypes = [ctypes.c_int]
lib.fi_strerror.restype = ctypes.c_char_p
lib.fi_tile_at.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(fi_tile)]
lib.fi_tile_at.restype = ctypes.c_int
lib.fi_conv_static.argtypes = [ctypes.POINTER(fi_config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p]
lib.fi_conv_static.restype = ctypes.c_int
lib.fi_stack_create.argtypes = [ctypes.POINTER(fi_stack_config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.POINTER(_H)]
lib.fi_stack_create.restype = ctypes.c_int
lib.fi_stack_run.argtypes = [_H, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
lib.fi_stack_run.restype = ctypes.c_int
lib.fi_stack_destroy.argtypes = [_H]
lib.fi_stack_destroy.restype = None
# only in the phase-timing build (include/fi_profile.h)
HAS_PROFILE = hasattr(lib, "fi_profile_read")
if HAS_PROFILE:
    lib.fi_profile_read.argtypes = [_H, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64]
    lib.fi_profile_read.restype = ctypes.c_int64


class FiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {fi_strerror(status)} ({status})")


def _check(status: int, where: str) -> int:
    if status < 0:
        raise FiError(status, where)
    return status


def _ptr(x) -> int:
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int:
    if s is None:
        return 0
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def fi_strerror(status: int) -> str:
    return lib.fi_strerror(int(status)).decode()


def fi_create(cfg: fi_config, h) -> int:
    """Returns the handle (an integer); raises FiError on failure."""
    out = _H()
    _check(lib.fi_create(ctypes.byref(cfg), _ptr(h), ctypes.byref(out)), "fi_create")
    return int(out.value)


def fi_step(s: int, x_t, y_t) -> None:
    _check(lib.fi_step(s, _ptr(x_t), _ptr(y_t)), "fi_step")


def fi_run_closed_loop(s: int, x_in, fb: int, y, x_out=None) -> None:
    _check(lib.fi_run_closed_loop(s, _ptr(x_in), int(fb), _ptr(y), _ptr(x_out)), "fi_run_closed_loop")


def fi_run_prompted(s: int, x_prompt, p: int, y, x_out=None) -> None:
    _check(lib.fi_run_prompted(s, _ptr(x_prompt), int(p), _ptr(y), _ptr(x_out)), "fi_run_prompted")


def fi_reset(s: int) -> None:
    _check(lib.fi_reset(s), "fi_reset")


def fi_destroy(s) -> None:
    lib.fi_destroy(s)


def fi_position(s) -> int:
    return int(lib.fi_position(s))


def fi_tile_at(L: int, i: int) -> fi_tile:
    t = fi_tile()
    _check(lib.fi_tile_at(int(L), int(i), ctypes.byref(t)), "fi_tile_at")
    return t


def fi_conv_static(cfg: fi_config, h, x_in, fb: int, y, x_out=None) -> None:
    """The no-allocation one-shot run (fixed per-device workspace)."""
    _check(lib.fi_conv_static(ctypes.byref(cfg), _ptr(h), _ptr(x_in), int(fb), _ptr(y), _ptr(x_out)),
           "fi_conv_static")


def fi_stack_create(cfg: fi_stack_config, rho, w1, w2) -> int:
    out = _H()
    _check(lib.fi_stack_create(ctypes.byref(cfg), _ptr(rho), _ptr(w1), _ptr(w2), ctypes.byref(out)),
           "fi_stack_create")
    return int(out.value)


def fi_stack_run(s: int, x0, noise, sigma: float, y, x_out=None) -> None:
    _check(lib.fi_stack_run(s, _ptr(x0), _ptr(noise), float(sigma), _ptr(y), _ptr(x_out)), "fi_stack_run")


def fi_stack_destroy(s) -> None:
    lib.fi_stack_destroy(s)


class Stack:
    """Owning wrapper of one layer stack (marshalling only)."""

    def __init__(self, B, D, L, M, rho, w1, w2, act=FI_ACT_GELU, small_tile_max=0, stream=None):
        self.cfg = fi_stack_config(B=int(B), D=int(D), L=int(L), M=int(M), act=int(act), stream=_stream(stream),
                                   small_tile_max=int(small_tile_max))
        self.handle = fi_stack_create(self.cfg, rho, w1, w2)

    def run(self, x0, y, x_out=None, noise=None, sigma=0.0):
        fi_stack_run(self.handle, x0, noise, sigma, y, x_out)

    def close(self):
        if self.handle:
            fi_stack_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fi_profile_read(s: int):
    """Phase-timing build only: the last pass's record (a list of ints)."""
    if not HAS_PROFILE:
        raise RuntimeError(f"{LIB_PATH} is not the phase-timing build (libfi_prof.so)")
    n = _check(int(lib.fi_profile_read(s, (ctypes.c_uint64 * 1)(), 0)), "fi_profile_read")
    buf = (ctypes.c_uint64 * max(n, 1))()
    _check(int(lib.fi_profile_read(s, buf, n)), "fi_profile_read")
    return list(buf[:n])


def make_config(B: int, D: int, L: int, io_dtype: int = FI_F32, small_tile_max: int = 0,
                stream=None) -> fi_config:
    return fi_config(B=int(B), D=int(D), L=int(L), io_dtype=int(io_dtype), stream=_stream(stream),
                     small_tile_max=int(small_tile_max))


class Mixer:
    """Owning wrapper of one handle (marshalling only)."""

    def __init__(self, B, D, L, h, io_dtype=FI_F32, small_tile_max=0, stream=None):
        self.cfg = make_config(B, D, L, io_dtype, small_tile_max, stream)
        self.B, self.D, self.L = int(B), int(D), int(L)
        self.handle = fi_create(self.cfg, h)

    def step(self, x_t, y_t):
        fi_step(self.handle, x_t, y_t)

    def run(self, x_in, fb, y, x_out=None):
        fi_run_closed_loop(self.handle, x_in, fb, y, x_out)

    def run_prompted(self, x_prompt, p, y, x_out=None):
        fi_run_prompted(self.handle, x_prompt, p, y, x_out)

    def reset(self):
        fi_reset(self.handle)

    @property
    def position(self) -> int:
        return fi_position(self.handle)

    def close(self):
        if self.handle:
            fi_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
