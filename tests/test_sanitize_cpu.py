"""Sanitizer builds of the host code (CPU only, no GPU needed).

* The oracle (oracle/fi_oracle.c) with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, driven through every entry point on small
  inputs and edge arguments (tests/sanitize_oracle_driver.c).
* The library's host code (fi_api.cpp and the launch code in
  fi_kernels.hip) with clang's AddressSanitizer and UndefinedBehaviorSanitizer
  on the host side only (``-Xarch_host``; the device code is built as usual),
  loaded under the sanitizer runtime in a child process that calls every
  entry point a machine without a gfx950 device can reach: argument
  validation, size limits, error strings, the schedule helper, and the
  cleanup of a failed create.
Each child must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _no_report(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    for bad in ("AddressSanitizer", "runtime error", "LeakSanitizer"):
        assert bad not in out, out[-3000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", str(ROOT / "oracle" / "fi_oracle.c"),
           str(ROOT / "tests" / "sanitize_oracle_driver.c"), "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
    _no_report(r)
    assert r.stdout.startswith("checksum ")


PROBE = r'''
import ctypes, os, sys
lib = ctypes.CDLL(sys.argv[1])
INVALID, NOMEM, HIP, STATE, UNSUPPORTED = -1, -2, -3, -4, -5
lib.fi_strerror.restype = ctypes.c_char_p
for c in (0, -1, -2, -3, -4, -5, -6, 7, -2**31):
    assert lib.fi_strerror(c)
class cfg_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("D", ctypes.c_int64), ("L", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("stream", ctypes.c_void_p), ("small_tile_max", ctypes.c_int32)]
class stack_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("D", ctypes.c_int64), ("L", ctypes.c_int64), ("M", ctypes.c_int64),
                ("act", ctypes.c_int32), ("stream", ctypes.c_void_p), ("small_tile_max", ctypes.c_int32)]
class tile_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("U", "in_lo", "in_hi", "out_lo", "out_hi")]
P = ctypes.c_void_p(4096)          # a stand-in device pointer: never dereferenced on these paths
out = ctypes.c_void_p(1)
def create(*a):
    return lib.fi_create(ctypes.byref(cfg_t(*a)), P, ctypes.byref(out))
# argument checks
assert lib.fi_create(None, P, ctypes.byref(out)) == INVALID
assert lib.fi_create(ctypes.byref(cfg_t(1, 4, 16, 0, None, 0)), None, ctypes.byref(out)) == INVALID
assert lib.fi_create(ctypes.byref(cfg_t(1, 4, 16, 0, None, 0)), P, None) == INVALID
for bad in ((0, 4, 16, 0, None, 0), (1, 0, 16, 0, None, 0), (1, 4, 0, 0, None, 0), (-1, 4, 16, 0, None, 0),
            (1, 4, 16, 2, None, 0), (1, 4, 16, -7, None, 0), (1, 4, 16, 0, None, 32), (1, 4, 16, 0, None, 96),
            (1, 4, 16, 0, None, 512), (2**62, 2**62, 16, 0, None, 0), (1, 2**40, 2**40, 0, None, 0)):
    assert create(*bad) == INVALID, bad
    assert out.value is None
assert create(1, 4, 2**26, 0, None, 0) == UNSUPPORTED     # beyond FI_MAX_L
# valid sizes, no gfx950 device here: refused after validation, nothing left behind
for T in (0, 64, 128, 256):
    assert create(1, 4, 100, 1, None, T) in (UNSUPPORTED, HIP), T
# the environment's T, used only when the config leaves it 0
os.environ["FI_SMALL_TILE_MAX"] = "100"
assert create(1, 4, 100, 0, None, 0) == INVALID
assert create(1, 4, 100, 0, None, 128) in (UNSUPPORTED, HIP)
os.environ["FI_SMALL_TILE_MAX"] = "256"
assert create(1, 4, 100, 0, None, 0) in (UNSUPPORTED, HIP)
del os.environ["FI_SMALL_TILE_MAX"]
# NULL handles
lib.fi_position.restype = ctypes.c_int64
assert lib.fi_position(None) == -1
lib.fi_destroy(None)
lib.fi_stack_destroy(None)
assert lib.fi_reset(None) == INVALID
assert lib.fi_step(None, P, P) == INVALID
assert lib.fi_run_closed_loop(None, P, 1, P, None) == INVALID
assert lib.fi_run_prompted(None, P, ctypes.c_int64(3), P, None) == INVALID
assert lib.fi_stack_run(None, P, None, ctypes.c_float(0.0), P, None) == INVALID
# the entry point that allocates nothing
assert lib.fi_conv_static(None, P, P, 1, P, None) == INVALID
assert lib.fi_conv_static(ctypes.byref(cfg_t(0, 4, 16, 0, None, 0)), P, P, 1, P, None) == INVALID
assert lib.fi_conv_static(ctypes.byref(cfg_t(1, 4, 16, 0, None, 0)), P, P, 9, P, None) == INVALID
# the stack
sout = ctypes.c_void_p(1)
def screate(*a, rho=P):
    return lib.fi_stack_create(ctypes.byref(stack_t(*a)), rho, P, P, ctypes.byref(sout))
assert lib.fi_stack_create(None, P, P, P, ctypes.byref(sout)) == INVALID
assert screate(1, 4, 16, 2, 0, None, 0, rho=None) == INVALID
for bad in ((1, 4, 16, 0, 0, None, 0), (0, 4, 16, 2, 0, None, 0), (1, 4, 16, 2, 3, None, 0),
            (1, 4, 16, 2, -1, None, 0), (2**40, 4, 16, 2**40, 0, None, 0), (1, 4, 16, 2, 0, None, 48)):
    assert screate(*bad) == INVALID, bad
    assert sout.value is None
assert screate(1, 8193, 16, 2, 0, None, 0) == UNSUPPORTED           # D beyond a block's LDS vector
assert screate(1, 4, 2**24, 2**7, 0, None, 0) == UNSUPPORTED        # L M beyond the run's tags
assert screate(1, 4, 100, 3, 1, None, 0) in (UNSUPPORTED, HIP)
# the schedule helper
t = tile_t()
assert lib.fi_tile_at(ctypes.c_int64(16), ctypes.c_int64(12), ctypes.byref(t)) == 0
assert (t.U, t.in_lo, t.in_hi, t.out_lo, t.out_hi) == (4, 8, 12, 12, 16)
assert lib.fi_tile_at(ctypes.c_int64(100), ctypes.c_int64(96), ctypes.byref(t)) == 0 and t.out_hi == 100
for L, i in ((16, 0), (16, 16), (1, 0), (16, -3)):
    assert lib.fi_tile_at(ctypes.c_int64(L), ctypes.c_int64(i), ctypes.byref(t)) == INVALID
assert lib.fi_tile_at(ctypes.c_int64(16), ctypes.c_int64(3), None) == INVALID
print("probe ok")
'''


def _asan_runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = Path(r.stdout.strip())
    if p.is_file():
        return p
    hits = sorted(Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc missing")
def test_host_library_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is missing")
    sys.path.insert(0, str(ROOT / "exact_online_amd"))
    import build as fib
    lib = tmp_path / "libfi_asan.so"
    san = ["-O1", "-g"]
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    fib.build(out=lib, extra=san)
    probe = tmp_path / "probe.py"
    probe.write_text(PROBE)
    env = dict(os.environ, LD_PRELOAD=str(rt), ASAN_OPTIONS="detect_leaks=0")
    env.pop("FI_SMALL_TILE_MAX", None)
    r = subprocess.run([sys.executable, str(probe), str(lib)], capture_output=True, text=True, timeout=300,
                       env=env)
    _no_report(r)
    assert "probe ok" in r.stdout
