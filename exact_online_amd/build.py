"""Build libfi.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libfi.so"
PROFILE_LIB = PKG / "libfi_prof.so"   # the phase-timing build (-DFI_PROFILE=1), for bench.py --phases
SOURCES = [CSRC / "fi_kernels.hip", CSRC / "fi_api.cpp"]
HEADERS = [ROOT / "include" / "fi.h", ROOT / "include" / "fi_profile.h", CSRC / "fi_internal.h",
           CSRC / "fi_device.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = False, out: Path | None = None, extra: list | None = None) -> Path:
    out = Path(out) if out is not None else LIB
    tmp = out.with_suffix(".so.tmp")
    cmd = [HIPCC, *FLAGS, *(extra or []), f"-I{ROOT / 'include'}", f"-I{CSRC}",
           "-o", str(tmp), *map(str, SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libfi.so")
    if verbose and r.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        noise = "'-packed-fp32-ops' is not a recognized feature"
        rest = [ln for ln in r.stderr.splitlines() if noise not in ln]
        if rest:
            sys.stderr.write("\n".join(rest) + "\n")
    os.replace(tmp, out)
    return out


def build_profile(verbose: bool = False) -> Path:
    """The phase-timing library (not loaded by the product path)."""
    return build(verbose, out=PROFILE_LIB, extra=["-DFI_PROFILE=1"])


def is_stale(lib: Path = LIB) -> bool:
    if not lib.exists():
        return True
    t = lib.stat().st_mtime
    return any(p.stat().st_mtime > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    if "--profile" in sys.argv[1:]:
        print(build_profile(verbose=True))
    else:
        build(verbose=True)
        print(LIB)
