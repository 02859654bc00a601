"""CPU-only checks of the C ABI: the library loads and exports every symbol
include/fi.h declares, arguments are validated before any device work, and the
schedule helper reproduces the relaxed tiling of the page "Flash Inference:
Inferenza in Tempo Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga
e Oltre", section "Strategia di Tiling (Algoritmo 1)"."""
import ctypes
import json
import os
import re

import pytest

import exact_online_amd as fi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "fi.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fi_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(fi.EXPORTS), names
    for n in names:
        assert hasattr(fi.lib, n), n


def test_strerror_and_null_handles():
    for code in (fi.FI_OK, fi.FI_ERR_INVALID, fi.FI_ERR_NOMEM, fi.FI_ERR_HIP,
                 fi.FI_ERR_STATE, fi.FI_ERR_UNSUPPORTED, -99):
        assert isinstance(fi.fi_strerror(code), str) and fi.fi_strerror(code)
    assert fi.fi_position(None) == -1
    fi.fi_destroy(None)  # no-op
    assert fi.lib.fi_step(None, 1, 1) == fi.FI_ERR_INVALID
    assert fi.lib.fi_run_closed_loop(None, 1, 1, 1, None) == fi.FI_ERR_INVALID
    assert fi.lib.fi_run_prompted(None, 1, 1, 1, None) == fi.FI_ERR_INVALID
    assert fi.lib.fi_reset(None) == fi.FI_ERR_INVALID


def _create_status(cfg, h=0x1000):
    out = ctypes.c_void_p(123)
    st = fi.lib.fi_create(ctypes.byref(cfg) if cfg is not None else None, h, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw", [
    dict(B=0, D=4, L=16), dict(B=1, D=0, L=16), dict(B=1, D=4, L=0), dict(B=-1, D=4, L=16),
    dict(B=1, D=4, L=16, io_dtype=2), dict(B=1, D=4, L=16, small_tile_max=96),
    dict(B=1, D=4, L=16, small_tile_max=32), dict(B=1, D=4, L=16, small_tile_max=512),
    dict(B=1 << 31, D=4, L=16), dict(B=1 << 20, D=1 << 20, L=1 << 20),
])
def test_create_rejects_invalid(kw):
    st, out = _create_status(fi.make_config(**kw))
    assert st == fi.FI_ERR_INVALID
    assert out is None


def test_create_rejects_null():
    assert _create_status(None)[0] == fi.FI_ERR_INVALID
    assert _create_status(fi.make_config(1, 4, 16), h=0)[0] == fi.FI_ERR_INVALID
    cfg = fi.make_config(1, 4, 16)
    assert fi.lib.fi_create(ctypes.byref(cfg), 0x1000, None) == fi.FI_ERR_INVALID


def test_create_rejects_too_long_filter():
    # valid sizes beyond the supported length: unsupported, with or without a GPU
    st, out = _create_status(fi.make_config(1, 4, fi.FI_MAX_L + 1))
    assert st == fi.FI_ERR_UNSUPPORTED and out is None


def test_create_without_gpu_is_unsupported():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, out = _create_status(fi.make_config(1, 4, 16))
    assert st == fi.FI_ERR_UNSUPPORTED and out is None


# --------------------------------------------------------------- schedule
def _tiles(L):
    return [fi.fi_tile_at(L, i) for i in range(1, L)]


@pytest.mark.parametrize("L", [2, 3, 8, 16, 64, 100, 1000, 1024])
def test_schedule_exact_cover(L):
    """Every pair s < t is added by exactly one tile, and a tile only reads
    completed positions and writes positions not yet produced."""
    cover = {}
    for i, t in enumerate(_tiles(L), start=1):
        assert t.in_hi == i and t.out_lo == i and t.U == (i & -i)
        assert t.in_lo == i - t.U and t.out_hi == min(i + t.U, L)
        for s in range(t.in_lo, t.in_hi):
            for o in range(t.out_lo, t.out_hi):
                cover[(s, o)] = cover.get((s, o), 0) + 1
    want = {(s, o) for o in range(L) for s in range(o)}
    assert set(cover) == want
    assert all(v == 1 for v in cover.values())


def test_schedule_counts_match_the_page():
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "schedule_facts.json")))["facts"]
    P = 14
    L = 1 << P
    tiles = _tiles(L)
    assert len(tiles) == L - 1                                   # L-1 invocations
    for q in range(P):
        assert sum(t.U == (1 << q) for t in tiles) == 1 << (P - 1 - q)   # 2^(P-1-q)
    f4 = sum(t.U <= 4 for t in tiles) / len(tiles)
    f8 = sum(t.U <= 8 for t in tiles) / len(tiles)
    assert abs(f4 - facts[2]["value"]) < 1e-3
    assert abs(f8 - facts[3]["value"]) < 1e-3


def test_tile_at_rejects_out_of_range():
    t = fi.fi_tile()
    for L, i in [(1, 1), (16, 0), (16, 16), (16, -1)]:
        assert fi.lib.fi_tile_at(L, i, ctypes.byref(t)) == fi.FI_ERR_INVALID
    assert fi.lib.fi_tile_at(16, 3, None) == fi.FI_ERR_INVALID


# ------------------------------------------------------------------ bench
def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_algorithmic_bytes():
    # D=1024, L=16K, fp32, closed loop, T=128: the per-pass figure the
    # roofline divides by; a prompt of 8192 feeds back only the later half
    import bench
    assert bench.algorithmic_bytes(1, 1024, 16384, 4, 4, 128, True) == 2550915072
    assert bench.algorithmic_bytes(1, 1024, 16384, 4, 4, 128, True, 16384 - 8192) == 2550915072 - 1024 * 8192 * 4
    assert bench.algorithmic_bytes(1, 1024, 16384, 4, 4, 128, False) == 2550915072 - 1024 * 16384 * 4


def test_config_layout_matches_the_header(tmp_path):
    """The binding's fi_config has the C struct's size and field offsets, and
    the enum types are int-sized (a C compiler reads include/fi.h)."""
    import subprocess
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "fi.h"\n'
        'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(fi_config),'
        ' offsetof(fi_config, B), offsetof(fi_config, D), offsetof(fi_config, L),'
        ' offsetof(fi_config, io_dtype), offsetof(fi_config, stream),'
        ' offsetof(fi_config, small_tile_max), sizeof(fi_dtype), sizeof(fi_feedback)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True, capture_output=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    C = fi.fi_config
    want = [ctypes.sizeof(C), C.B.offset, C.D.offset, C.L.offset, C.io_dtype.offset, C.stream.offset,
            C.small_tile_max.offset, 4, 4]
    assert got == want


def test_run_rejects_unknown_feedback():
    # the handle is checked first; an unknown feedback value is rejected before
    # any device work even with a handle (checked on the GPU in the state tests)
    assert fi.lib.fi_run_closed_loop(None, 1, 7, 1, None) == fi.FI_ERR_INVALID


def test_bench_oracle_sample_sizes():
    """The oracle's timed sample: whole workloads when they fit the budget,
    else every thread's worth of channels over a power-of-two prefix."""
    import bench
    B = bench.ORACLE_BUDGET_MACS
    assert bench.oracle_sample(16, 1024, 16) == (16, 1024)            # small mixer: whole
    assert bench.oracle_sample(1024, 16384, 16) == (1024, 16384)      # D=1024, L=16K: whole
    n, lp = bench.oracle_sample(16384, 65536, 16)
    assert n == 256 and lp == 32768 and n * lp * (lp + 1) / 2 <= B
    n, lp = bench.oracle_sample(768, 1 << 20, 16)
    assert n == 256 and lp < (1 << 20) and n * lp * (lp + 1) / 2 <= B < n * (2 * lp) * (2 * lp + 1) / 2


def test_bench_cpu_baseline_small_mixer():
    import bench
    import workloads
    w = workloads.get("mixer-d16-l1k")
    h = workloads.make_filter(w)
    for closed, x in ((True, workloads.make_x0(w)), (False, workloads.make_x(w))):
        cb = bench.cpu_baseline(w, h, x, closed)
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["seconds"] > 0
        assert cb["cores"] == 1 and cb["host_cpus"] >= 1 and cb["cpu_model"]
        assert ("closed loop" if closed else "open loop") in cb["sample"]
        assert "16 of 16 channels" in cb["sample"] and "[0, 1024) of 1024" in cb["sample"]


def test_stack_config_layout_matches_the_header(tmp_path):
    import subprocess
    src = tmp_path / "layout_stack.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "fi.h"\n'
        'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(fi_stack_config),'
        ' offsetof(fi_stack_config, B), offsetof(fi_stack_config, D), offsetof(fi_stack_config, L),'
        ' offsetof(fi_stack_config, M), offsetof(fi_stack_config, act), offsetof(fi_stack_config, stream),'
        ' offsetof(fi_stack_config, small_tile_max)); return 0; }\n')
    exe = tmp_path / "layout_stack"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True, capture_output=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    C = fi.fi_stack_config
    assert got == [ctypes.sizeof(C), C.B.offset, C.D.offset, C.L.offset, C.M.offset, C.act.offset,
                   C.stream.offset, C.small_tile_max.offset]


@pytest.mark.parametrize("kw", [dict(M=0), dict(act=3), dict(B=0), dict(D=0), dict(L=0)])
def test_stack_create_rejects_invalid(kw):
    base = dict(B=1, D=4, L=16, M=2, act=0, stream=None, small_tile_max=0)
    base.update(kw)
    cfg = fi.fi_stack_config(**base)
    out = ctypes.c_void_p(123)
    st = fi.lib.fi_stack_create(ctypes.byref(cfg), 0x1000, 0x1000, 0x1000, ctypes.byref(out))
    assert st == fi.FI_ERR_INVALID and out.value is None
    assert fi.lib.fi_stack_run(None, 1, None, 0.0, 1, None) == fi.FI_ERR_INVALID
    fi.fi_stack_destroy(None)
