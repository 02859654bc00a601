"""GPU parity, element by element, on every route of the FFT tile and of the
online interface fi_step, through the C ABI.

Delta filters h = delta_k give the closed form y[t] = x[t-k] (0 for t < k):
each channel's one nonzero tap sits on or next to a tile side, so every
level's transform moves the data exactly once at a known place, and a
mistake at one tile boundary or in one pass shows at the positions it
reaches.  Routes covered here:
 * fi_step (one position per call): the fused red cell + direct tile for
   U <= T (T = 64 and T = 256), the FFT tiles of k_tile_fft from global
   memory at 2048 and 4096 points, the two-LDS-half 8192-point tile and the
   global-scratch passes at 16384 points;
 * the persistent pass at L = 2^17 (tiles up to 65536 points: the fused
   first/last global passes, the radix-8/4 global stages and the paired-block
   untangle) and at L = 2^20 (tiles up to 2^19 points).
Tolerance: 2e-5 absolute per element (|x| < 6, FFT rounding of a unit tap);
fi_step exact below its first FFT tile; the persistent pass (open loop here)
within 2^-21 relative up to 1024: there every contribution is a matrix-core
block product of fp16 halves (the block's own triangle, the tiles of side
256 and 512).  A random filter through fi_step at L = 2^15
is compared with the oracle (relative L2 <= 1e-5 overall and per channel).
"""
import numpy as np
import pytest

import oracle
import workloads
from fi_harness import gpu_run, gpu_steps, host, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import exact_online_amd as fi  # noqa: E402  (fails loudly if libfi.so is missing)


def _delta_case(L, ks, seed, run):
    D = len(ks)
    h = np.zeros((L, D), np.float32)
    for c, k in enumerate(ks):
        h[k, c] = 1.0
    x = np.random.default_rng(seed).standard_normal((1, L, D)).astype(np.float32)
    y = host(run(to_dev(h, "f32"), D, to_dev(x, "f32")))
    return x, y


def _check_delta(x, y, ks, exact_below, tol=2e-5, close_below=0):
    """Every position within tol; exact below exact_below; below close_below
    (the reach of the persistent pass's fp16-half block products) within
    2^-21 of |x| plus a floor of 2^-30 of the largest |x|."""
    L = x.shape[1]
    for c, k in enumerate(ks):
        ref = np.zeros(L)
        ref[k:] = x[0, :L - k, c]
        err = np.abs(y[0, :, c] - ref)
        bad = np.nonzero(err > tol)[0]
        assert bad.size == 0, (k, int(bad[0]), float(err.max()))
        assert np.array_equal(y[0, :exact_below, c], ref[:exact_below].astype(np.float32)), k
        if close_below:
            # x = hi + lo + r, |r| <= 2^-22 |x|, or an absolute 2^-24 of the
            # scaled block (2^-37 of its largest |x|) where lo is subnormal
            bound = 2.0 ** -21 * np.abs(ref[:close_below]) + 2.0 ** -30 * np.abs(x[0, :close_below, c]).max()
            assert (err[:close_below] <= bound).all(), k


@pytest.mark.parametrize("T", [64, 256])
def test_fi_step_fft_routes_delta(T):
    """fi_step at L = 2^15: every tile level up to 16384 points, one call per
    position; with T = 256 the tiles of side 256 are direct (k_step_tile)."""
    L = 1 << 15
    ks = [1, 2, T - 1, T, T + 1, 2 * T - 1, 2 * T, 1023, 1024, 2047, 2048, 2049, 3000, 4095, 4096, 4097,
          6000, 8191, 8192, 8193, 12000, 16383, 16384, 16385, 24576, 32767]
    log("case fi_step delta filters L=32768 T", T)
    x, y = _delta_case(L, ks, 21 + T, lambda hd, D, xd: gpu_steps(hd, 1, D, L, "f32", xd, T))
    _check_delta(x, y, ks, exact_below=2 * T)


def test_fi_step_random_filter_against_oracle():
    """A decaying-Gaussian filter through fi_step at L = 2^15 (every FFT level
    of the per-step path, including the global-scratch 16384-point tile),
    against the oracle: relative L2 <= 1e-5 overall and on every channel."""
    w = workloads.get("hyena-d1024-l16k").with_(B=2, D=3, L=1 << 15, seed=7)
    h = workloads.make_filter(w)
    x = workloads.make_x(w)
    log("case fi_step random filter L=32768")
    y = host(gpu_steps(to_dev(h, "f32"), w.B, w.D, w.L, "f32", to_dev(x, "f32"), 0))
    ref = oracle.default().conv_open(h, x)
    err = rel_l2(y, ref)
    per = [rel_l2(y[b, :, c], ref[b, :, c]) for b in range(w.B) for c in range(w.D)]
    log("rel l2", err, "worst channel", max(per))
    assert err <= 1e-5
    assert max(per) <= 1e-5


def test_persistent_delta_l128k():
    """The persistent pass at L = 2^17: k on and around every level from
    8192 to 65536 points, checked at every position."""
    L = 1 << 17
    ks = [1, 255, 256, 257, 511, 512, 4095, 4096, 8191, 8192, 8193, 12288, 16383, 16384, 16385, 20000,
          24576, 32767, 32768, 32769, 40000, 49152, 65535, 65536, 65537, 81920, 98304, 114688, 131071]
    log("case persistent delta filters L=131072")
    x, y = _delta_case(L, ks, 31, lambda hd, D, xd: gpu_run(hd, 1, D, L, "f32", xd, closed=False,
                                                              want_x=False)[0])
    _check_delta(x, y, ks, exact_below=0, close_below=1024)


def test_persistent_delta_l1m():
    """The persistent pass at L = 2^20 (tiles up to 2^19 points through the
    global-scratch passes), every position of six channels."""
    L = 1 << 20
    ks = [1, 131071, 262144, 524287, 524288, 1048575]
    log("case persistent delta filters L=1048576")
    x, y = _delta_case(L, ks, 41, lambda hd, D, xd: gpu_run(hd, 1, D, L, "f32", xd, closed=False,
                                                              want_x=False)[0])
    _check_delta(x, y, ks, exact_below=0, tol=4e-5, close_below=1024)


def test_create_out_of_device_memory():
    """Sizes that pass every overflow check but need about 1 TiB of device
    memory: fi_create returns FI_ERR_NOMEM and leaves nothing allocated; a
    handle created afterwards works (the failed allocation leaves no error
    behind for later calls)."""
    h = torch.zeros((16, 4), dtype=torch.float32, device="cuda")
    cfg = fi.make_config(1, 1 << 14, 1 << 24, fi.FI_F32, 0, torch.cuda.current_stream())
    log("case fi_create out of memory")
    with pytest.raises(fi.FiError) as e:
        fi.fi_create(cfg, h)
    assert e.value.status == fi.FI_ERR_NOMEM
    w = workloads.get("mixer-d16-l1k").with_(D=4, L=16)
    hd = to_dev(workloads.make_filter(w), "f32")
    xd = to_dev(workloads.make_x(w), "f32")
    y, _ = gpu_run(hd, 1, 4, 16, "f32", xd, closed=False, want_x=False)
    ref = oracle.default().conv_open(workloads.make_filter(w), workloads.make_x(w))
    assert rel_l2(host(y), ref) <= 1e-6
