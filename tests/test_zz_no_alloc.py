"""fi_conv_static, the entry point that allocates nothing (a fixed per-device
workspace), through the C ABI: two calls in a row on one stream, the second
with a smaller problem than the first, each compared with the handle path
(fi_create + fi_run_closed_loop, which runs the same kernels: equal bit for
bit) and with the oracle (closed loop: max abs error <= 1e-3 against the
oracle fed the recorded inputs; open loop: relative L2 error <= 1e-5).  A
problem larger than the workspace is refused with FI_ERR_UNSUPPORTED."""
import numpy as np
import pytest

import oracle
import workloads
from fi_harness import gpu_run, host, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import exact_online_amd as fi  # noqa: E402  (fails loudly if libfi.so is missing)


def _static(w, closed, h_dev, x_dev):
    t = torch
    io = fi.FI_BF16 if w.dtype == "bf16" else fi.FI_F32
    y = t.empty((w.B, w.L, w.D), dtype=t.float32, device="cuda")
    xo = t.empty((w.B, w.L, w.D), dtype=t.bfloat16 if w.dtype == "bf16" else t.float32, device="cuda")
    cfg = fi.make_config(w.B, w.D, w.L, io, 0, t.cuda.current_stream())
    fi.fi_conv_static(cfg, h_dev, x_dev, fi.FI_FEEDBACK_TANH if closed else fi.FI_FEEDBACK_NONE, y, xo)
    return y, xo


def test_static_entry_two_calls_second_smaller():
    cases = [
        (workloads.get("hyena-d1024-l16k").with_(B=2, D=6, L=16384, seed=31), True),   # FFT scratch in use
        (workloads.get("mixer-d16-l1k").with_(B=1, D=5, L=700, seed=32), False),
    ]
    outs = []
    for w, closed in cases:
        h = workloads.make_filter(w)
        x = workloads.make_x0(w) if closed else workloads.make_x(w)
        hd, xd = to_dev(h, w.dtype), to_dev(x, w.dtype)
        log("case fi_conv_static", w.B, w.D, w.L, "closed" if closed else "open")
        ys, xs = _static(w, closed, hd, xd)
        outs.append((w, closed, h, x, hd, xd, ys, xs))
    torch.cuda.synchronize()
    for w, closed, h, x, hd, xd, ys, xs in outs:
        log("check fi_conv_static", w.B, w.D, w.L)
        yh, xh = gpu_run(hd, w.B, w.D, w.L, w.dtype, xd, closed=closed)
        assert torch.equal(ys, yh)
        y = host(ys).astype(np.float64)
        if closed:
            assert torch.equal(xs, xh)
            xr = host(xs).astype(np.float64)
            assert np.array_equal(xr[:, 0, :], x.astype(np.float64))
            assert np.abs(xr[:, 1:, :] - np.tanh(y[:, :-1, :])).max() <= 1e-6
            assert np.abs(y - oracle.default().conv_open(h, xr)).max() <= 1e-3
        else:
            assert rel_l2(y, oracle.default().conv_open(h, x)) <= 1e-5


def test_static_entry_refuses_beyond_workspace():
    w = workloads.get("hyena-d1024-l16k")
    h = torch.zeros((16, 4), dtype=torch.float32, device="cuda")
    y = torch.zeros((4,), dtype=torch.float32, device="cuda")
    cfg = fi.make_config(w.B, w.D, w.L, fi.FI_F32, 0, torch.cuda.current_stream())   # ~200 MB of buffers
    with pytest.raises(fi.FiError) as e:
        fi.fi_conv_static(cfg, h, h, fi.FI_FEEDBACK_TANH, y)
    assert e.value.status == fi.FI_ERR_UNSUPPORTED
    with pytest.raises(fi.FiError) as e:
        fi.fi_conv_static(cfg, h, h, 7, y)
    assert e.value.status == fi.FI_ERR_INVALID
