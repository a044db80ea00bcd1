"""The allocation-free fused add + RMS norm (row_exact_mv_add_rmsnorm_noalloc)
called through the C ABI: its outputs (y and h) are bitwise those of the
entry point it is a variant of, row_exact_mv_add_rmsnorm_ws (same kernels on
a caller work buffer), on the same inputs, for two calls in a row (the
second smaller, so the fixed scratch array holds the first call's contents
when the second starts), and a call that needs more scratch than the array
holds is refused without touching y."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_few_row_amd as qfr
import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(t, n, k, m, seed):
    W = wl.weights(t, n, k, seed=seed)
    x = wl.activations(m, k, seed=seed + 1)
    r = wl.activations(m, k, seed=seed + 2)
    g = (1.0 + 0.1 * wl.activations(1, k, seed=seed + 3)[0]).astype(np.float32)
    dev = torch.device("cuda:0")
    return [torch.from_numpy(np.ascontiguousarray(a).ravel()).to(dev) for a in (W, x, r, g)]


def _call(entry, t, Wd, xd, rd, gd, n, k, m):
    lib = qfr.load_library()
    y = torch.full((m * n,), float("nan"), device="cuda:0")
    h = torch.full((m * k,), float("nan"), device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    extra = ()
    if entry.endswith("_ws"):
        work = torch.full((qfr.norm_work_bytes(k, m) // 4,), float("nan"), device="cuda:0")
        extra = (work.data_ptr(), work.numel() * 4)
    rc = getattr(lib, entry)(int(t), Wd.data_ptr(), xd.data_ptr(), rd.data_ptr(), gd.data_ptr(), ctypes.c_float(1e-5),
                             h.data_ptr(), y.data_ptr(), n, k, m, 1, None, *extra, stream)
    assert rc == 0, (rc, qfr.row_exact_last_error())
    torch.cuda.synchronize()
    return y, h


def test_noalloc_matches_the_allocating_entry_point_twice():
    calls = [(wl.Q8_0, 517, 4096, 8, 7100), (wl.Q4_K, 133, 2304, 3, 7200)]  # the second is smaller
    for t, n, k, m, seed in calls:
        print(f"[noalloc] type {wl.TYPE_NAMES[t]} n={n} k={k} m={m}", flush=True)
        Wd, xd, rd, gd = _inputs(t, n, k, m, seed)
        y_na, h_na = _call("row_exact_mv_add_rmsnorm_noalloc", t, Wd, xd, rd, gd, n, k, m)
        y_ref, h_ref = _call("row_exact_mv_add_rmsnorm_ws", t, Wd, xd, rd, gd, n, k, m)
        assert torch.equal(y_na.view(torch.int32), y_ref.view(torch.int32)), "y differs"
        assert torch.equal(h_na.view(torch.int32), h_ref.view(torch.int32)), "h differs"
        assert not torch.isnan(y_na).any()


def test_noalloc_refuses_calls_beyond_its_scratch():
    # batch * m * k * 4 bytes of u alone beyond the array: refused before any launch
    t, n, k, m = wl.Q8_0, 64, 32768 * 4 + 32, 8
    assert m * k * 4 > qfr.NOALLOC_SCRATCH_BYTES
    lib = qfr.load_library()
    y = torch.full((m * n,), 7.0, device="cuda:0")
    x = torch.zeros(m * k, device="cuda:0")
    W = torch.zeros(n * (k // 32) * 34, dtype=torch.uint8, device="cuda:0")
    before = qfr.row_exact_launch_count()
    rc = lib.row_exact_mv_add_rmsnorm_noalloc(int(t), W.data_ptr(), x.data_ptr(), x.data_ptr(), None,
                                              ctypes.c_float(1e-5), None, y.data_ptr(), n, k, m, 1, None, None)
    assert rc == -5 and "scratch" in qfr.row_exact_last_error()
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and qfr.row_exact_launch_count() == before
