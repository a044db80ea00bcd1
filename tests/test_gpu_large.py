"""Weights past 4 GiB: 64-bit row and batch offsets.

The weight buffer is a block of P seeded rows repeated on the device, so row
r holds the bytes of block row r mod P and its exact output is the oracle's
output for that block row.  Every output is compared with the oracle (within
the tolerance) and, bitwise, with the output of the same block row in the
first P rows: a row read from a wrong (truncated) address breaks both."""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import TOL_ABS, TOL_REL, bits, to_dev
from quantized_few_row_amd import Strides

pytestmark = pytest.mark.gpu

P = 1024  # rows in the repeated block


def _tiled(t, k, rows, seed):
    W = wl.weights(t, P, k, seed=seed)
    rb = wl.row_bytes(t, k)
    reps = -(-rows // P)
    Wd = to_dev(W.ravel()).view(1, -1).expand(reps, -1).reshape(-1)[: rows * rb].contiguous()
    return W, Wd


def _check(y, yref, a, rows, label):
    """y [m, rows] against the block outputs yref / a [m, P]."""
    idx = np.arange(rows) % P
    ref, mag = yref[:, idx], a[:, idx]
    err = np.abs(y.astype(np.float64) - ref)
    bad = err > TOL_REL * mag + TOL_ABS
    assert not bad.any(), f"{label}: {bad.sum()} outputs out of tolerance, first at {np.argwhere(bad)[0]}"
    yb = y.view(np.int32)
    assert np.array_equal(yb, yb[:, idx]), f"{label}: a row differs from the same block row below 4 GiB"


@pytest.mark.parametrize("m", [1, 8])
def test_weights_past_4gib(m):
    t, k = wl.Q8_0, 4096
    rows = 1_000_003  # 4.35 GB of weights, ragged tail
    assert rows * wl.row_bytes(t, k) > (1 << 32)
    W, Wd = _tiled(t, k, rows, seed=4242)
    x = wl.activations(8, k, seed=4243)[:m]
    yref, a = oracle.matvec(t, W, x.ravel(), P, k, m)
    y = torch.full((m * rows,), float("nan"), device="cuda:0")
    qfr.row_exact_mv(t, Wd, to_dev(x.ravel()), y, rows, k, m)
    torch.cuda.synchronize()
    _check(y.cpu().numpy().reshape(m, rows), yref[0], a[0], rows, f"m={m}")


def test_batches_past_4gib():
    """Two batch entries of 2.6 GB each: the second starts past 2^31 bytes and
    ends past 2^32; the gathered call selects the second set for entry 0."""
    t, k, m = wl.Q8_0, 4096, 4
    n = 600_064  # a multiple of P, so both entries hold the same rows
    rb = wl.row_bytes(t, k)
    assert 2 * n * rb > (1 << 32)
    W, Wd = _tiled(t, k, 2 * n, seed=4244)
    x = wl.activations(8, 2 * k, seed=4245)[:m]
    xd = to_dev(x.ravel())
    yref0, a0 = oracle.matvec(t, W, x.ravel(), P, k, m, x_row_stride=2 * k)
    yref1, a1 = oracle.matvec(t, W, x[:, k:].ravel(), P, k, m)
    s = Strides(2 * k, k, n, m * n)  # x rows of 2k values, batch b at column b*k; y [batch, m, n]
    y = torch.full((2 * m * n,), float("nan"), device="cuda:0")
    qfr.row_exact_mv(t, Wd, xd, y, n, k, m, 2, s)
    torch.cuda.synchronize()
    yy = y.cpu().numpy().reshape(2, m, n)
    _check(yy[0], yref0[0], a0[0], n, "batch 0")
    _check(yy[1], yref1[0], a1[0], n, "batch 1")
    ids = to_dev(np.array([1], dtype=np.int32))
    yg = torch.full((m * n,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_gather(t, Wd, 2, ids, xd, yg, n, k, m, 1, s)
    torch.cuda.synchronize()
    assert np.array_equal(bits(yg).reshape(m, n), yy[0].view(np.int32)), "gathered entry 1 differs from batch 0"
