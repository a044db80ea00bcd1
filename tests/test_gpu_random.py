"""Seeded random configurations against the oracle: every weight type, row
counts and k values around the lane-map and wave-step boundaries, 1..8 input
rows, batches with batch-major or token-major strides (with gaps), plain,
gathered and fused-norm calls.  Each case checks the tolerance against the
float64 oracle, that nothing outside the output view is written, and that a
sampled input row is bitwise its m = 1 result."""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import bits, check_tolerance, to_dev
from quantized_few_row_amd import Strides

pytestmark = pytest.mark.gpu

PER = {wl.F16: 4, wl.F32: 4, wl.BF16: 4, wl.Q8_0: 32, wl.Q5_0: 32, wl.Q4_K: 256, wl.Q6_K: 256}
# k in units of PER: up to just past two 64-lane wave steps
UNITS = {wl.F16: 300, wl.F32: 140, wl.BF16: 300, wl.Q8_0: 140, wl.Q5_0: 140, wl.Q4_K: 36, wl.Q6_K: 36}


def _cases(count=48, seed=20261202):
    rng = np.random.default_rng(seed)
    types = sorted(PER)
    out = []
    for c in range(count):
        t = types[c % len(types)]
        k = PER[t] * int(rng.integers(1, UNITS[t] + 1))
        n = int(rng.integers(1, 160))
        m = int(rng.integers(1, 9))
        batch = int(rng.integers(1, 4))
        layout = ["contiguous", "batch", "token"][int(rng.integers(0, 3))] if batch > 1 else "contiguous"
        mode = ["plain", "plain", "gather", "norm"][int(rng.integers(0, 4))]
        out.append((c, t, n, k, m, batch, layout, mode))
    return out


CASES = _cases()


def _strides(layout, n, k, m, batch):
    if layout == "contiguous":
        return Strides(k, m * k if batch > 1 else 0, n, m * n if batch > 1 else 0)
    if layout == "batch":
        return Strides(k + 4, m * (k + 4) + 8, n + 3, m * (n + 3) + 5)
    return Strides(batch * k + 8, k, batch * n + 7, n)


@pytest.mark.parametrize("c,t,n,k,m,batch,layout,mode", CASES,
                         ids=[f"{c}-{wl.TYPE_NAMES[t]}-n{n}-k{k}-m{m}-b{b}-{lay}-{mode}"
                              for c, t, n, k, m, b, lay, mode in CASES])
def test_random_configuration(c, t, n, k, m, batch, layout, mode):
    s = _strides(layout, n, k, m, batch)
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    x = wl.activations(1, xb // 4, seed=5000 + c)[0]
    xd = to_dev(x)
    y = torch.full((yb // 4 + 8,), 7.0, device="cuda:0")
    if mode == "gather":
        E = batch + 2
        W = wl.weights(t, E * n, k, seed=6000 + c)
        ids = ((np.arange(batch) * 3 + c) % (E + 1)).astype(np.int32)  # may include E (out of range)
        Wd = to_dev(W.ravel())
        qfr.row_exact_mv_gather(t, Wd, E, torch.from_numpy(ids).to("cuda:0"), xd, y, n, k, m, batch, s)
        ref, a = oracle.matvec_gather(t, W, E, ids, x, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    elif mode == "norm":
        W = wl.weights(t, batch * n, k, seed=6000 + c)
        r = wl.activations(1, xb // 4, seed=7000 + c)[0]
        g = (1.0 + 0.1 * wl.activations(1, k, seed=8000 + c)[0]).astype(np.float32)
        Wd = to_dev(W.ravel())
        qfr.row_exact_mv_add_rmsnorm(t, Wd, xd, to_dev(r), to_dev(g), 1e-5, None, y, n, k, m, batch, s)
        _, _, ref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    else:
        W = wl.weights(t, batch * n, k, seed=6000 + c)
        Wd = to_dev(W.ravel())
        qfr.row_exact_mv(t, Wd, xd, y, n, k, m, batch, s)
        ref, a = oracle.matvec(t, W, x, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    got = np.empty((batch, m, n))
    mask = np.ones(yc.size, bool)
    for b in range(batch):
        for j in range(m):
            o = b * s.y_batch_stride + j * s.y_row_stride
            got[b, j] = yc[o:o + n]
            mask[o:o + n] = False
    valid = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~valid), "NaN outputs differ from the oracle's"
    if valid.any():
        check_tolerance(np.where(valid, got, 0.0), np.where(valid, ref, 0.0), np.where(valid, a, 0.0), f"case {c}")
    assert np.all(yc[mask] == 7.0), "an element outside the output view was written"
    # row exactness: the last input row alone (m = 1, same batch layout)
    if m > 1 and mode != "gather":
        j = m - 1
        s1 = Strides(s.x_row_stride, s.x_batch_stride, s.y_row_stride, s.y_batch_stride)
        y1 = torch.full((yb // 4 + 8,), 7.0, device="cuda:0")
        xj = xd[j * s.x_row_stride:]
        if mode == "norm":
            rj = to_dev(r[j * s.x_row_stride:])
            qfr.row_exact_mv_add_rmsnorm(t, Wd, xj, rj, to_dev(g), 1e-5, None, y1, n, k, 1, batch, s1)
        else:
            qfr.row_exact_mv(t, Wd, xj, y1, n, k, 1, batch, s1)
        torch.cuda.synchronize()
        y1b, yb_ = bits(y1), bits(y)
        for b in range(batch):
            o1 = b * s.y_batch_stride
            o = o1 + j * s.y_row_stride
            assert np.array_equal(y1b[o1:o1 + n], yb_[o:o + n]), f"batch {b}: row {j} differs from its m = 1 run"
