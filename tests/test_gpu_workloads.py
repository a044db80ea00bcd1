"""The synthetic workloads at full size, in the launch configuration the
benchmark times (the default schedule).  Every output of every m of each
workload is compared with the oracle (the oracle split by output rows over
host threads), every weight row's dequantized values are compared bit for
bit, and row exactness and repeatability are checked on every output, GPU
against GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import bits, check_tolerance, oracle_dequant_rows, oracle_full, run_mv, to_dev

pytestmark = pytest.mark.gpu

NAMES = [w.name for w in wl.WORKLOADS if not w.experts and not w.fused_norm]
NORM_NAMES = [w.name for w in wl.WORKLOADS if w.fused_norm]
GATHER_NAMES = [w.name for w in wl.WORKLOADS if w.experts]


def check_all_weights(t, W, Wd, n, k, chunk_values=1 << 26):
    """row_exact_dequant of every weight row, bit-exact against the oracle,
    in chunks of rows."""
    rb = qfr.row_exact_row_bytes(t, k)
    step = max(1, chunk_values // k)
    out = torch.empty((min(step, n), k), dtype=torch.float32, device="cuda:0")
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        qfr.row_exact_dequant(t, Wd.data_ptr() + r0 * rb, out, r1 - r0, k)
        torch.cuda.synchronize()
        got = out[:r1 - r0].cpu().numpy()
        ref = oracle_dequant_rows(t, W, r0, r1, k)
        bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"weight rows {r0}..{r1}: {bad.shape[0]} values differ, first at {bad[0].tolist()}"


@pytest.mark.parametrize("name", NAMES)
def test_full_size_workload(name):
    w = wl.get(name)
    t, n, k, batch = w.wtype, w.n, w.k, w.batch
    print(f"[workload] {name}: type {wl.TYPE_NAMES[t]} n={n} k={k} batch={batch} m={w.ms}", flush=True)
    W = w.make_weights()
    x = w.make_x(8)
    Wd = to_dev(W.ravel())
    xd = to_dev(x.ravel())

    check_all_weights(t, W, Wd, n * batch, k)
    print(f"[workload] {name}: all {n * batch} weight rows bit-exact", flush=True)

    xrs, xbs, yrs, ybs = w.strides(8)
    strides = qfr.Strides(xrs, xbs, yrs, ybs)
    ones = {}
    for m in sorted(set(w.ms) | {1}):
        y = run_mv(t, Wd, xd, n, k, m, batch, strides=strides)
        yc = y.cpu().numpy()
        ref, a = oracle_full(t, W, x.ravel(), n, k, m, batch, xrs, xbs)
        got = np.empty_like(ref)
        for b in range(batch):
            for j in range(m):
                got[b, j] = yc[b * ybs + j * yrs:b * ybs + j * yrs + n]
        ratio = check_tolerance(got, ref, a, f"{name} m={m}")
        print(f"[workload] {name} m={m}: all {batch} x {m} x {n} outputs within tolerance, "
              f"worst |err|/bound = {ratio:.3g}", flush=True)
        ybits = bits(y)
        if m == 1:
            # m = 1 run of each input row j, for the row-exactness check
            for j in range(8):
                yj = run_mv(t, Wd, xd, n, k, 1, batch, strides=strides, x_offset=j * xrs)
                ones[j] = bits(yj)
        for j in range(m):
            for b in range(batch):
                o = b * ybs + j * yrs
                assert np.array_equal(ybits[o:o + n], ones[j][b * ybs:b * ybs + n]), \
                    f"{name}: m={m} row {j} batch {b} differs from m=1"
        again = bits(run_mv(t, Wd, xd, n, k, m, batch, strides=strides))
        assert np.array_equal(again, ybits), f"{name}: m={m} not repeatable"


@pytest.mark.parametrize("name", GATHER_NAMES)
def test_full_size_gather_workload(name):
    """Mixture-of-experts decode: every output against the oracle's gathered
    product, bitwise against row_exact_mv on the selected expert, row-exact
    across m and repeatable."""
    w = wl.get(name)
    t, n, k, batch, E = w.wtype, w.n, w.k, w.batch, w.experts
    print(f"[workload] {name}: type {wl.TYPE_NAMES[t]} {E} experts of n={n} k={k}, {batch} selected, m={w.ms}",
          flush=True)
    W = w.make_weights()
    ids = w.make_ids()
    x = w.make_x(8)
    Wd, xd = to_dev(W.ravel()), to_dev(x.ravel())
    idd = torch.from_numpy(ids).to("cuda:0")
    xrs, xbs, yrs, ybs = w.strides(8)
    strides = qfr.Strides(xrs, xbs, yrs, ybs)
    rb = qfr.row_exact_row_bytes(t, k)
    ones = {}
    for m in sorted(set(w.ms) | {1}):
        _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
        y = torch.full((yb // 4,), float("nan"), device="cuda:0")
        qfr.row_exact_mv_gather(t, Wd, E, idd, xd, y, n, k, m, batch, strides)
        torch.cuda.synchronize()
        yc = y.cpu().numpy()
        ref, a = oracle.matvec_gather(t, W, E, ids, x.ravel(), n, k, m, batch, xrs, xbs)
        got = np.empty_like(ref)
        for b in range(batch):
            for j in range(m):
                got[b, j] = yc[b * ybs + j * yrs: b * ybs + j * yrs + n]
        ratio = check_tolerance(got, ref, a, f"{name} m={m}")
        print(f"[workload] {name} m={m}: {batch} x {m} x {n} outputs ok, worst |err|/bound = {ratio:.3g}", flush=True)
        ybits = bits(y)
        if m == 1:
            for j in range(8):
                yj = torch.full((yb // 4,), float("nan"), device="cuda:0")
                qfr.row_exact_mv_gather(t, Wd, E, idd, xd[j * xrs:], yj, n, k, 1, batch, strides)
                torch.cuda.synchronize()
                ones[j] = bits(yj)
        for j in range(m):
            for b in range(batch):
                o = b * ybs + j * yrs
                assert np.array_equal(ybits[o:o + n], ones[j][b * ybs:b * ybs + n]), \
                    f"{name}: m={m} row {j} entry {b} differs from m=1"
        # each entry equals the plain product with its expert's weights
        for b in (0, batch - 1):
            ye = run_mv(t, Wd.data_ptr() + int(ids[b]) * n * rb, xd, n, k, m, 1, strides=qfr.Strides(xrs, 0, n, 0))
            yeb = bits(ye).reshape(m, n)
            for j in range(m):
                o = b * ybs + j * yrs
                assert np.array_equal(ybits[o:o + n], yeb[j]), f"{name}: entry {b} row {j} differs from row_exact_mv"
        again = torch.full((yb // 4,), float("nan"), device="cuda:0")
        qfr.row_exact_mv_gather(t, Wd, E, idd, xd, again, n, k, m, batch, strides)
        torch.cuda.synchronize()
        assert np.array_equal(bits(again), ybits), f"{name}: m={m} not repeatable"


@pytest.mark.parametrize("name", NORM_NAMES)
def test_full_size_fused_norm_workload(name):
    """The projection with its input made by the fused add + RMS norm: h
    bit-exact, every output against the oracle, row-exact across m."""
    w = wl.get(name)
    t, n, k = w.wtype, w.n, w.k
    print(f"[workload] {name}: type {wl.TYPE_NAMES[t]} n={n} k={k} m={w.ms}, fused add + RMS norm", flush=True)
    W, x, r, g = w.make_weights(), w.make_x(8), w.make_residual(8), w.make_norm_weight()
    Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel()), to_dev(g)
    href, _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, 8)
    ones = []
    for j in range(8):
        y1 = torch.empty(n, device="cuda:0")
        qfr.row_exact_mv_add_rmsnorm(t, Wd, xd[j * k:], rd[j * k:], gd, 1e-5, None, y1, n, k, 1)
        torch.cuda.synchronize()
        ones.append(bits(y1))
    for m in w.ms:
        y = torch.full((m * n,), float("nan"), device="cuda:0")
        h = torch.full((m * k,), float("nan"), device="cuda:0")
        qfr.row_exact_mv_add_rmsnorm(t, Wd, xd, rd, gd, 1e-5, h, y, n, k, m)
        torch.cuda.synchronize()
        assert np.array_equal(bits(h), href[:m * k].view(np.int32)), f"m={m}: h"
        ratio = check_tolerance(y.cpu().numpy().reshape(1, m, n), yref[:, :m], a[:, :m], f"{name} m={m}")
        print(f"[workload] {name} m={m}: {m} x {n} outputs ok, worst |err|/bound = {ratio:.3g}", flush=True)
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"{name}: m={m} row {j} differs from m=1"
