"""Skinny outputs: the reduction split across K waves (k_split > 1).

A product with few output rows n and long rows gives each row's wave steps
to K waves (K = the largest power of two within 1024 / n, 8 and the row's
whole wave steps, for rows of 3 or more of them) and adds the K wave sums by
a fixed pairwise tree.  Checked
here, against the float64 oracle and GPU against GPU:
  - every output within the tolerance at every m, row-exact across m, for
    each weight type at n = 1, 5, 64, 200, 300 (K = 8, 8, 8, 4, 2) and k of
    8 wave steps plus a ragged tail;
  - the derived K as stated, and every pinned K (1, 2, 4, 8) within the
    tolerance: the split decides the bits, not the accuracy;
  - packing inert under a fixed K (rows per wave, waves, workgroups, LDS
    passes of one, K - 1 and K + 1 wave steps);
  - batched and gathered calls bitwise equal to separate calls per entry (K
    depends on n, not on the batch);
  - the fused add + RMS norm: one kernel and two launches bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import bits, check_tolerance, gather_y, run_mv, to_dev
from quantized_few_row_amd import Schedule, Strides

pytestmark = pytest.mark.gpu

STEP = {wl.F16: 512, wl.Q8_0: 2048, wl.Q4_K: 4096, wl.Q6_K: 4096, wl.Q5_0: 2048, wl.F32: 256, wl.BF16: 512}
# 8 whole wave steps and a ragged tail of one block / 4 values
TAIL = {wl.F16: 4, wl.Q8_0: 32, wl.Q4_K: 256, wl.Q6_K: 256, wl.Q5_0: 32, wl.F32: 4, wl.BF16: 4}
TYPES = list(STEP)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]
NS = (1, 5, 64, 200, 300)


def _k(t):
    return 8 * STEP[t] + TAIL[t]


def _expected_k(t, n, k):
    steps = k // STEP[t]
    if steps < 3:
        return 1
    K = 1
    while K < 8 and 2 * K * n <= 1024 and 2 * K <= steps:
        K *= 2
    return K


@pytest.fixture(scope="module")
def data():
    out = {}
    for t in TYPES:
        k = _k(t)
        nmax = max(NS)
        W = wl.weights(t, nmax, k, seed=1300 + t)
        x = wl.activations(8, k, seed=1400 + t)
        y, a = oracle.matvec(t, W, x, nmax, k, 8)
        out[t] = dict(W=W, x=x, Wd=to_dev(W.ravel()), xd=to_dev(x.ravel()), y=y[0], a=a[0], k=k)
    return out


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("n", NS)
def test_split_tolerance_and_row_exactness(t, n, data):
    d = data[t]
    k = d["k"]
    K = qfr.row_exact_schedule(t, n, k, 1).k_split
    assert K == _expected_k(t, n, k) and K > 1
    print(f"[ksplit] {wl.TYPE_NAMES[t]} n={n} k={k}: K={K}", flush=True)
    # the first n rows of the weights are a product of their own
    ones = [bits(run_mv(t, d["Wd"], d["xd"][j * k:], n, k, 1)) for j in range(8)]
    for m in range(1, 9):
        y = run_mv(t, d["Wd"], d["xd"], n, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, n), d["y"][:m, :n], d["a"][:m, :n], f"n={n} m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"n={n} m={m} row {j} differs from its m=1 result"
    again = bits(run_mv(t, d["Wd"], d["xd"], n, k, 8))
    assert np.array_equal(again, bits(run_mv(t, d["Wd"], d["xd"], n, k, 8))), "not repeatable"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_every_pinned_split_within_tolerance(t, data):
    d = data[t]
    k, n, m = d["k"], 64, 3
    default = bits(run_mv(t, d["Wd"], d["xd"], n, k, m))
    sd = qfr.row_exact_schedule(t, n, k, m)
    for K in (1, 2, 4, 8):
        s = Schedule(K, 1, 8, (n + 8 // K - 1) // (8 // K), sd.k_chunk)
        y = run_mv(t, d["Wd"], d["xd"], n, k, m, schedule=s)
        check_tolerance(y.cpu().numpy().reshape(m, n), d["y"][:m, :n], d["a"][:m, :n], f"K={K}")
        if K == sd.k_split:
            assert np.array_equal(bits(y), default), "the derived split pinned differs from the default call"


def _packings(t, K, kc_max):
    """Packings with split K; LDS passes no larger than kc_max (the default
    schedule's pass, the largest that fits the device at this m)."""
    out = []
    for nr in (1, 2, 4):
        for waves in sorted({K, 2 * K, 8} - {16}):
            if waves <= 8:
                for wgs in (1, 3, 1000):
                    out.append(Schedule(K, nr, waves, wgs, 1 << 30))
        out.append(Schedule(K, nr, 8, 5, STEP[t]))           # LDS passes of one wave step
        out.append(Schedule(K, nr, K, 2, (K + 1) * STEP[t]))  # passes across the K waves' steps
        out.append(Schedule(K, nr, 8, 1, (K - 1) * STEP[t]))
    return [s for s in out if s.k_chunk <= kc_max]


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("m", [1, 4, 8])
def test_split_packing_is_inert(t, m, data):
    d = data[t]
    k = d["k"]
    for n in (5, 200, 300):
        sd = qfr.row_exact_schedule(t, n, k, m)
        K = sd.k_split
        ref = bits(run_mv(t, d["Wd"], d["xd"], n, k, m))
        for s in _packings(t, K, 1 << 30 if sd.k_chunk >= k else sd.k_chunk):
            got = bits(run_mv(t, d["Wd"], d["xd"], n, k, m, schedule=s))
            assert np.array_equal(got, ref), f"n={n}: schedule {s} changed the bits"


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q4_K, wl.F16], ids=["Q8_0", "Q4_K", "F16"])
def test_split_batched_equals_per_entry(t):
    """A batched strided call and a gathered call give every entry the bits
    of a separate call on that entry's weights."""
    n, k, m, batch = 40, _k(t), 4, 3
    W = wl.weights(t, n * batch, k, seed=1500 + t)
    s = Strides(k + 12, 5 * (k + 12), n + 3, 5 * (n + 3))
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    x = wl.activations(1, xb // 4, seed=1600 + t)[0]
    Wd, xd = to_dev(W.ravel()), to_dev(x)
    y = run_mv(t, Wd, xd, n, k, m, batch, strides=s, y_elems=yb // 4)
    got = gather_y(y.cpu().numpy(), n, m, batch, s.y_row_stride, s.y_batch_stride)
    ref, a = oracle.matvec(t, W, x, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    check_tolerance(got, ref, a, "batched")
    rb = qfr.row_exact_row_bytes(t, k)
    single = Strides(s.x_row_stride, 0, n, 0)
    for b in range(batch):
        yb1 = run_mv(t, Wd.data_ptr() + b * n * rb, xd[b * s.x_batch_stride:], n, k, m, 1, strides=single)
        assert np.array_equal(got[b].view(np.uint32), yb1.cpu().numpy().reshape(m, n).view(np.uint32)), f"entry {b}"
    # gathered: entries pick weight sets 2, 0, 2 of the three
    ids = np.array([2, 0, 2], dtype=np.int32)
    idd = torch.from_numpy(ids).to("cuda:0")
    yg = torch.full((yb // 4,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_gather(t, Wd, batch, idd, xd, yg, n, k, m, batch, s)
    torch.cuda.synchronize()
    gg = gather_y(yg.cpu().numpy(), n, m, batch, s.y_row_stride, s.y_batch_stride)
    for b in range(batch):
        yb1 = run_mv(t, Wd.data_ptr() + int(ids[b]) * n * rb, xd[b * s.x_batch_stride:], n, k, m, 1, strides=single)
        assert np.array_equal(gg[b].view(np.uint32), yb1.cpu().numpy().reshape(m, n).view(np.uint32)), \
            f"gathered entry {b}"


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q6_K], ids=["Q8_0", "Q6_K"])
def test_split_fused_norm_one_kernel_equals_two_launches(t):
    n, k = 96, _k(t)
    W = wl.weights(t, n, k, seed=1700 + t)
    x = wl.activations(8, k, seed=1710 + t)
    r = wl.activations(8, k, seed=1720 + t)
    g = wl.activations(1, k, seed=1730 + t)[0]
    Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel()), to_dev(g)
    assert qfr.row_exact_schedule(t, n, k, 1).k_split > 1
    href, _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, 8)
    for m in (1, 4, 8):
        y1 = torch.full((m * n,), float("nan"), device="cuda:0")
        y2 = torch.full((m * n,), float("nan"), device="cuda:0")
        h = torch.full((m * k,), float("nan"), device="cuda:0")
        qfr.row_exact_mv_add_rmsnorm(t, Wd, xd, rd, gd, 1e-5, h, y1, n, k, m)
        qfr.row_exact_mv_add_rmsnorm_ws(t, Wd, xd, rd, gd, 1e-5, None, y2, n, k, m)
        torch.cuda.synchronize()
        assert np.array_equal(bits(h), href[:m * k].view(np.int32)), f"m={m}: h"
        check_tolerance(y1.cpu().numpy().reshape(1, m, n), yref[:, :m], a[:, :m], f"m={m}")
        assert np.array_equal(bits(y1), bits(y2)), f"m={m}: one kernel and two launches differ"


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q6_K, wl.Q5_0], ids=["Q8_0", "Q6_K", "Q5_0"])
def test_split_two_byte_aligned_weights(t, data):
    """W 2 bytes past a 4-byte boundary (the page accepts any even address
    for these types) with the split: the same bits as W aligned, every m."""
    d = data[t]
    k, n = d["k"], 64
    rb = qfr.row_exact_row_bytes(t, k)
    raw = d["W"].ravel()[:n * rb]
    buf = torch.zeros(raw.size + 32, dtype=torch.uint8, device="cuda:0")
    buf[2:2 + raw.size].copy_(torch.from_numpy(raw.copy()))
    Wo = buf[2:2 + raw.size]
    assert Wo.data_ptr() % 4 == 2
    assert qfr.row_exact_schedule(t, n, k, 1).k_split > 1
    for m in (1, 5, 8):
        y = run_mv(t, Wo, d["xd"], n, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, n), d["y"][:m, :n], d["a"][:m, :n], f"m={m}")
        assert np.array_equal(bits(y), bits(run_mv(t, d["Wd"], d["xd"], n, k, m))), f"m={m}: differs from aligned W"
