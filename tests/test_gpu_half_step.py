"""Rows whose last 64-lane wave step would be at most half full.

A row of 64 s + r pieces, 0 < r <= 32 (Q6_K k = 14336: 224 pieces, 3.5
steps of 64 lanes), of a block-quantized type takes 32 lanes per row
instead, two rows per wave, unless the reduction is split across waves (the
split keeps 64 lanes); the dense types keep 64 lanes.  The lane map is part
of the numerics and follows from (type, k, split) alone.  Checked here for
every weight type at 66, 96, 130 and 224 pieces (tails of 2 and 32):
  - every output within the tolerance of the float64 oracle at every m, each
    row bitwise equal to its m = 1 result, repeats bitwise equal;
  - packing inert: rows per wave, waves, workgroups and LDS passes (one and
    two 64-lane steps per pass, where the 32-lane rows take the several-pass
    path) give the bits of the default call;
  - a pinned split (64 lanes per row) within the tolerance;
  - batched and gathered calls bitwise equal to separate calls per entry;
  - the fused add + RMS norm: one kernel (several passes at m = 8) and two
    launches bitwise equal, h exact.
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

# values per 64-lane wave step (64 pieces)
STEP = {wl.F16: 512, wl.Q8_0: 2048, wl.Q4_K: 4096, wl.Q6_K: 4096, wl.Q5_0: 2048, wl.F32: 256, wl.BF16: 512}
TYPES = list(STEP)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]
# 64 s + r pieces, r = 2 (4 where a piece is a quarter of a 256-value
# super-block, so that k stays whole super-blocks) or 32
PIECES = ("short_tail_1", 96, "short_tail_2", 224)
N = 600  # enough rows that the derived split is 1 (a split keeps 64 lanes)


def _pieces(t, p):
    r = 4 if t in (wl.Q4_K, wl.Q6_K) else 2
    return {"short_tail_1": 64 + r, "short_tail_2": 128 + r}.get(p, p)


def _k(t, p):
    return STEP[t] // 64 * _pieces(t, p)


@pytest.fixture(scope="module")
def data():
    out = {}
    for t in TYPES:
        for h in PIECES:
            k = _k(t, h)
            W = wl.weights(t, N, k, seed=2100 + 1000 * t + _pieces(t, h))
            x = wl.activations(8, k, seed=2200 + 1000 * t + _pieces(t, h))
            y, a = oracle.matvec(t, W, x, N, k, 8)
            out[t, h] = dict(W=W, x=x, Wd=to_dev(W.ravel()), xd=to_dev(x.ravel()), y=y[0], a=a[0], k=k)
    return out


@pytest.mark.parametrize("h", PIECES, ids=[str(p) for p in PIECES])
@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_half_step_rows_tolerance_and_row_exactness(t, h, data):
    d = data[t, h]
    k = d["k"]
    assert qfr.row_exact_schedule(t, N, k, 1).k_split == 1
    print(f"[half-step] {wl.TYPE_NAMES[t]} n={N} k={k}", flush=True)
    ones = [bits(run_mv(t, d["Wd"], d["xd"][j * k:], N, k, 1)) for j in range(8)]
    for m in range(1, 9):
        y = run_mv(t, d["Wd"], d["xd"], N, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, N), d["y"][:m], d["a"][:m], f"m={m}")
        yb = bits(y).reshape(m, N)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
    # odd row counts (a wave's second row slot past n) give the same rows;
    # split 1 pinned, as the derived split of so few rows may differ
    s1 = qfr.row_exact_schedule(t, N, k, 3)
    for n in (1, 77):
        y = bits(run_mv(t, d["Wd"], d["xd"], n, k, 3, schedule=s1)).reshape(3, n)
        for j in range(3):
            assert np.array_equal(y[j], ones[j][:n]), f"n={n} row {j}"
    again = bits(run_mv(t, d["Wd"], d["xd"], N, k, 8))
    assert np.array_equal(again, bits(run_mv(t, d["Wd"], d["xd"], N, k, 8))), "not repeatable"


def _packings(t, kc_max):
    out = []
    for nr in (1, 2, 4):
        for waves, wgs in ((1, 1), (8, 2), (3, 5), (8, 1000)):
            out.append(Schedule(1, nr, waves, wgs, 1 << 30))
        out.append(Schedule(1, nr, 8, 3, STEP[t]))       # passes of one 64-lane step
        out.append(Schedule(1, nr, 4, 1000, 2 * STEP[t]))
    return [s for s in out if min(s.k_chunk, 1 << 30) <= kc_max]


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_half_step_packing_is_inert(t, m, data):
    for h in PIECES:
        d = data[t, h]
        k = d["k"]
        sd = qfr.row_exact_schedule(t, N, k, m)
        ref = bits(run_mv(t, d["Wd"], d["xd"], N, k, m))
        for s in _packings(t, 1 << 30 if sd.k_chunk >= k else sd.k_chunk):
            got = bits(run_mv(t, d["Wd"], d["xd"], N, k, m, schedule=s))
            assert np.array_equal(got, ref), f"k={k}: schedule {s} changed the bits"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_half_step_pinned_split_within_tolerance(t, data):
    d = data[t, 224]
    k, m = d["k"], 4
    sd = qfr.row_exact_schedule(t, N, k, m)
    for K in (2,):
        s = Schedule(K, 1, 8, (N + 8 // K - 1) // (8 // K), sd.k_chunk)
        y = run_mv(t, d["Wd"], d["xd"], N, k, m, schedule=s)
        check_tolerance(y.cpu().numpy().reshape(m, N), d["y"][:m], d["a"][:m], f"K={K}")


@pytest.mark.parametrize("t", [wl.Q6_K, wl.Q8_0, wl.F16], ids=["Q6_K", "Q8_0", "F16"])
def test_half_step_batched_and_gathered_equal_per_entry(t):
    n, k, m, batch = 521, _k(t, 224), 5, 3
    assert qfr.row_exact_schedule(t, n, k, m, batch).k_split == 1
    W = wl.weights(t, n * batch, k, seed=2300 + t)
    s = Strides(k + 8, 5 * (k + 8), n + 3, 5 * (n + 3))
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    x = wl.activations(1, xb // 4, seed=2400 + t)[0]
    Wd, xd = to_dev(W.ravel()), to_dev(x)
    y = run_mv(t, Wd, xd, n, k, m, batch, strides=s, y_elems=yb // 4)
    got = gather_y(y.cpu().numpy(), n, m, batch, s.y_row_stride, s.y_batch_stride)
    ref, a = oracle.matvec(t, W, x, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    check_tolerance(got, ref, a, "batched")
    rb = qfr.row_exact_row_bytes(t, k)
    single = Strides(s.x_row_stride, 0, n, 0)
    for b in range(batch):
        y1 = run_mv(t, Wd.data_ptr() + b * n * rb, xd[b * s.x_batch_stride:], n, k, m, 1, strides=single)
        assert np.array_equal(got[b].view(np.uint32), y1.cpu().numpy().reshape(m, n).view(np.uint32)), f"entry {b}"
    ids = np.array([1, 2, 1], dtype=np.int32)
    idd = torch.from_numpy(ids).to("cuda:0")
    yg = torch.full((yb // 4,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_gather(t, Wd, batch, idd, xd, yg, n, k, m, batch, s)
    torch.cuda.synchronize()
    gg = gather_y(yg.cpu().numpy(), n, m, batch, s.y_row_stride, s.y_batch_stride)
    for b in range(batch):
        y1 = run_mv(t, Wd.data_ptr() + int(ids[b]) * n * rb, xd[b * s.x_batch_stride:], n, k, m, 1, strides=single)
        assert np.array_equal(gg[b].view(np.uint32), y1.cpu().numpy().reshape(m, n).view(np.uint32)), \
            f"gathered entry {b}"


@pytest.mark.parametrize("t", [wl.Q6_K, wl.Q8_0, wl.BF16], ids=["Q6_K", "Q8_0", "BF16"])
def test_half_step_fused_norm_one_kernel_equals_two_launches(t):
    n, k = 600, _k(t, 224)
    W = wl.weights(t, n, k, seed=2500 + t)
    x = wl.activations(8, k, seed=2510 + t)
    r = wl.activations(8, k, seed=2520 + t)
    g = wl.activations(1, k, seed=2530 + t)[0]
    Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel()), to_dev(g)
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


@pytest.mark.parametrize("h", (96, 224))
@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_pinned_lanes_per_row(t, h, data):
    """Each lane map pinned (16, 32, 64 lanes per row, unsplit): within the
    tolerance at m = 1 and 8, every row of m = 8 bitwise equal to its m = 1
    result under the same map, two packings at m = 3 bitwise equal; the
    derived value pinned gives the default call's bits."""
    d = data[t, h]
    k = d["k"]
    derived = qfr.row_exact_schedule(t, N, k, 1).lanes_per_row
    one = lambda L: Schedule(1, 1, 8, 1000, 1 << 30, L)       # noqa: E731
    passes = lambda nr, wv, kc, L: Schedule(1, nr, wv, 1000, kc, L)  # noqa: E731
    for L in (16, 32, 64):
        ones = [bits(run_mv(t, d["Wd"], d["xd"][j * k:], N, k, 1, schedule=one(L))) for j in range(8)]
        check_tolerance(np.stack([o.view(np.float32) for o in ones]), d["y"], d["a"], f"L={L} m=1")
        y8 = run_mv(t, d["Wd"], d["xd"], N, k, 8, schedule=passes(1, 8, STEP[t], L))
        check_tolerance(y8.cpu().numpy().reshape(8, N), d["y"], d["a"], f"L={L} m=8")
        yb = bits(y8).reshape(8, N)
        for j in range(8):
            assert np.array_equal(yb[j], ones[j]), f"L={L}: m=8 row {j} differs from its m=1 result"
        a = bits(run_mv(t, d["Wd"], d["xd"], N, k, 3, schedule=passes(1, 8, STEP[t], L)))
        b = bits(run_mv(t, d["Wd"], d["xd"], N, k, 3, schedule=passes(2, 4, 2 * STEP[t], L)))
        assert np.array_equal(a, b), f"L={L}: packing changed the bits"
        if L == derived:
            assert np.array_equal(ones[0], bits(run_mv(t, d["Wd"], d["xd"], N, k, 1))), \
                f"L={L} pinned differs from the default call"


def _rule_lanes(t, k, K):
    """The documented lane map: 16 / 32 for rows of at most 16 / 32 pieces;
    32 for unsplit block-type rows of 64 s + r pieces, 0 < r <= 32, under
    2^29 bytes; 64 otherwise."""
    p = k // (STEP[t] // 64)
    if p <= 16:
        return 16
    if p <= 32:
        return 32
    blocks = t in (wl.Q8_0, wl.Q4_K, wl.Q6_K, wl.Q5_0)
    if blocks and K == 1 and 0 < p % 64 <= 32 and qfr.row_exact_row_bytes(t, k) < (1 << 29):
        return 32
    return 64


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_derived_lanes_follow_the_rule(t):
    """row_exact_schedule's lanes_per_row against the documented rule over
    row lengths of 1..9 wave steps with every tail class, several n (split
    and unsplit) and every m (the lane map never depends on m)."""
    vpp = STEP[t] // 64
    quantum = 4 if t in (wl.Q4_K, wl.Q6_K) else 1  # pieces per 256-value super-block
    checked = 0
    for p in sorted({quantum * i for i in range(1, 160 // quantum)} | {64 * s + r for s in range(1, 9)
                                                                        for r in (quantum, 16, 32, 36, 60)}):
        if p % quantum:
            continue
        k = p * vpp
        for n in (1, 40, 300, 1024, 5000):
            lanes = {qfr.row_exact_schedule(t, n, k, m).lanes_per_row for m in (1, 3, 8)}
            assert len(lanes) == 1, f"p={p} n={n}: lanes depend on m: {lanes}"
            K = qfr.row_exact_schedule(t, n, k, 1).k_split
            assert lanes == {_rule_lanes(t, k, K)}, f"p={p} k={k} n={n} K={K}: {lanes}"
            checked += 1
    assert checked > 100
