"""GPU parity of the products with a normalisation of their input against
the oracle.  The fused add + RMS norm (row_exact_mv_add_rmsnorm and its two
forms): h = x + r bit-exact, y within the tolerance of the float64
reference, row exactness across m and packing inertness (single and
multi-pass LDS staging), with and without g, batched strides.  The residual
RMS norm (row_exact_mv_residual_rmsnorm_ws): hs within float32 rounding of
the oracle's, y within the tolerance, row exactness, the add form's bits
when x = 0, in-place update of h, batched strides, several LDS passes."""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import bits, check_tolerance, to_dev
from quantized_few_row_amd import Strides

pytestmark = pytest.mark.gpu

SHAPES = {wl.F16: (41, 1028), wl.Q8_0: (45, 4160), wl.Q4_K: (37, 4352), wl.Q6_K: (29, 4352), wl.Q5_0: (33, 2112),
          wl.F32: (35, 516), wl.BF16: (39, 1028)}
TYPES = list(SHAPES)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]


def _run(t, Wd, xd, rd, gd, eps, n, k, m, batch=1, strides=None):
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
    y = torch.full((yb // 4,), float("nan"), device="cuda:0")
    h = torch.full((xb // 4,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_add_rmsnorm(t, Wd, xd, rd, gd, eps, h, y, n, k, m, batch, strides)
    torch.cuda.synchronize()
    return h, y


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("with_g", [True, False])
def test_add_rmsnorm_parity(t, with_g):
    n, k = SHAPES[t]
    W = wl.weights(t, n, k, seed=970 + t)
    x = wl.activations(8, k, seed=971 + t)
    r = wl.activations(8, k, seed=972 + t)
    g = (1.0 + 0.1 * wl.activations(1, k, seed=973 + t)[0]).astype(np.float32) if with_g else None
    eps = 1e-5
    Wd, xd, rd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel())
    gd = to_dev(g) if with_g else None
    href, _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, eps, n, k, 8)
    ones = []
    for j in range(8):
        _, y1 = _run(t, Wd, xd[j * k:], rd[j * k:], gd, eps, n, k, 1)
        ones.append(bits(y1))
    for m in (1, 2, 3, 5, 8):
        h, y = _run(t, Wd, xd, rd, gd, eps, n, k, m)
        assert np.array_equal(bits(h), href[:m * k].view(np.int32)), f"m={m}: h differs from x + r"
        check_tolerance(y.cpu().numpy().reshape(1, m, n), yref[:, :m], a[:, :m], f"m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
    again = bits(_run(t, Wd, xd, rd, gd, eps, n, k, 8)[1])
    assert np.array_equal(again, bits(_run(t, Wd, xd, rd, gd, eps, n, k, 8)[1]))


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q4_K, wl.F16], ids=["Q8_0", "Q4_K", "F16"])
def test_add_rmsnorm_batched_strided(t):
    """Batch-major strided x / r / h with gaps: per-row statistics, h written
    once per element, nothing outside the views touched."""
    n, k = SHAPES[t]
    batch, m = 3, 4
    s = Strides(k + 8, 5 * (k + 8), n + 3, 5 * (n + 3))
    W = wl.weights(t, n * batch, k, seed=980 + t)
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    x = wl.activations(1, xb // 4, seed=981 + t)[0]
    r = wl.activations(1, xb // 4, seed=982 + t)[0]
    g = (1.0 + 0.1 * wl.activations(1, k, seed=983 + t)[0]).astype(np.float32)
    h = torch.full((xb // 4 + 8,), 7.0, device="cuda:0")
    y = torch.full((yb // 4 + 8,), 7.0, device="cuda:0")
    qfr.row_exact_mv_add_rmsnorm(t, to_dev(W.ravel()), to_dev(x), to_dev(r), to_dev(g), 1e-6, h, y, n, k, m, batch, s)
    torch.cuda.synchronize()
    href, _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-6, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
    hc, yc = h.cpu().numpy(), y.cpu().numpy()
    hmask = np.zeros(hc.size, bool)
    for b in range(batch):
        for j in range(m):
            o = b * s.x_batch_stride + j * s.x_row_stride
            hmask[o:o + k] = True
    assert np.array_equal(hc[hmask].view(np.uint32), href[hmask[:href.size]].view(np.uint32))
    assert np.all(hc[~hmask] == 7.0), "h written outside its view"
    got = np.empty((batch, m, n))
    ymask = np.zeros(yc.size, bool)
    for b in range(batch):
        for j in range(m):
            o = b * s.y_batch_stride + j * s.y_row_stride
            got[b, j] = yc[o:o + n]
            ymask[o:o + n] = True
    check_tolerance(got, yref, a, "batched")
    assert np.all(yc[~ymask] == 7.0), "y written outside its view"


def test_add_rmsnorm_multipass_matches_single_pass():
    """k = 14336 at m = 8 does not fit LDS in one pass (the fused statistic is
    taken before the passes); every row equals its m = 1 (single-pass) run."""
    t, n, k = wl.Q6_K, 9, 14336
    W = wl.weights(t, n, k, seed=990)
    x = wl.activations(8, k, seed=991)
    r = wl.activations(8, k, seed=992)
    g = (1.0 + 0.1 * wl.activations(1, k, seed=993)[0]).astype(np.float32)
    Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel()), to_dev(g)
    assert qfr.row_exact_schedule(t, n, k, 8).k_chunk < k and qfr.row_exact_schedule(t, n, k, 1).k_chunk >= k
    _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, 8)[1:]
    h8, y8 = _run(t, Wd, xd, rd, gd, 1e-5, n, k, 8)
    check_tolerance(y8.cpu().numpy().reshape(1, 8, n), yref, a, "m=8 multi-pass")
    y8b = bits(y8).reshape(8, n)
    for j in range(8):
        _, y1 = _run(t, Wd, xd[j * k:], rd[j * k:], gd, 1e-5, n, k, 1)
        assert np.array_equal(bits(y1), y8b[j]), f"row {j}: multi-pass m=8 differs from single-pass m=1"
    assert np.array_equal(h8.cpu().numpy(), (x + r).ravel())


@pytest.mark.parametrize("t,n,k", [(wl.Q8_0, 2048, 4160), (wl.F16, 4096, 1028), (wl.Q6_K, 2048, 14336)],
                         ids=["q8_0-single-pass", "f16-short-rows", "q6_k-multi-pass"])
def test_add_rmsnorm_full_workgroups(t, n, k):
    """Enough rows for workgroups of 4 and 8 waves, where a thread keeps one
    virtual lane of the statistic and takes several input rows: every m
    within tolerance, h bit-exact, each row bitwise equal to its m = 1 run."""
    W = wl.weights(t, n, k, seed=1500 + t)
    x = wl.activations(8, k, seed=1501)
    r = wl.activations(8, k, seed=1502)
    g = (1.0 + 0.1 * wl.activations(1, k, seed=1503)[0]).astype(np.float32)
    Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel()), to_dev(g)
    waves = {qfr.row_exact_schedule(t, n, k, m).waves_per_workgroup for m in range(1, 9)}
    assert waves & {4, 8}, waves
    _, _, yref, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, 8)
    y1 = [bits(_run(t, Wd, xd[j * k:], rd[j * k:], gd, 1e-5, n, k, 1)[1]) for j in range(8)]
    for m in range(1, 9):
        h, y = _run(t, Wd, xd, rd, gd, 1e-5, n, k, m)
        check_tolerance(y.cpu().numpy().reshape(1, m, n), yref[:, :m], a[:, :m], f"m={m}")
        assert np.array_equal(h.cpu().numpy(), (x[:m] + r[:m]).ravel()), f"m={m}: h"
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], y1[j]), f"m={m} row {j} differs from its m = 1 run"


def _run_ws(t, Wd, xd, rd, gd, eps, n, k, m, batch=1, strides=None, fill=float("nan")):
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
    y = torch.full((yb // 4,), fill, device="cuda:0")
    h = torch.full((xb // 4,), fill, device="cuda:0")
    # a work buffer full of garbage: the call writes everything it reads
    work = torch.full((qfr.norm_work_bytes(k, m, batch) // 4 + 4,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_add_rmsnorm_ws(t, Wd, xd, rd, gd, eps, h, y, n, k, m, batch, strides, work=work)
    torch.cuda.synchronize()
    return h, y


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("with_g", [True, False])
def test_add_rmsnorm_two_launch_matches_one_kernel(t, with_g):
    """row_exact_mv_add_rmsnorm_ws (statistic in a kernel of its own, then the
    plain product on u) gives every output and h the bits of the one-kernel
    call, at every m."""
    n, k = SHAPES[t]
    W = wl.weights(t, n, k, seed=1600 + t)
    x = wl.activations(8, k, seed=1601 + t)
    r = wl.activations(8, k, seed=1602 + t)
    g = (1.0 + 0.1 * wl.activations(1, k, seed=1603 + t)[0]).astype(np.float32) if with_g else None
    Wd, xd, rd = to_dev(W.ravel()), to_dev(x.ravel()), to_dev(r.ravel())
    gd = to_dev(g) if with_g else None
    for m in range(1, 9):
        h1, y1 = _run(t, Wd, xd, rd, gd, 1e-5, n, k, m)
        h2, y2 = _run_ws(t, Wd, xd, rd, gd, 1e-5, n, k, m)
        assert np.array_equal(bits(y1), bits(y2)), f"m={m}: y differs between the two forms"
        assert np.array_equal(bits(h1), bits(h2)), f"m={m}: h differs between the two forms"


def test_add_rmsnorm_two_launch_batched_and_multipass():
    """Batch-major strided views with gaps (nothing outside them written) and
    a k that needs several LDS passes at m = 8: the two forms agree bitwise."""
    t = wl.Q6_K
    for n, k, m, batch, s in ((29, 4352, 4, 3, Strides(4352 + 8, 5 * (4352 + 8), 29 + 3, 5 * (29 + 3))),
                              (9, 14336, 8, 1, None)):
        W = wl.weights(t, n * batch, k, seed=1700 + k)
        _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
        x = wl.activations(1, xb // 4, seed=1701)[0]
        r = wl.activations(1, xb // 4, seed=1702)[0]
        g = (1.0 + 0.1 * wl.activations(1, k, seed=1703)[0]).astype(np.float32)
        Wd, xd, rd, gd = to_dev(W.ravel()), to_dev(x), to_dev(r), to_dev(g)
        h1, y1 = _run(t, Wd, xd, rd, gd, 1e-6, n, k, m, batch, s)
        h2, y2 = _run_ws(t, Wd, xd, rd, gd, 1e-6, n, k, m, batch, s)
        assert np.array_equal(bits(y1), bits(y2)), f"k={k}: y"
        assert np.array_equal(bits(h1), bits(h2)), f"k={k}: h"
        if s is not None:
            yc = y2.cpu().numpy()
            ymask = np.zeros(yc.size, bool)
            for b in range(batch):
                for j in range(m):
                    o = b * s.y_batch_stride + j * s.y_row_stride
                    ymask[o:o + n] = True
            assert np.all(np.isnan(yc[~ymask])), "y written outside its view"


# ------------------------------------------------------- residual RMS norm


def _run_res(t, Wd, hd, xd, wd, cd, w2d, eps, eps2, n, k, m, batch=1, strides=None, hout="new"):
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
    y = torch.full((yb // 4,), float("nan"), device="cuda:0")
    ho = torch.full((xb // 4,), float("nan"), device="cuda:0") if hout == "new" else hout
    qfr.row_exact_mv_residual_rmsnorm_ws(t, Wd, hd, xd, wd, cd, w2d, eps, eps2, ho, y, n, k, m, batch, strides)
    torch.cuda.synchronize()
    return ho, y


def _check_hs(got, ref, h, what):
    """hs against the oracle: the same float32 steps, the first statistic's
    float64 sum in another order (a last-place difference of the scale can
    move a rounding): within 1e-6 of |h| + |hs| + 1."""
    got, ref = got.astype(np.float64), ref.astype(np.float64)
    lim = 1e-6 * (np.abs(h.astype(np.float64)) + np.abs(ref) + 1.0)
    bad = ~(np.abs(got - ref) <= lim)
    assert not bad.any(), f"{what}: {int(bad.sum())} hs values off, e.g. {got[bad][:3]} vs {ref[bad][:3]}"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("opt", ["all", "none"])
def test_residual_rmsnorm_parity(t, opt):
    """hs within the float32 rounding of the oracle's, y within the
    tolerance, every row of m <= 8 bitwise its m = 1 result, repeatable."""
    n, k = SHAPES[t]
    W = wl.weights(t, n, k, seed=1970 + t)
    h = wl.activations(8, k, seed=1971 + t)
    x = wl.activations(8, k, seed=1972 + t)
    vec = lambda s, c0, sc: (c0 + sc * wl.activations(1, k, seed=s)[0]).astype(np.float32)
    w, c, w2 = ((vec(1973 + t, 1.0, 0.1), vec(1974 + t, 0.7, 0.05), vec(1975 + t, 1.0, 0.1)) if opt == "all"
                else (None, None, None))
    eps, eps2 = 1e-5, 1e-6
    Wd, hd, xd = to_dev(W.ravel()), to_dev(h.ravel()), to_dev(x.ravel())
    wd, cd, w2d = (None if v is None else to_dev(v) for v in (w, c, w2))
    hsref, _, yref, a = oracle.mv_residual_rmsnorm(t, W, h, x, w, c, w2, eps, eps2, n, k, 8)
    ones = []
    for j in range(8):
        _, y1 = _run_res(t, Wd, hd[j * k:], xd[j * k:], wd, cd, w2d, eps, eps2, n, k, 1)
        ones.append(bits(y1))
    for m in (1, 2, 3, 5, 8):
        hs, y = _run_res(t, Wd, hd, xd, wd, cd, w2d, eps, eps2, n, k, m)
        _check_hs(hs.cpu().numpy(), hsref[:m * k], h.ravel()[:m * k], f"m={m}")
        check_tolerance(y.cpu().numpy().reshape(1, m, n), yref[:, :m], a[:, :m], f"m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
    again = bits(_run_res(t, Wd, hd, xd, wd, cd, w2d, eps, eps2, n, k, 8)[1])
    assert np.array_equal(again, bits(_run_res(t, Wd, hd, xd, wd, cd, w2d, eps, eps2, n, k, 8)[1]))


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q6_K, wl.BF16], ids=["Q8_0", "Q6_K", "BF16"])
def test_residual_rmsnorm_x_zero_is_the_add_form(t):
    """With x = 0 the residual form adds nothing to h, and its second
    statistic is summed over the same values in the same order as the add
    form's: hout equals h and y equals the add form's (x := h, r := 0,
    g := w2) bit for bit."""
    n, k, m = SHAPES[t][0], SHAPES[t][1], 5
    W = wl.weights(t, n, k, seed=1980 + t)
    h = wl.activations(m, k, seed=1981 + t)
    w = (1.0 + 0.1 * wl.activations(1, k, seed=1982 + t)[0]).astype(np.float32)
    w2 = (1.0 + 0.1 * wl.activations(1, k, seed=1983 + t)[0]).astype(np.float32)
    Wd, hd, wd, w2d = to_dev(W.ravel()), to_dev(h.ravel()), to_dev(w), to_dev(w2)
    zero = torch.zeros_like(hd)
    hs, y = _run_res(t, Wd, hd, zero, wd, None, w2d, 1e-3, 1e-5, n, k, m)
    y2 = torch.full((m * n,), float("nan"), device="cuda:0")
    qfr.row_exact_mv_add_rmsnorm_ws(t, Wd, hd, zero, w2d, 1e-5, None, y2, n, k, m)
    torch.cuda.synchronize()
    assert np.array_equal(bits(hs), bits(hd))
    assert np.array_equal(bits(y), bits(y2))


@pytest.mark.parametrize("t", [wl.Q8_0, wl.Q4_K, wl.F16], ids=["Q8_0", "Q4_K", "F16"])
def test_residual_rmsnorm_in_place_and_batched(t):
    """hout = h updates the residual stream in place with the bits of a
    separate hout; batch-major strides with gaps against the oracle, elements
    outside the views untouched."""
    n, k = SHAPES[t]
    batch, m = 3, 4
    W = wl.weights(t, n * batch, k, seed=1990 + t)
    s = Strides(k + 12, 5 * (k + 12), n + 3, 5 * (n + 3))
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    h = wl.activations(1, xb // 4, seed=1991 + t)[0]
    x = wl.activations(1, xb // 4, seed=1992 + t)[0]
    w = (1.0 + 0.1 * wl.activations(1, k, seed=1993 + t)[0]).astype(np.float32)
    Wd, xd = to_dev(W.ravel()), to_dev(x)
    hs_sep, y_sep = _run_res(t, Wd, to_dev(h), xd, to_dev(w), None, None, 1e-5, 1e-5, n, k, m, batch, s)
    hd = to_dev(h)
    hs_in, y_in = _run_res(t, Wd, hd, xd, to_dev(w), None, None, 1e-5, 1e-5, n, k, m, batch, s, hout=hd)
    assert hs_in.data_ptr() == hd.data_ptr()
    views = np.zeros(xb // 4, bool)
    for b in range(batch):
        for j in range(m):
            o = b * s.x_batch_stride + j * s.x_row_stride
            views[o:o + k] = True
    hsn, hin = hs_sep.cpu().numpy(), hs_in.cpu().numpy()
    assert np.array_equal(hsn[views].view(np.uint32), hin[views].view(np.uint32))
    assert np.array_equal(hin[~views].view(np.uint32), h[~views].view(np.uint32)), "in place: gaps changed"
    assert np.all(np.isnan(hsn[~views])), "separate hout: gaps written"
    assert np.array_equal(bits(y_sep), bits(y_in))
    hsref, _, yref, a = oracle.mv_residual_rmsnorm(t, W, h, x, w, None, None, 1e-5, 1e-5, n, k, m, batch,
                                                   s.x_row_stride, s.x_batch_stride)
    _check_hs(hsn[views], hsref[views], h[views], "batched")
    got = np.empty((batch, m, n))
    yc = y_sep.cpu().numpy()
    for b in range(batch):
        for j in range(m):
            o = b * s.y_batch_stride + j * s.y_row_stride
            got[b, j] = yc[o:o + n]
    check_tolerance(got, yref, a, "batched")


def test_residual_rmsnorm_several_passes():
    """Q6_K rows of k = 14336 at m = 8 (several LDS passes of the product):
    tolerance against the oracle and row exactness."""
    t, n, k, m = wl.Q6_K, 64, 14336, 8
    W = wl.weights(t, n, k, seed=1995)
    h = wl.activations(m, k, seed=1996)
    x = wl.activations(m, k, seed=1997)
    Wd, hd, xd = to_dev(W.ravel()), to_dev(h.ravel()), to_dev(x.ravel())
    hsref, _, yref, a = oracle.mv_residual_rmsnorm(t, W, h, x, None, None, None, 1e-5, 1e-5, n, k, m)
    hs, y = _run_res(t, Wd, hd, xd, None, None, None, 1e-5, 1e-5, n, k, m)
    _check_hs(hs.cpu().numpy(), hsref, h.ravel(), "k = 14336")
    check_tolerance(y.cpu().numpy().reshape(1, m, n), yref, a, "k = 14336")
    y1 = _run_res(t, Wd, hd[3 * k:], xd[3 * k:], None, None, None, 1e-5, 1e-5, n, k, 1)[1]
    assert np.array_equal(bits(y).reshape(m, n)[3], bits(y1))
