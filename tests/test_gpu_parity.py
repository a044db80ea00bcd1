"""GPU parity of the HIP path against the oracle, at oracle-friendly sizes
that span several wave steps and end in a ragged tail.

Conditions checked (the acceptance conditions of the row-exact mat-vec):
  1. row_exact_dequant output is bit-identical to the oracle's weights;
  2. |y - y_ref| <= 1e-5 * sum|w x| + 1e-6 against the float64 oracle;
  3. row j of an m-row call is bitwise the m = 1 call on row j
     (mlx-native row_exact_matvec.rs, "Row exactness");
  4. repeated calls are bitwise identical;
plus: every packing schedule gives the same bits, strided/grouped layouts,
ragged n and k tails, and outputs outside the view are never written.
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

# (type, n, k): k spans more than one wave step and ends in a partial one;
# n is not a multiple of any rows-per-wave packing.
SHAPES = {
    wl.F16: (77, 1028),    # 129 pieces of 8 values, the last one half
    wl.Q8_0: (70, 2080),   # 65 blocks
    wl.Q4_K: (67, 4352),   # 17 super-blocks = 68 pieces
    wl.Q6_K: (41, 4352),   # 17 super-blocks = 68 pieces
    wl.Q5_0: (53, 2112),   # 66 blocks
    wl.F32: (69, 1028),    # 257 pieces of 4 values: 4 wave steps and one piece
    wl.BF16: (77, 1028),   # as F16
}
# Rows of 5 wave steps and a ragged 60-piece tail (380 pieces), long enough
# for packings with several LDS passes at every m and, with n < 128, a
# reduction split of 4 waves.
SHAPES64 = {
    wl.F16: (77, 3040), wl.Q8_0: (70, 12160), wl.Q4_K: (67, 24320), wl.Q6_K: (41, 24320),
    wl.Q5_0: (53, 12160), wl.F32: (69, 1520), wl.BF16: (77, 3040),
}
TYPES = list(SHAPES)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]


@pytest.fixture(scope="module")
def data():
    out = {}
    for t, (n, k) in SHAPES.items():
        W = wl.weights(t, n, k, seed=300 + t)
        x = wl.activations(8, k, seed=400 + t)
        y, a = oracle.matvec(t, W, x, n, k, 8)
        out[t] = dict(W=W, x=x, Wd=to_dev(W.ravel()), xd=to_dev(x.ravel()), y=y[0], a=a[0], n=n, k=k)
    return out


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_dequant_bit_exact(t, data):
    d = data[t]
    n, k = d["n"], d["k"]
    out = torch.full((n, k), float("nan"), dtype=torch.float32, device="cuda:0")
    qfr.row_exact_dequant(t, d["Wd"], out, n, k)
    torch.cuda.synchronize()
    ref = oracle.dequant(t, d["W"], n, k)
    got = out.cpu().numpy()
    diff = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
    assert diff.size == 0, f"{diff.shape[0]} weights differ, first {diff[:4].tolist()}: {got[tuple(diff[0])]} vs {ref[tuple(diff[0])]}"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_tolerance_and_row_exactness_every_m(t, data):
    d = data[t]
    n, k = d["n"], d["k"]
    ones = [bits(run_mv(t, d["Wd"], d["xd"][j * k:], n, k, 1)) for j in range(8)]
    for m in range(1, 9):
        y = run_mv(t, d["Wd"], d["xd"], n, k, m)
        got = y.cpu().numpy().reshape(m, n)
        check_tolerance(got, d["y"][:m], d["a"][:m], f"{wl.TYPE_NAMES[t]} m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_repeat_bitwise(t, data):
    d = data[t]
    first = bits(run_mv(t, d["Wd"], d["xd"], d["n"], d["k"], 5))
    for _ in range(3):
        assert np.array_equal(bits(run_mv(t, d["Wd"], d["xd"], d["n"], d["k"], 5)), first)


STEP = {wl.F16: 512, wl.Q8_0: 2048, wl.Q4_K: 4096, wl.Q6_K: 4096, wl.Q5_0: 2048, wl.F32: 256, wl.BF16: 512}


def _schedules(t, K):
    """Packings with reduction split K: waves a multiple of K, LDS passes of
    a multiple of K wave steps."""
    step = STEP[t] * K
    out = []
    for nr in (1, 2, 4):
        for waves, wgs in ((1, 1), (1, 1000), (4, 3), (8, 2), (8, 64), (3, 5), (6, 7)):
            if waves % K == 0:
                out.append(Schedule(K, nr, waves, wgs, 1 << 30))
    out.append(Schedule(K, 2, 8, 4, step))      # several LDS passes
    out.append(Schedule(K, 4, max(2, K), 1, step))
    out.append(Schedule(K, 1, 8 if K > 1 else 5, 7, 2 * step))
    return out


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("m", [1, 3, 8])
def test_packing_is_inert(t, m, data):
    d = data[t]
    n, k = d["n"], d["k"]
    ref = bits(run_mv(t, d["Wd"], d["xd"], n, k, m))
    K = qfr.row_exact_schedule(t, n, k, m).k_split
    for s in _schedules(t, K):
        got = bits(run_mv(t, d["Wd"], d["xd"], n, k, m, schedule=s))
        assert np.array_equal(got, ref), f"schedule {s} changed the bits"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_several_passes_and_split(t):
    """Rows of several wave steps and a ragged tail: tolerance and row
    exactness at m = 1, 3, 8, every packing that fits (several LDS passes
    included, with the derived split) bitwise equal; for the 2-byte-aligned
    types also W 2 bytes past a 4-byte boundary, in one and several passes."""
    n, k = SHAPES64[t]
    W = wl.weights(t, n, k, seed=330 + t)
    x = wl.activations(8, k, seed=430 + t)
    Wd, xd = to_dev(W.ravel()), to_dev(x.ravel())
    ref, a = oracle.matvec(t, W, x, n, k, 8)
    ones = [bits(run_mv(t, Wd, xd[j * k:], n, k, 1)) for j in range(8)]
    for m in (1, 3, 8):
        y = run_mv(t, Wd, xd, n, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, n), ref[0, :m], a[0, :m], f"m={m}")
        yb = bits(y)
        for j in range(m):
            assert np.array_equal(yb.reshape(m, n)[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
        sd = qfr.row_exact_schedule(t, n, k, m)
        K = sd.k_split
        assert K == 4, K
        kc_max = 1 << 30 if sd.k_chunk >= k else sd.k_chunk  # the largest pass that fits at this m
        for s in _schedules(t, K):
            if s.k_chunk <= kc_max:
                assert np.array_equal(bits(run_mv(t, Wd, xd, n, k, m, schedule=s)), yb), f"m={m}: schedule {s}"
        if t in (wl.Q8_0, wl.Q6_K, wl.Q5_0):
            raw = W.ravel()
            buf = torch.zeros(raw.size + 32, dtype=torch.uint8, device="cuda:0")
            buf[2:2 + raw.size].copy_(torch.from_numpy(raw.copy()))
            Wo = buf[2:2 + raw.size]
            for s in (None, Schedule(K, 2, 8, 4, STEP[t])):
                got = bits(run_mv(t, Wo, xd, n, k, m, schedule=s))
                assert np.array_equal(got, yb), f"m={m}: 2-byte-aligned W, schedule {s}"


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_ragged_n_and_minimal_k(t):
    kmin = {wl.F16: 4, wl.Q8_0: 32, wl.Q4_K: 256, wl.Q6_K: 256, wl.Q5_0: 32, wl.F32: 4, wl.BF16: 4}[t]
    for n in (1, 2, 3, 5, 7, 9, 63, 65):
        for k in (kmin, kmin * 3):
            W = wl.weights(t, n, k, seed=500 + n + k)
            x = wl.activations(3, k, seed=600 + n)
            y = run_mv(t, to_dev(W.ravel()), to_dev(x.ravel()), n, k, 3)
            ref, a = oracle.matvec(t, W, x, n, k, 3)
            check_tolerance(y.cpu().numpy().reshape(3, n), ref[0], a[0], f"n={n} k={k}")


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_strided_batched_with_gaps(t):
    """Batch-major and token-major strided layouts; elements outside the
    view keep their sentinel."""
    n, k = 37, {wl.F16: 516, wl.Q8_0: 2080, wl.Q4_K: 2304, wl.Q6_K: 4352, wl.Q5_0: 2112, wl.F32: 516,
                wl.BF16: 516}[t]
    batch, m = 3, 4
    W = wl.weights(t, n * batch, k, seed=700 + t)
    for s in (Strides(k + 12, 5 * (k + 12), n + 3, 5 * (n + 3)),          # batch-major with gaps
              Strides(batch * k + 8, k, batch * n + 5, n)):                  # token-major (grouped) with gaps
        _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
        x = wl.activations(1, xb // 4, seed=800 + t)[0]
        y = run_mv(t, to_dev(W.ravel()), to_dev(x), n, k, m, batch, strides=s, y_elems=yb // 4 + 16)
        yc = y.cpu().numpy()
        ref, a = oracle.matvec(t, W, x, n, k, m, batch, s.x_row_stride, s.x_batch_stride)
        got = gather_y(yc, n, m, batch, s.y_row_stride, s.y_batch_stride)
        check_tolerance(got, ref, a, f"strides {s}")
        mask = np.ones(yc.size, bool)
        for b in range(batch):
            for j in range(m):
                o = b * s.y_batch_stride + j * s.y_row_stride
                mask[o:o + n] = False
        assert np.all(np.isnan(yc[mask])), "an element outside the output view was written"


def test_grouped_token_major_matches_per_group():
    """grouped_token_major(m, G, n, k) == G separate contiguous products,
    bitwise (the split depends on (type, k) only)."""
    t, G, n, k, m = wl.Q5_0, 4, 96, 2048, 8
    W = wl.weights(t, G * n, k, seed=901)
    x = wl.activations(m, G * k, seed=902)
    s = qfr.grouped_token_major(m, G, n, k)
    yg = run_mv(t, to_dev(W.ravel()), to_dev(x.ravel()), n, k, m, G, strides=s).cpu().numpy().reshape(m, G * n)
    rb = qfr.row_exact_row_bytes(t, k)
    for g in range(G):
        Wg = W.ravel()[g * n * rb:(g + 1) * n * rb]
        xg = np.ascontiguousarray(x[:, g * k:(g + 1) * k])
        y1 = run_mv(t, to_dev(Wg), to_dev(xg.ravel()), n, k, m).cpu().numpy().reshape(m, n)
        assert np.array_equal(yg[:, g * n:(g + 1) * n].view(np.uint32), y1.view(np.uint32))


def test_error_leaves_output_untouched(data):
    d = data[wl.Q8_0]
    y = torch.full((8 * d["n"],), 7.0, device="cuda:0")
    before = qfr.row_exact_launch_count()
    with pytest.raises(qfr.RowExactError) as e:
        qfr.row_exact_mv(wl.Q8_0, d["Wd"], d["xd"], y, d["n"], d["k"], 9)
    assert e.value.code == -1
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and qfr.row_exact_launch_count() == before


def test_default_schedule_properties():
    """k_split is a function of (type, k, n): the largest power of two within
    1024 / n, 8 and the row's whole 64-piece wave steps (1 below 3 steps),
    the same for every m and batch; packing fields in range."""
    for t in TYPES:
        for k in (512 if t in wl.DENSE else 4096, 14336 if t in (wl.Q4_K, wl.Q6_K) else 8192):
            steps = k // STEP[t]
            for n in (1, 5, 64, 200, 1023, 1024, 4096, 128256):
                splits = {qfr.row_exact_schedule(t, n, k, m, batch).k_split for m in (1, 4, 8) for batch in (1, 3)}
                assert len(splits) == 1, (t, k, n, splits)
                K = splits.pop()
                assert K in (1, 2, 4, 8) and K * n <= max(1024, n) and K <= max(1, steps)
                if n >= 1024 or steps < 3:
                    assert K == 1
                else:
                    assert 2 * K * n > 1024 or 2 * K > 8 or 2 * K > steps, (t, k, n, K)
            s = qfr.row_exact_schedule(t, 4096, k, 8)
            assert s.rows_per_wave in (1, 2, 4) and 1 <= s.waves_per_workgroup <= 8


# Short rows: a row of at most 16 / 32 pieces is split by 16 / 32 lanes and a
# wave covers 4 / 2 rows at once (the lane map is a function of (type, k)).
SHORT_K = {wl.F16: (124, 252), wl.Q8_0: (512, 1024), wl.Q4_K: (1024, 2048), wl.Q6_K: (1024, 2048),
           wl.Q5_0: (480, 1024), wl.F32: (64, 100), wl.BF16: (60, 256)}
SHORT = [(t, k) for t in TYPES for k in SHORT_K[t]]


@pytest.mark.parametrize("t,k", SHORT, ids=[f"{wl.TYPE_NAMES[t]}-k{k}" for t, k in SHORT])
def test_short_rows_lane_maps(t, k):
    n = 67
    W = wl.weights(t, n, k, seed=950 + t)
    x = wl.activations(8, k, seed=960 + t)
    Wd, xd = to_dev(W.ravel()), to_dev(x.ravel())
    ref, a = oracle.matvec(t, W, x, n, k, 8)
    ones = [bits(run_mv(t, Wd, xd[j * k:], n, k, 1)) for j in range(8)]
    for m in range(1, 9):
        y = run_mv(t, Wd, xd, n, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, n), ref[0, :m], a[0, :m], f"k={k} m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
    base = bits(run_mv(t, Wd, xd, n, k, 3))
    for nr in (1, 2, 4):
        for waves, wgs in ((1, 1), (8, 2), (3, 5), (1, 1000), (4, 3)):
            got = bits(run_mv(t, Wd, xd, n, k, 3, schedule=Schedule(1, nr, waves, wgs, 1 << 30)))
            assert np.array_equal(got, base), f"nr={nr} waves={waves} wgs={wgs} changed the bits"


def test_stream_read_probe_runs_every_shape():
    """The read probe (a measurement aid) accepts every shape on a device
    buffer, including a size that is not a whole KiB."""
    buf = torch.ones(3 * 1024 * 1024 + 48, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    before = qfr.row_exact_launch_count()
    for shape in range(qfr.row_exact_stream_read_shapes()):
        qfr.row_exact_stream_read(buf, buf.numel() // 16 * 16, sink, shape)
    torch.cuda.synchronize()
    assert qfr.row_exact_launch_count() == before + qfr.row_exact_stream_read_shapes()


# The page's validate() accepts Q8_0, Q6_K and Q5_0 weights at any even
# address.  W at a 2-byte offset (the first row then starts 2 bytes past a
# 4-byte boundary and is read from its own start): dequant bit-exact, every
# output against the oracle at every m, row exactness, and the same bits as
# W at an aligned address, for the default and a multi-pass schedule.
TWO_BYTE = [wl.Q8_0, wl.Q6_K, wl.Q5_0]


@pytest.mark.parametrize("t", TWO_BYTE, ids=[wl.TYPE_NAMES[t] for t in TWO_BYTE])
@pytest.mark.parametrize("off", [2, 6, 14])
def test_two_byte_aligned_weights(t, off, data):
    d = data[t]
    n, k = d["n"], d["k"]
    raw = d["W"].ravel()
    buf = torch.zeros(raw.size + 32, dtype=torch.uint8, device="cuda:0")
    buf[off:off + raw.size].copy_(torch.from_numpy(raw.copy()))
    Wo = buf[off:off + raw.size]
    assert Wo.data_ptr() % 4 == 2 and Wo.data_ptr() % 16 == off
    out = torch.full((n, k), float("nan"), dtype=torch.float32, device="cuda:0")
    qfr.row_exact_dequant(t, Wo, out, n, k)
    torch.cuda.synchronize()
    ref = oracle.dequant(t, d["W"], n, k)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    ones = [bits(run_mv(t, Wo, d["xd"][j * k:], n, k, 1)) for j in range(8)]
    step = {wl.Q8_0: 2048, wl.Q6_K: 4096, wl.Q5_0: 2048}[t]
    for m in range(1, 9):
        y = run_mv(t, Wo, d["xd"], n, k, m)
        check_tolerance(y.cpu().numpy().reshape(m, n), d["y"][:m], d["a"][:m], f"off={off} m={m}")
        yb = bits(y).reshape(m, n)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} row {j} differs from its m=1 result"
        assert np.array_equal(bits(y), bits(run_mv(t, d["Wd"], d["xd"], n, k, m))), "differs from aligned W"
        multi = bits(run_mv(t, Wo, d["xd"], n, k, m, schedule=Schedule(1, 2, 8, 4, step)))
        assert np.array_equal(multi, bits(y)), "multi-pass schedule changed the bits"
