"""Inputs whose staged x fills more than a third of a CU's LDS.

With m*k*4 bytes of x (plus pads) over about 53 KB, one workgroup's stage
leaves room for at most one more on a CU, and the default schedule launches
one workgroup per CU, two rows per wave at m = 2 where every wave still gets
a row group.  Packing is inert: its bits must equal a pinned schedule of one
row group per wave (several rounds of workgroups), and its outputs stay
within the float64 oracle's tolerance (row ranges at the start, middle and
end of every batch entry).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import bits, check_tolerance, run_mv, to_dev
from quantized_few_row_amd import Schedule, Strides, row_exact_schedule

pytestmark = pytest.mark.gpu

# (type, n, k, batch, m): x stages of 92 KB (Q8_0 k = 10240 at m = 2 and
# k = 20480 at m = 1, 64-lane rows), 99 KB (Q5_0 k = 11008 at m = 2, 32-lane
# rows), 122 KB (Q6_K k = 14336 at m = 2, piece-major, 32-lane rows), 72 KB
# (Q8_0 k = 8192 at m = 2) and 57 KB (Q4_K k = 14336 at m = 1, 32-lane rows)
SHAPES = [
    (wl.Q8_0, 4096, 10240, 1, 2),
    (wl.Q8_0, 4096, 20480, 1, 1),
    (wl.Q5_0, 1024, 11008, 8, 2),
    (wl.Q6_K, 4096, 14336, 2, 2),
    (wl.Q8_0, 4096, 8192, 1, 2),
    (wl.Q4_K, 4096, 14336, 2, 1),
]
# The other rules for few input rows on large inputs (x of 16-24 KB, several
# workgroups per CU): rows that give each of 32 waves per CU between one and
# two of them (single rows on 24 waves per CU; Q8_0 14336 x 4096 at m = 1),
# and rows of several wave steps at m = 2 (16 waves per CU; Q4_K 14336 x 6144,
# 32-lane rows).  Only the bits and the tolerance are checked for these.
OTHER = [
    (wl.Q8_0, 14336, 4096, 1, 1),
    (wl.Q4_K, 14336, 6144, 1, 2),
]
IDS = [f"{wl.TYPE_NAMES[t]}_{b}x{n}x{k}_m{m}" for t, n, k, b, m in SHAPES + OTHER]


@pytest.mark.parametrize("shape", SHAPES + OTHER, ids=IDS)
def test_one_round_default_is_inert_and_within_tolerance(shape):
    t, n, k, batch, m = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    d = row_exact_schedule(t, n, k, m, batch)
    assert d.k_split == 1 and d.k_chunk >= k
    if shape in SHAPES:
        assert d.workgroups_per_batch * batch <= cus + batch - 1, d.asdict()
    W = wl.weights(t, n * batch, k, seed=3100 + 100 * t + m)
    x = wl.activations(batch * m, k, seed=3200 + 100 * t + m)
    Wd, xd = to_dev(W.ravel()), to_dev(x.ravel())
    st = Strides(k, m * k, n, m * n)  # dense [batch, m, k] inputs, [batch, m, n] outputs
    y = bits(run_mv(t, Wd, xd, n, k, m, batch, st))
    many = Schedule(1, 1, 8, 1 << 30, 1 << 30, d.lanes_per_row)
    assert np.array_equal(y, bits(run_mv(t, Wd, xd, n, k, m, batch, st, schedule=many))), \
        "default packing differs from one row group per wave"
    assert np.array_equal(y, bits(run_mv(t, Wd, xd, n, k, m, batch, st))), "repeat differs"
    got = y.view(np.float32).reshape(batch, m, n)
    for lo, hi in ((0, 64), (n // 2 - 32, n // 2 + 32), (n - 64, n)):
        ref, a = oracle.matvec(t, W, x, n, k, m, batch, k, m * k, rows=(lo, hi))
        check_tolerance(got[..., lo:hi], ref[..., lo:hi], a[..., lo:hi], f"rows {lo}..{hi}")
