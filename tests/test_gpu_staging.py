"""The x staging paths against the oracle.

Up to 4 input rows, x is requested ahead of the weights in one batch of a
few 16-byte chunks per thread; whatever a batch does not cover (large k, few
threads per workgroup) is staged behind the weights.  From 5 rows on, half
of a workgroup's waves request their weights after the staging barrier.
These cases take k past what the first batch covers, at 1 and 8 waves per
workgroup (m = 1..4, one LDS pass; m = 5..8 with the default schedule,
several passes at these k), and check the tolerance against the float64
oracle and that every row of an m-row call is bitwise its m = 1 result."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import bits, check_tolerance, run_mv, to_dev
from quantized_few_row_amd import Schedule

pytestmark = pytest.mark.gpu

# (type, k): one LDS pass at m <= 4, and more 16-byte chunks than a
# 512-thread workgroup requests ahead of the weights (4 per thread at
# m = 2..4: 8192 values; 2 at m = 1: 4096).
CASES = [(wl.Q8_0, 8832), (wl.Q4_K, 9216), (wl.Q6_K, 9216), (wl.F32, 8832)]
N = 1031  # n >= 1024: one wave per output (no split), the path these cases stage for


@pytest.mark.parametrize("t,k", CASES, ids=[f"{wl.TYPE_NAMES[t]}-k{k}" for t, k in CASES])
@pytest.mark.parametrize("waves", [1, 8])
def test_x_staged_beyond_the_first_batch(t, k, waves):
    W = wl.weights(t, N, k, seed=900 + t)
    x = wl.activations(8, k, seed=910 + t)
    Wd, xd = to_dev(W.ravel()), to_dev(x.ravel())
    ref, a = oracle.matvec(t, W, x, N, k, 8)
    sched = Schedule(1, 1, waves, 4, 1 << 30)
    ones = [bits(run_mv(t, Wd, xd[j * k:(j + 1) * k], N, k, 1, schedule=sched)) for j in range(8)]
    for m in range(1, 9):
        y = run_mv(t, Wd, xd, N, k, m, schedule=sched if m <= 4 else None)
        got = y.cpu().numpy().reshape(m, N)
        check_tolerance(got, ref[0][:m], a[0][:m], f"m={m} waves={waves}")
        yb = bits(y).reshape(m, N)
        for j in range(m):
            assert np.array_equal(yb[j], ones[j]), f"m={m} waves={waves}: row {j} differs from its m=1 result"
