"""GPU parity of the gathered (mixture-of-experts) product against the
oracle, at oracle-friendly sizes, for every weight type: tolerance against
the float64 gathered reference, NaN for ids outside the expert range,
bitwise equality with row_exact_mv on the selected expert's weights, and no
writes outside the output view."""
import numpy as np
import pytest
import torch

import oracle
import quantized_few_row_amd as qfr
import workloads as wl
from gpu_util import bits, check_tolerance, run_mv, to_dev
from quantized_few_row_amd import Strides

pytestmark = pytest.mark.gpu

SHAPES = {wl.F16: (41, 516), wl.Q8_0: (45, 2080), wl.Q4_K: (37, 512), wl.Q6_K: (29, 512), wl.Q5_0: (33, 2112),
          wl.F32: (35, 516), wl.BF16: (39, 516)}
TYPES = list(SHAPES)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]
E = 6


@pytest.mark.parametrize("t", TYPES, ids=IDS)
@pytest.mark.parametrize("m", [1, 3, 8])
def test_gather_matches_oracle_and_plain_product(t, m):
    n, k = SHAPES[t]
    batch = 6
    ids = np.array([4, 0, 4, E + 2, 2, -1], np.int32)
    W = wl.weights(t, E * n, k, seed=900 + t)
    xbs = m * k + 12                                   # per-entry tokens with a gap
    s = Strides(k, xbs, batch * n + 5, n)              # token-major y with a gap
    _, xb, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
    x = wl.activations(1, xb // 4, seed=910 + t)[0]
    Wd, xd = to_dev(W.ravel()), to_dev(x)
    y = torch.full((yb // 4 + 16,), 7.0, device="cuda:0")
    qfr.row_exact_mv_gather(t, Wd, E, torch.from_numpy(ids).to("cuda:0"), xd, y, n, k, m, batch, s)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    ref, a = oracle.matvec_gather(t, W, E, ids, x, n, k, m, batch, s.x_row_stride, xbs)
    rb = qfr.row_exact_row_bytes(t, k)
    mask = np.ones(yc.size, bool)
    for b, e in enumerate(ids):
        got = np.stack([yc[b * n + j * s.y_row_stride: b * n + j * s.y_row_stride + n] for j in range(m)])
        for j in range(m):
            mask[b * n + j * s.y_row_stride: b * n + j * s.y_row_stride + n] = False
        if e < 0 or e >= E:
            assert np.all(np.isnan(got)), f"entry {b} (id {e}) not NaN"
            continue
        check_tolerance(got[None], ref[b][None], a[b][None], f"entry {b} id {e}")
        ye = run_mv(t, to_dev(W.ravel()[e * n * rb:(e + 1) * n * rb]), to_dev(x[b * xbs:]), n, k, m)
        assert np.array_equal(bits(ye).reshape(m, n).view(np.uint32), got.view(np.uint32)), \
            f"entry {b} differs from row_exact_mv"
    assert np.all(yc[mask] == 7.0), "an element outside the output view was written"
