"""The product's own decode: unit input vectors return the weights exactly.

row_exact_dequant checks the per-value decoders; the product decodes the
block types differently (integer-valued q per value, the segment's scale
applied once to the segment's sum, Q4_K's offset by a second fma).  With
input row j equal to the unit vector e_c, every product term is a weight
times 1 or times 0, so each output is that weight: s * q exactly (Q8_0, Q5_0,
Q6_K: the sum of the segment's q * x is q), round(s * q - o) for Q4_K (one
fma, the value the oracle's decode rounds once), the value itself for the
dense types.  Every column class is covered (first and last value of a piece,
of a segment, of a 64-lane wave step, the ragged tail) for rows on 64, 32 and
16 lanes, against oracle.dequant bit for bit; a zero weight may come out as
either zero (the sum starts from +0), so zeros compare by value.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import bits, run_mv, to_dev

pytestmark = pytest.mark.gpu

STEP = {wl.F16: 512, wl.Q8_0: 2048, wl.Q4_K: 4096, wl.Q6_K: 4096, wl.Q5_0: 2048, wl.F32: 256, wl.BF16: 512}
TYPES = list(STEP)
IDS = [wl.TYPE_NAMES[t] for t in TYPES]
# values per piece and per scaled segment (0: unscaled)
PIECE = {t: STEP[t] // 64 for t in TYPES}
SEG = {wl.F16: 0, wl.Q8_0: 32, wl.Q4_K: 32, wl.Q6_K: 16, wl.Q5_0: 32, wl.F32: 0, wl.BF16: 0}


def _ks(t):
    """k of rows on 64 lanes (two steps and a tail of one block / 4 values),
    on 32 lanes (24 pieces; for a block type also 96, half a step past one)
    and on 16 lanes (16 pieces)."""
    tail = 256 if t in (wl.Q4_K, wl.Q6_K) else (32 if t in (wl.Q8_0, wl.Q5_0) else 4)
    out = [2 * STEP[t] + tail, PIECE[t] * 24, PIECE[t] * 16]
    if t in (wl.Q8_0, wl.Q4_K, wl.Q6_K, wl.Q5_0):
        out.append(STEP[t] * 3 // 2)
    return out


def _columns(t, k):
    """Columns at the first and last value of pieces, segments, 64-lane and
    32-lane wave steps (up to 8 boundaries of each, spread over the row) and
    of the row."""
    cols = {0, 1, 3, 4, k - 1, k - 4}
    for unit in (PIECE[t], SEG[t] or PIECE[t], STEP[t], STEP[t] // 2):
        bounds = list(range(unit, k, unit))
        for c in bounds[::max(1, len(bounds) // 8)][:8]:
            cols.update({c - 1, c})
    return sorted(c for c in cols if 0 <= c < k)


@pytest.mark.parametrize("t", TYPES, ids=IDS)
def test_unit_vectors_return_the_weights(t):
    n = 72
    for k in _ks(t):
        W = wl.weights(t, n, k, seed=2600 + t + k)
        ref = oracle.dequant(t, W, n, k)  # [n, k], exact float32
        Wd = to_dev(W.ravel())
        cols = _columns(t, k)
        for i in range(0, len(cols), 8):
            cs = cols[i:i + 8]
            m = len(cs)
            x = np.zeros((m, k), dtype=np.float32)
            for j, c in enumerate(cs):
                x[j, c] = 1.0
            y = run_mv(t, Wd, to_dev(x.ravel()), n, k, m).cpu().numpy().reshape(m, n)
            for j, c in enumerate(cs):
                want = ref[:, c]
                got = y[j]
                nz = want != 0
                assert np.array_equal(got[nz].view(np.uint32), want[nz].view(np.uint32)), \
                    f"k={k} column {c}: product decode differs from the exact weights"
                assert np.all(got[~nz] == 0), f"k={k} column {c}: zero weights"
        torch.cuda.synchronize()
