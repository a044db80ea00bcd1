"""Helpers for the GPU parity tests: run the HIP path through the binding,
compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_few_row_amd as qfr

TOL_REL = 1e-5   # |y - y_ref| <= 1e-5 * sum|w x| + 1e-6
TOL_ABS = 1e-6


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def run_mv(t, Wd: torch.Tensor, xd: torch.Tensor, n: int, k: int, m: int, batch: int = 1,
           strides=None, schedule=None, y_elems: int | None = None, fill: float = float("nan"),
           x_offset: int = 0) -> torch.Tensor:
    """Run the mat-vec into a fresh y buffer (filled with ``fill``); returns y."""
    if y_elems is None:
        _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
        y_elems = yb // 4
    y = torch.full((y_elems,), fill, dtype=torch.float32, device=dev())
    xv = xd[x_offset:] if x_offset else xd
    if schedule is None:
        qfr.row_exact_mv(t, Wd, xv, y, n, k, m, batch, strides)
    else:
        qfr.row_exact_mv_scheduled(t, Wd, xv, y, n, k, m, batch, strides, schedule)
    torch.cuda.synchronize()
    return y


def gather_y(y: np.ndarray, n: int, m: int, batch: int, yrs: int, ybs: int) -> np.ndarray:
    """Strided y -> dense [batch, m, n]."""
    out = np.empty((batch, m, n), dtype=y.dtype)
    for b in range(batch):
        for j in range(m):
            o = b * ybs + j * yrs
            out[b, j] = y[o:o + n]
    return out


def check_tolerance(got: np.ndarray, ref: np.ndarray, absum: np.ndarray, what: str = "") -> float:
    got = got.astype(np.float64)
    lim = TOL_REL * absum + TOL_ABS
    err = np.abs(got - ref)
    bad = ~(err <= lim)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside tolerance, e.g. at {idx.tolist()}: "
                             f"got {got[tuple(idx[0])]} ref {ref[tuple(idx[0])]} lim {lim[tuple(idx[0])]}")
    return float((err / lim).max()) if err.size else 0.0


def oracle_sampled(t, W: np.ndarray, x: np.ndarray, n: int, k: int, m: int, batch: int, xrs: int, xbs: int,
                   rows: list) -> tuple:
    """Oracle outputs for the given output rows only; returns (y, a) [batch, m, len(rows)]."""
    ys = np.empty((batch, m, len(rows)))
    as_ = np.empty((batch, m, len(rows)))
    for c, i in enumerate(rows):
        y, a = oracle.matvec(t, W, x, n, k, m, batch, xrs, xbs, rows=(i, i + 1))
        ys[:, :, c] = y[:, :, i]
        as_[:, :, c] = a[:, :, i]
    return ys, as_
