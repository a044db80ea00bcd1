"""Helpers for the GPU parity tests: run the HIP path through the binding,
compare with the oracle."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


def host_threads() -> int:
    """Host threads for oracle work: the CPUs this process may use, at most
    one GPU's share of the box (16)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return max(1, min(avail, 16))


def _ranges(n: int, parts: int) -> list:
    parts = max(1, min(parts, n))
    return [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]


def oracle_full(t, W: np.ndarray, x: np.ndarray, n: int, k: int, m: int, batch: int, xrs: int, xbs: int) -> tuple:
    """The oracle over every output row, ``(y, a)`` [batch, m, n]: the
    unchanged oracle called on disjoint output-row ranges from several host
    threads (each call computes its rows exactly as one call over all rows
    would; the calls run outside the interpreter lock)."""
    y = np.empty((batch, m, n))
    a = np.empty((batch, m, n))

    def work(r):
        lo, hi = r
        yy, aa = oracle.matvec(t, W, x, n, k, m, batch, xrs, xbs, rows=(lo, hi))
        y[..., lo:hi] = yy[..., lo:hi]
        a[..., lo:hi] = aa[..., lo:hi]

    with ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(work, _ranges(n, 4 * host_threads())))
    return y, a


def oracle_dequant_rows(t, W: np.ndarray, r0: int, r1: int, k: int) -> np.ndarray:
    """The oracle's exact weights of rows [r0, r1), over host threads."""
    rb = oracle.row_bytes(t, k)
    flat = W.ravel()
    out = np.empty((r1 - r0, k), dtype=np.float32)

    def work(r):
        lo, hi = r
        out[lo - r0:hi - r0] = oracle.dequant(t, flat[lo * rb:hi * rb], hi - lo, k)

    with ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(lambda r: work((r0 + r[0], r0 + r[1])), _ranges(r1 - r0, 2 * host_threads())))
    return out
