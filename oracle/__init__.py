"""Oracle for the row-exact few-row mat-vec (CPU, float64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``quantized_few_row_amd``) never imports, loads or calls it, and this
package imports nothing from the product path.

The arithmetic lives in ``row_exact_oracle.c`` (plain C, built with gcc).
This module only marshals numpy arrays in and out.

What it computes (mlx-native 0.18.0, ``src/ops/row_exact_matvec.rs``, module
docs and "Batched / grouped products"; for dense float32 / bfloat16 weights
the same product under nuvec-core 0.6.0 ``src/gpu.rs``'s row-independence
contract of ``gemv_rows``): for batch ``b``, input row ``j`` and output ``i``,
``y[b, j, i] = sum_kk Wd[b*n + i, kk] * x[b*xbs + j*xrs + kk]`` and
``a[b, j, i] = sum_kk |Wd[b*n + i, kk] * x[...]|``, both in float64, where
``Wd`` is the exact float32 value of each weight decoded from its block.

Every function here is pinned by the ``not gpu`` tests in
``tests/test_oracle.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "row_exact_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, Q8_0, Q4_K, Q6_K, Q5_0, F32, BF16 = 0, 1, 2, 3, 4, 5, 6

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        u32 = ctypes.c_uint32
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f32_from_bits.restype = ctypes.c_float
        lib.oracle_f32_from_bits.argtypes = [ctypes.c_uint32]
        lib.oracle_row_bytes.restype = ctypes.c_uint64
        lib.oracle_row_bytes.argtypes = [ctypes.c_int, u32]
        lib.oracle_weight.restype = ctypes.c_float
        lib.oracle_weight.argtypes = [ctypes.c_int, P, u32]
        lib.oracle_dequant.restype = ctypes.c_int
        lib.oracle_dequant.argtypes = [ctypes.c_int, P, u32, u32, P]
        lib.oracle_matvec_rows.restype = ctypes.c_int
        lib.oracle_matvec_rows.argtypes = [ctypes.c_int, P, P, u32, u32, u32, u32, u32, u32, u32, u32, P, P]
        lib.oracle_mv_residual_rmsnorm.restype = ctypes.c_int
        lib.oracle_mv_residual_rmsnorm.argtypes = [ctypes.c_int, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                                   u32, u32, u32, u32, u32, u32, P, P, P, P]
        lib.oracle_mv_add_rmsnorm.restype = ctypes.c_int
        lib.oracle_mv_add_rmsnorm.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_float, u32, u32, u32, u32, u32,
                                              u32, P, P, P, P]
        lib.oracle_matvec_gather.restype = ctypes.c_int
        lib.oracle_matvec_gather.argtypes = [ctypes.c_int, P, u32, P, P, u32, u32, u32, u32, u32, u32, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode uint16 half-precision bit patterns (one call per value)."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    for i, b in enumerate(flat.tolist()):
        out[i] = lib.oracle_f16_to_f32(b)
    return out.reshape(np.shape(bits))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode uint16 bfloat16 bit patterns (one call per value)."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    for i, b in enumerate(flat.tolist()):
        out[i] = lib.oracle_bf16_to_f32(b)
    return out.reshape(np.shape(bits))


def f32_from_bits(bits: np.ndarray) -> np.ndarray:
    """Decode uint32 binary32 bit patterns (one call per value)."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint32).ravel()
    out = np.empty(flat.size, dtype=np.float32)
    for i, b in enumerate(flat.tolist()):
        out[i] = lib.oracle_f32_from_bits(b)
    return out.reshape(np.shape(bits))


def row_bytes(wtype: int, k: int) -> int:
    return int(_load().oracle_row_bytes(wtype, k))


def dequant(wtype: int, W: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Exact float32 weights, shape ``[rows, k]``."""
    lib = _load()
    Wb = np.ascontiguousarray(W, dtype=np.uint8).ravel()
    need = row_bytes(wtype, k) * rows
    if Wb.size < need:
        raise ValueError(f"weight holds {Wb.size} bytes, needs {need}")
    out = np.empty((rows, k), dtype=np.float32)
    if lib.oracle_dequant(wtype, _ptr(Wb), rows, k, _ptr(out)) != 0:
        raise ValueError("oracle_dequant: bad type or k")
    return out


def matvec(wtype: int, W: np.ndarray, x: np.ndarray, n: int, k: int, m: int, batch: int = 1,
           x_row_stride: Optional[int] = None, x_batch_stride: int = 0,
           rows: Optional[Tuple[int, int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Float64 reference ``(y, a)``, each shaped ``[batch, m, n]``.

    ``x`` is a flat float32 buffer addressed with the element strides.
    ``rows=(i0, i1)`` restricts the work to outputs ``i0 <= i < i1`` (others
    are NaN).
    """
    lib = _load()
    xrs = k if x_row_stride is None else x_row_stride
    Wb = np.ascontiguousarray(W, dtype=np.uint8).ravel()
    xf = np.ascontiguousarray(x, dtype=np.float32).ravel()
    need_w = row_bytes(wtype, k) * n * batch
    need_x = (batch - 1) * x_batch_stride + (m - 1) * xrs + k
    if Wb.size < need_w or xf.size < need_x:
        raise ValueError("oracle.matvec: buffers too small")
    y = np.full((batch, m, n), np.nan, dtype=np.float64)
    a = np.full((batch, m, n), np.nan, dtype=np.float64)
    i0, i1 = (0, n) if rows is None else rows
    rc = lib.oracle_matvec_rows(wtype, _ptr(Wb), _ptr(xf), n, k, m, batch, xrs, x_batch_stride, i0, i1,
                                _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_matvec_rows failed ({rc})")
    return y, a


def matvec_gather(wtype: int, W: np.ndarray, num_experts: int, ids: np.ndarray, x: np.ndarray, n: int, k: int,
                  m: int, batch: int, x_row_stride: Optional[int] = None,
                  x_batch_stride: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Float64 reference ``(y, a)`` of the gathered product, each ``[batch, m, n]``:
    batch entry ``b`` uses weight set ``ids[b]``; ids outside the sets give NaN."""
    lib = _load()
    xrs = k if x_row_stride is None else x_row_stride
    Wb = np.ascontiguousarray(W, dtype=np.uint8).ravel()
    ib = np.ascontiguousarray(ids, dtype=np.int32).ravel()
    xf = np.ascontiguousarray(x, dtype=np.float32).ravel()
    if Wb.size < row_bytes(wtype, k) * n * num_experts or ib.size < batch:
        raise ValueError("oracle.matvec_gather: buffers too small")
    if xf.size < (batch - 1) * x_batch_stride + (m - 1) * xrs + k:
        raise ValueError("oracle.matvec_gather: input too small")
    y = np.empty((batch, m, n), dtype=np.float64)
    a = np.empty((batch, m, n), dtype=np.float64)
    rc = lib.oracle_matvec_gather(wtype, _ptr(Wb), num_experts, _ptr(ib), _ptr(xf), n, k, m, batch, xrs,
                                  x_batch_stride, _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_matvec_gather failed ({rc})")
    return y, a


def mv_add_rmsnorm(wtype: int, W: np.ndarray, x: np.ndarray, r: np.ndarray, g: Optional[np.ndarray], eps: float,
                   n: int, k: int, m: int, batch: int = 1, x_row_stride: Optional[int] = None,
                   x_batch_stride: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Float64 reference of the product with a fused add + RMS norm of its
    input: returns ``(h, xn, y, a)``; ``h`` (float32) in x's flat layout,
    ``xn`` [batch, m, k] float64, ``y`` and ``a`` [batch, m, n]."""
    lib = _load()
    xrs = k if x_row_stride is None else x_row_stride
    Wb = np.ascontiguousarray(W, dtype=np.uint8).ravel()
    xf = np.ascontiguousarray(x, dtype=np.float32).ravel()
    rf = np.ascontiguousarray(r, dtype=np.float32).ravel()
    need_x = (batch - 1) * x_batch_stride + (m - 1) * xrs + k
    if Wb.size < row_bytes(wtype, k) * n * batch or xf.size < need_x or rf.size < need_x:
        raise ValueError("oracle.mv_add_rmsnorm: buffers too small")
    gf = None if g is None else np.ascontiguousarray(g, dtype=np.float32).ravel()
    if gf is not None and gf.size < k:
        raise ValueError("oracle.mv_add_rmsnorm: g too small")
    h = np.full(xf.size, np.nan, dtype=np.float32)
    xn = np.empty((batch, m, k), dtype=np.float64)
    y = np.empty((batch, m, n), dtype=np.float64)
    a = np.empty((batch, m, n), dtype=np.float64)
    rc = lib.oracle_mv_add_rmsnorm(wtype, _ptr(Wb), _ptr(xf), _ptr(rf), None if gf is None else _ptr(gf), eps, n,
                                   k, m, batch, xrs, x_batch_stride, _ptr(h), _ptr(xn), _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_mv_add_rmsnorm failed ({rc})")
    return h, xn, y, a


def mv_residual_rmsnorm(wtype: int, W: np.ndarray, h: np.ndarray, x: np.ndarray, w: Optional[np.ndarray],
                        c: Optional[np.ndarray], w2: Optional[np.ndarray], eps: float, eps2: float, n: int, k: int,
                        m: int, batch: int = 1, x_row_stride: Optional[int] = None,
                        x_batch_stride: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Float64 reference of the product whose input is the residual RMS
    normalisation: ``hs = (h + rms_norm(x) * w) * c`` (float32 steps) and
    ``xn = rms_norm(hs) * w2``.  Returns ``(hs, xn, y, a)``; ``hs`` (float32)
    in x's flat layout, ``xn`` [batch, m, k] float64, ``y`` and ``a``
    [batch, m, n].  ``w``, ``c``, ``w2``: k float32 values or None (1, no
    scaling, 1)."""
    lib = _load()
    xrs = k if x_row_stride is None else x_row_stride
    Wb = np.ascontiguousarray(W, dtype=np.uint8).ravel()
    hf = np.ascontiguousarray(h, dtype=np.float32).ravel()
    xf = np.ascontiguousarray(x, dtype=np.float32).ravel()
    need_x = (batch - 1) * x_batch_stride + (m - 1) * xrs + k
    if Wb.size < row_bytes(wtype, k) * n * batch or xf.size < need_x or hf.size < need_x:
        raise ValueError("oracle.mv_residual_rmsnorm: buffers too small")
    vecs = []
    for v in (w, c, w2):
        vf = None if v is None else np.ascontiguousarray(v, dtype=np.float32).ravel()
        if vf is not None and vf.size < k:
            raise ValueError("oracle.mv_residual_rmsnorm: weight vector too small")
        vecs.append(vf)
    hs = np.full(xf.size, np.nan, dtype=np.float32)
    xn = np.empty((batch, m, k), dtype=np.float64)
    y = np.empty((batch, m, n), dtype=np.float64)
    a = np.empty((batch, m, n), dtype=np.float64)
    rc = lib.oracle_mv_residual_rmsnorm(wtype, _ptr(Wb), _ptr(hf), _ptr(xf),
                                        *[None if v is None else _ptr(v) for v in vecs], eps, eps2, n, k, m, batch,
                                        xrs, x_batch_stride, _ptr(hs), _ptr(xn), _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError(f"oracle_mv_residual_rmsnorm failed ({rc})")
    return hs, xn, y, a
