"""Row-exact few-row mat-vec for MI355X: Python binding of ``librow_exact_mv.so``.

Argument marshalling only.  Every function here has the name of the C entry
point it calls (``include/row_exact_mv.h``); the work runs in the library's
HIP kernels on the caller's current HIP stream.  PyTorch only supplies device
memory (tensors) and the stream handle.

If the shared library has not been built, importing works but every call
raises :class:`LibraryMissing` -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import enum
import os
from typing import Any, Optional, Tuple

__all__ = [
    "Weight", "Strides", "Schedule", "RowExactError", "LibraryMissing", "MAX_ROWS",
    "contiguous", "grouped_token_major", "library_path", "load_library",
    "row_exact_mv", "row_exact_mv_scheduled", "row_exact_mv_gather", "row_exact_mv_add_rmsnorm",
    "row_exact_mv_add_rmsnorm_ws", "norm_work_bytes", "row_exact_mv_add_rmsnorm_noalloc", "NOALLOC_SCRATCH_BYTES",
    "row_exact_schedule", "row_exact_row_bytes",
    "row_exact_required_bytes", "row_exact_dequant", "row_exact_last_error", "row_exact_launch_count",
    "row_exact_stream_read", "row_exact_stream_read_shapes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librow_exact_mv.so")

MAX_ROWS = 8
NOALLOC_SCRATCH_BYTES = 4 << 20  # ROW_EXACT_NOALLOC_SCRATCH_BYTES

ERRORS = {-1: "EARG", -2: "EALIGN", -3: "ESTRIDE", -4: "EALIAS", -5: "EEXTENT", -6: "ESCHEDULE", -7: "EHIP"}


class Weight(enum.IntEnum):
    """Weight storage (``row_exact_weight_t``)."""
    F16 = 0
    Q8_0 = 1
    Q4_K = 2
    Q6_K = 3
    Q5_0 = 4
    F32 = 5
    BF16 = 6


class Strides(ctypes.Structure):
    """``row_exact_strides_t``: element strides of x and y."""
    _fields_ = [("x_row_stride", ctypes.c_uint32), ("x_batch_stride", ctypes.c_uint32),
                ("y_row_stride", ctypes.c_uint32), ("y_batch_stride", ctypes.c_uint32)]

    def astuple(self) -> Tuple[int, int, int, int]:
        return (self.x_row_stride, self.x_batch_stride, self.y_row_stride, self.y_batch_stride)

    def __repr__(self) -> str:
        return "Strides(%d, %d, %d, %d)" % self.astuple()


class Schedule(ctypes.Structure):
    """``row_exact_schedule_t``."""
    _fields_ = [("k_split", ctypes.c_uint32), ("rows_per_wave", ctypes.c_uint32),
                ("waves_per_workgroup", ctypes.c_uint32), ("workgroups_per_batch", ctypes.c_uint32),
                ("k_chunk", ctypes.c_uint32), ("lanes_per_row", ctypes.c_uint32)]

    def asdict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}

    def __repr__(self) -> str:
        return "Schedule(%s)" % ", ".join("%s=%d" % kv for kv in self.asdict().items())


class RowExactError(RuntimeError):
    """A non-zero status from the library; ``code`` is the ROW_EXACT_E* value."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{ERRORS.get(code, code)}] {message}")
        self.code = code
        self.message = message


class LibraryMissing(RuntimeError):
    pass


def contiguous(m: int, n: int, k: int) -> Strides:
    """x [m, k], y [m, n], batch strides 0 (RowExactMatvecShape::contiguous)."""
    return Strides(k, 0, n, 0)


def grouped_token_major(m: int, groups: int, n: int, k: int) -> Strides:
    """x [m, groups*k], W [groups*n, k], y [m, groups*n]; use batch = groups
    (RowExactMatvecShape::grouped_token_major)."""
    return Strides(groups * k, k, groups * n, n)


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LibraryMissing(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                             "(or python -m quantized_few_row_amd._build)")
    _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_variant(path: str) -> ctypes.CDLL:
    """Another build of the library (e.g. one with a code-generation switch
    overridden, ``python -m quantized_few_row_amd._build --out PATH -D ...``),
    with the same ctypes signatures, for interleaved comparisons."""
    if not os.path.exists(path):
        raise LibraryMissing(f"{path} is not built")
    return _declare(ctypes.CDLL(os.path.abspath(path)))


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
    SP, SchP = ctypes.POINTER(Strides), ctypes.POINTER(Schedule)
    lib.row_exact_mv.restype = ctypes.c_int
    lib.row_exact_mv.argtypes = [ctypes.c_int, P, P, P, u32, u32, u32, u32, SP, P]
    lib.row_exact_mv_scheduled.restype = ctypes.c_int
    lib.row_exact_mv_scheduled.argtypes = [ctypes.c_int, P, P, P, u32, u32, u32, u32, SP, SchP, P]
    lib.row_exact_mv_gather.restype = ctypes.c_int
    lib.row_exact_mv_gather.argtypes = [ctypes.c_int, P, u32, P, P, P, u32, u32, u32, u32, SP, P]
    lib.row_exact_mv_add_rmsnorm.restype = ctypes.c_int
    lib.row_exact_mv_add_rmsnorm.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_float, P, P, u32, u32, u32, u32, SP, P]
    lib.row_exact_mv_add_rmsnorm_noalloc.restype = ctypes.c_int
    lib.row_exact_mv_add_rmsnorm_noalloc.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_float, P, P, u32, u32, u32, u32,
                                                     SP, P]
    lib.row_exact_mv_add_rmsnorm_ws.restype = ctypes.c_int
    lib.row_exact_mv_add_rmsnorm_ws.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_float, P, P, u32, u32, u32, u32, SP,
                                                P, u64, P]
    lib.row_exact_mv_residual_rmsnorm_ws.restype = ctypes.c_int
    lib.row_exact_mv_residual_rmsnorm_ws.argtypes = [ctypes.c_int, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, P,
                                                     P, u32, u32, u32, u32, SP, P, u64, P]
    lib.row_exact_schedule.restype = ctypes.c_int
    lib.row_exact_schedule.argtypes = [ctypes.c_int, u32, u32, u32, u32, SchP]
    lib.row_exact_row_bytes.restype = u64
    lib.row_exact_row_bytes.argtypes = [ctypes.c_int, u32]
    lib.row_exact_required_bytes.restype = ctypes.c_int
    lib.row_exact_required_bytes.argtypes = [ctypes.c_int, u32, u32, u32, u32, SP, ctypes.POINTER(u64),
                                             ctypes.POINTER(u64), ctypes.POINTER(u64)]
    lib.row_exact_dequant.restype = ctypes.c_int
    lib.row_exact_dequant.argtypes = [ctypes.c_int, P, P, u32, u32, P]
    lib.row_exact_last_error.restype = ctypes.c_char_p
    lib.row_exact_last_error.argtypes = []
    lib.row_exact_launch_count.restype = u64
    lib.row_exact_launch_count.argtypes = []
    lib.row_exact_stream_read.restype = ctypes.c_int
    lib.row_exact_stream_read.argtypes = [P, u64, P, u32, P]
    lib.row_exact_stream_read_shapes.restype = u32
    lib.row_exact_stream_read_shapes.argtypes = []
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise RowExactError(rc, load_library().row_exact_last_error().decode())


def _ptr_and_bytes(t: Any, what: str) -> Tuple[int, Optional[int]]:
    """(device pointer, byte length or None) of a torch tensor or a raw int."""
    if isinstance(t, int):
        return t, None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what} must be a GPU tensor or a device pointer")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (strides are given in elements to the call)")
    return t.data_ptr(), t.numel() * t.element_size()


def _stream_handle(stream: Any) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_check(wt: Weight, W: Any, x: Any, y: Any) -> None:
    if isinstance(W, int):
        return
    import torch
    want = {Weight.F16: torch.float16, Weight.F32: torch.float32, Weight.BF16: torch.bfloat16}.get(wt, torch.uint8)
    if W.dtype not in (want, torch.uint8):
        raise ValueError(f"{wt.name} weight must be {want} (or raw uint8 bytes), got {W.dtype}")
    for t, name in ((x, "x"), (y, "y")):
        if not isinstance(t, int) and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")


def _size_check(wt: Weight, W, x, y, n, k, m, batch, strides) -> None:
    wb, xb, yb = row_exact_required_bytes(wt, n, k, m, batch, strides)
    for t, need, name in ((W, wb, "weight"), (x, xb, "input"), (y, yb, "output")):
        _, have = _ptr_and_bytes(t, name)
        if have is not None and have < need:
            raise ValueError(f"{name} holds {have} bytes, needs {need}")


def row_exact_mv(wt: int, W: Any, x: Any, y: Any, n: int, k: int, m: int, batch: int = 1,
                 strides: Optional[Strides] = None, stream: Any = None) -> None:
    """Enqueue ``y[b, j, :] = W[b] . x[b, j, :]`` (see ``row_exact_mv`` in the header)."""
    wt = Weight(wt)
    lib = load_library()
    _dtype_check(wt, W, x, y)
    _size_check(wt, W, x, y, n, k, m, batch, strides)
    wp, _ = _ptr_and_bytes(W, "weight")
    xp, _ = _ptr_and_bytes(x, "input")
    yp, _ = _ptr_and_bytes(y, "output")
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib.row_exact_mv(int(wt), wp, xp, yp, n, k, m, batch, sp, _stream_handle(stream)))


def row_exact_mv_scheduled(wt: int, W: Any, x: Any, y: Any, n: int, k: int, m: int, batch: int,
                           strides: Optional[Strides], schedule: Schedule, stream: Any = None) -> None:
    """As :func:`row_exact_mv` with a pinned schedule."""
    wt = Weight(wt)
    lib = load_library()
    _dtype_check(wt, W, x, y)
    _size_check(wt, W, x, y, n, k, m, batch, strides)
    wp, _ = _ptr_and_bytes(W, "weight")
    xp, _ = _ptr_and_bytes(x, "input")
    yp, _ = _ptr_and_bytes(y, "output")
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib.row_exact_mv_scheduled(int(wt), wp, xp, yp, n, k, m, batch, sp, ctypes.byref(schedule),
                                      _stream_handle(stream)))


def row_exact_mv_gather(wt: int, W: Any, num_experts: int, expert_ids: Any, x: Any, y: Any, n: int, k: int,
                        m: int, batch: int, strides: Optional[Strides] = None, stream: Any = None) -> None:
    """Enqueue ``y[b, j, :] = W[expert_ids[b]] . x[b, j, :]`` (see ``row_exact_mv_gather``)."""
    wt = Weight(wt)
    lib = load_library()
    _dtype_check(wt, W, x, y)
    _, xb, yb = row_exact_required_bytes(wt, n, k, m, batch, strides)
    wb = row_exact_row_bytes(wt, k) * n * num_experts
    for t, need, name in ((W, wb, "weight"), (x, xb, "input"), (y, yb, "output"), (expert_ids, 4 * batch, "expert_ids")):
        _, have = _ptr_and_bytes(t, name)
        if have is not None and have < need:
            raise ValueError(f"{name} holds {have} bytes, needs {need}")
    if not isinstance(expert_ids, int):
        import torch
        if expert_ids.dtype != torch.int32:
            raise ValueError(f"expert_ids must be int32, got {expert_ids.dtype}")
    wp, _ = _ptr_and_bytes(W, "weight")
    ip, _ = _ptr_and_bytes(expert_ids, "expert_ids")
    xp, _ = _ptr_and_bytes(x, "input")
    yp, _ = _ptr_and_bytes(y, "output")
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib.row_exact_mv_gather(int(wt), wp, num_experts, ip, xp, yp, n, k, m, batch, sp, _stream_handle(stream)))


def _norm_call(entry: str, wt: int, W: Any, x: Any, r: Any, g: Any, eps: float, h: Any, y: Any, n: int, k: int,
               m: int, batch: int, strides: Optional[Strides], stream: Any, extra: tuple = ()) -> None:
    wt = Weight(wt)
    lib = load_library()
    _dtype_check(wt, W, x, y)
    _size_check(wt, W, x, y, n, k, m, batch, strides)
    _, xb, _ = row_exact_required_bytes(wt, n, k, m, batch, strides)
    for t, need, name in ((r, xb, "r"), (h, xb, "h"), (g, 4 * k, "g")):
        if t is None:
            continue
        _, have = _ptr_and_bytes(t, name)
        if have is not None and have < need:
            raise ValueError(f"{name} holds {have} bytes, needs {need}")
    ptr = lambda t, name: None if t is None else _ptr_and_bytes(t, name)[0]
    sp = ctypes.byref(strides) if strides is not None else None
    _check(getattr(lib, entry)(int(wt), ptr(W, "weight"), ptr(x, "input"), ptr(r, "r"), ptr(g, "g"), float(eps),
                               ptr(h, "h"), ptr(y, "output"), n, k, m, batch, sp, *extra, _stream_handle(stream)))


def row_exact_mv_add_rmsnorm(wt: int, W: Any, x: Any, r: Any, g: Any, eps: float, h: Any, y: Any, n: int, k: int,
                             m: int, batch: int = 1, strides: Optional[Strides] = None, stream: Any = None) -> None:
    """Enqueue ``h = x + r``, ``x' = h / sqrt(mean(h^2) + eps) * g``,
    ``y = W . x'`` per input row (see ``row_exact_mv_add_rmsnorm``); ``g`` and
    ``h`` may be None."""
    _norm_call("row_exact_mv_add_rmsnorm", wt, W, x, r, g, eps, h, y, n, k, m, batch, strides, stream)


def norm_work_bytes(k: int, m: int, batch: int = 1) -> int:
    """Bytes of the work buffer of :func:`row_exact_mv_add_rmsnorm_ws`
    (ROW_EXACT_NORM_WORK_BYTES)."""
    return ((batch * m * k * 4 + 255) & ~255) + batch * m * 8


def row_exact_mv_add_rmsnorm_ws(wt: int, W: Any, x: Any, r: Any, g: Any, eps: float, h: Any, y: Any, n: int, k: int,
                                m: int, batch: int = 1, strides: Optional[Strides] = None, work: Any = None,
                                stream: Any = None) -> None:
    """:func:`row_exact_mv_add_rmsnorm` as two launches on a work buffer
    (same bits; see ``row_exact_mv_add_rmsnorm_ws``).  ``work``: a GPU tensor
    or device pointer of at least :func:`norm_work_bytes` bytes; None takes
    one from torch's caching allocator on the call's stream."""
    need = norm_work_bytes(k, m, batch)
    if work is None:
        # torch's caching allocator reuses a block only after the stream it was
        # taken on has passed its last use, so the buffer is taken on the
        # call's own stream (a raw handle cannot be given to torch)
        if isinstance(stream, int):
            raise ValueError("pass work explicitly when the stream is a raw handle")
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            work = torch.empty(need, dtype=torch.uint8, device=s.device)
    wp, wlen = _ptr_and_bytes(work, "work")
    _norm_call("row_exact_mv_add_rmsnorm_ws", wt, W, x, r, g, eps, h, y, n, k, m, batch, strides, stream,
               (wp, need if wlen is None else wlen))

def _work_buffer(need: int, work: Any, stream: Any) -> Tuple[int, int]:
    """(pointer, bytes) of a work buffer: the caller's, or one from torch's
    caching allocator on the call's stream."""
    if work is None:
        # torch's caching allocator reuses a block only after the stream it was
        # taken on has passed its last use, so the buffer is taken on the
        # call's own stream (a raw handle cannot be given to torch)
        if isinstance(stream, int):
            raise ValueError("pass work explicitly when the stream is a raw handle")
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            work = torch.empty(need, dtype=torch.uint8, device=s.device)
    wp, wlen = _ptr_and_bytes(work, "work")
    return wp, need if wlen is None else wlen


def row_exact_mv_residual_rmsnorm_ws(wt: int, W: Any, h: Any, x: Any, w: Any, c: Any, w2: Any, eps: float,
                                     eps2: float, hout: Any, y: Any, n: int, k: int, m: int, batch: int = 1,
                                     strides: Optional[Strides] = None, work: Any = None,
                                     stream: Any = None) -> None:
    """Enqueue ``hs = (h + x / sqrt(mean(x^2) + eps) * w) * c`` (written to
    ``hout`` unless None; ``hout`` may be ``h``) and
    ``y = W . (hs / sqrt(mean(hs^2) + eps2) * w2)`` per input row (see
    ``row_exact_mv_residual_rmsnorm_ws``); ``w``, ``c``, ``w2`` may be None.
    ``work`` as in :func:`row_exact_mv_add_rmsnorm_ws`."""
    wt = Weight(wt)
    lib = load_library()
    _dtype_check(wt, W, x, y)
    _size_check(wt, W, x, y, n, k, m, batch, strides)
    _, xb, _ = row_exact_required_bytes(wt, n, k, m, batch, strides)
    for t, need, name in ((h, xb, "h"), (hout, xb, "hout"), (w, 4 * k, "w"), (c, 4 * k, "c"), (w2, 4 * k, "w2")):
        if t is None:
            continue
        _, have = _ptr_and_bytes(t, name)
        if have is not None and have < need:
            raise ValueError(f"{name} holds {have} bytes, needs {need}")
    wp, wlen = _work_buffer(norm_work_bytes(k, m, batch), work, stream)
    ptr = lambda t, name: None if t is None else _ptr_and_bytes(t, name)[0]
    sp = ctypes.byref(strides) if strides is not None else None
    _check(lib.row_exact_mv_residual_rmsnorm_ws(int(wt), ptr(W, "weight"), ptr(h, "h"), ptr(x, "input"), ptr(w, "w"),
                                                ptr(c, "c"), ptr(w2, "w2"), float(eps), float(eps2), ptr(hout, "hout"),
                                                ptr(y, "output"), n, k, m, batch, sp, wp, wlen,
                                                _stream_handle(stream)))


def row_exact_mv_add_rmsnorm_noalloc(wt: int, W: Any, x: Any, r: Any, g: Any, eps: float, h: Any, y: Any, n: int,
                                     k: int, m: int, batch: int = 1, strides: Optional[Strides] = None,
                                     stream: Any = None) -> None:
    """:func:`row_exact_mv_add_rmsnorm_ws` without any allocation (the
    library's fixed scratch array; see ``row_exact_mv_add_rmsnorm_noalloc``)."""
    _norm_call("row_exact_mv_add_rmsnorm_noalloc", wt, W, x, r, g, eps, h, y, n, k, m, batch, strides, stream)


def row_exact_schedule(wt: int, n: int, k: int, m: int, batch: int = 1) -> Schedule:
    """Default schedule for a shape on the current device."""
    s = Schedule()
    _check(load_library().row_exact_schedule(int(wt), n, k, m, batch, ctypes.byref(s)))
    return s


def row_exact_row_bytes(wt: int, k: int) -> int:
    return int(load_library().row_exact_row_bytes(int(wt), k))


def row_exact_required_bytes(wt: int, n: int, k: int, m: int, batch: int = 1,
                             strides: Optional[Strides] = None) -> Tuple[int, int, int]:
    """(weight, input, output) bytes the call touches."""
    w, x, y = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    sp = ctypes.byref(strides) if strides is not None else None
    _check(load_library().row_exact_required_bytes(int(wt), n, k, m, batch, sp, ctypes.byref(w),
                                                   ctypes.byref(x), ctypes.byref(y)))
    return w.value, x.value, y.value


def row_exact_dequant(wt: int, W: Any, out: Any, rows: int, k: int, stream: Any = None) -> None:
    """Enqueue ``out[r, v] = float32 value of weight v of row r``."""
    lib = load_library()
    wp, wlen = _ptr_and_bytes(W, "weight")
    op, olen = _ptr_and_bytes(out, "out")
    need_w = row_exact_row_bytes(wt, k) * rows
    if wlen is not None and wlen < need_w:
        raise ValueError(f"weight holds {wlen} bytes, needs {need_w}")
    if olen is not None and olen < rows * k * 4:
        raise ValueError(f"out holds {olen} bytes, needs {rows * k * 4}")
    _check(lib.row_exact_dequant(int(wt), wp, op, rows, k, _stream_handle(stream)))


def row_exact_last_error() -> str:
    return load_library().row_exact_last_error().decode()


def row_exact_launch_count() -> int:
    return int(load_library().row_exact_launch_count())


def row_exact_stream_read_shapes() -> int:
    """Launch shapes the read probe accepts (``include/row_exact_probe.h``)."""
    return int(load_library().row_exact_stream_read_shapes())


def row_exact_stream_read(W: Any, nbytes: int, sink: Any, shape: int = 0, stream: Any = None) -> None:
    """Enqueue a plain read of ``nbytes`` of ``W`` (the attainable-read-rate
    probe of ``include/row_exact_probe.h``; not part of the mat-vec)."""
    wp, wlen = _ptr_and_bytes(W, "buffer")
    sp, slen = _ptr_and_bytes(sink, "sink")
    if wlen is not None and wlen < nbytes:
        raise ValueError(f"buffer holds {wlen} bytes, {nbytes} requested")
    if slen is not None and slen < 4:
        raise ValueError("sink must hold 4 bytes")
    _check(load_library().row_exact_stream_read(wp, nbytes, sp, shape, _stream_handle(stream)))
