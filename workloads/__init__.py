"""Seeded synthetic inputs for the row-exact few-row mat-vec.

This module only draws random bytes and writes them into block fields.  It
decodes nothing and computes no product: both the oracle and the HIP path
take its output as input, and neither is imported here.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), vectorised over a counter:
output ``i`` of stream ``seed`` is ``mix(seed + (i + 1) * 0x9E3779B97F4A7C15)``.
Normals use the Box-Muller transform in float64.  Half-precision fields are
rounded to nearest-even by numpy's float64 -> float16 conversion.

Block field offsets follow the GGML block structs named by the weight types
(Q8_0, Q4_K, Q6_K, Q5_0); the byte sizes are those of the mlx-native
``row_exact_matvec`` page (block constants).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

F16, Q8_0, Q4_K, Q6_K, Q5_0, F32, BF16 = 0, 1, 2, 3, 4, 5, 6
TYPE_NAMES = {F16: "F16", Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q5_0: "Q5_0", F32: "F32", BF16: "BF16"}
NAME_TYPES = {v: k for k, v in TYPE_NAMES.items()}

# (values per block, bytes per block)
BLOCK = {F16: (1, 2), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210), Q5_0: (32, 22), F32: (1, 4), BF16: (1, 2)}
DENSE = (F16, F32, BF16)

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, count: int, offset: int = 0) -> np.ndarray:
    """``count`` outputs of SplitMix64 stream ``seed`` starting at output ``offset``."""
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


class Stream:
    """Sequential draws from one SplitMix64 stream."""

    def __init__(self, seed: int):
        self.seed = seed
        self.pos = 0

    def u64(self, count: int) -> np.ndarray:
        out = splitmix64(self.seed, count, self.pos)
        self.pos += count
        return out

    def bytes(self, count: int) -> np.ndarray:
        words = self.u64((count + 7) // 8)
        return words.view(np.uint8)[:count].copy()

    def uniform(self, count: int) -> np.ndarray:
        """Doubles in [0, 1) from the top 53 bits."""
        return (self.u64(count) >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))

    def normal(self, count: int) -> np.ndarray:
        """Standard normals, Box-Muller in float64 (one normal per pair)."""
        u1 = self.uniform(count)
        u2 = self.uniform(count)
        return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)

    def ints(self, count: int, lo: int, hi: int) -> np.ndarray:
        """Integers uniform on [lo, hi] (inclusive), via floor(u * span)."""
        span = hi - lo + 1
        return (np.floor(self.uniform(count) * span).astype(np.int64) + lo)


def _f16_bits(values: np.ndarray) -> np.ndarray:
    return values.astype(np.float16).view(np.uint16)


def _bf16_bits(values: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest even) -> bfloat16 (nearest even on the
    float32 bits; the values drawn here are finite)."""
    u = values.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _put_u16(blocks: np.ndarray, offset: int, bits: np.ndarray) -> None:
    blocks[:, offset] = (bits & 0xFF).astype(np.uint8)
    blocks[:, offset + 1] = (bits >> 8).astype(np.uint8)


def weights(wtype: int, rows: int, k: int, seed: int) -> np.ndarray:
    """Row-major weight bytes, ``rows`` rows of ``k`` values, drawn as in the
    synthetic workload recipe:

    - F16: N(0, 0.02) rounded to half.
    - F32: N(0, 0.02) rounded to float32.
    - BF16: N(0, 0.02) rounded to float32, then to bfloat16 (nearest even).
    - Q8_0: d = half(|N(0,1)| * 0.01); 32 int8 uniform on [-127, 127].
    - Q4_K: d, dmin = half(|N(0,1)| * 0.01); 12 scale bytes and 128 quant bytes
      uniform (all 6-bit scales/mins and 4-bit quants uniform).
    - Q6_K: 128 low-bit and 64 high-bit bytes uniform; 16 int8 scales uniform
      on [-64, 63]; d = half(|N(0,1)| * 0.001).
    - Q5_0: d = half(|N(0,1)| * 0.01); 4 high-bit and 16 nibble bytes uniform.
    """
    per, nbytes = BLOCK[wtype]
    if k % (4 if wtype in DENSE else per):
        raise ValueError(f"k={k} is not a multiple of the block size of {TYPE_NAMES[wtype]}")
    s = Stream(seed)
    if wtype == F16:
        vals = s.normal(rows * k) * 0.02
        return _f16_bits(vals).view(np.uint8).reshape(rows, 2 * k).copy()
    if wtype == F32:
        vals = s.normal(rows * k) * 0.02
        return vals.astype(np.float32).view(np.uint8).reshape(rows, 4 * k).copy()
    if wtype == BF16:
        vals = s.normal(rows * k) * 0.02
        return _bf16_bits(vals).view(np.uint8).reshape(rows, 2 * k).copy()
    nblk = rows * (k // per)
    blocks = s.bytes(nblk * nbytes).reshape(nblk, nbytes)
    if wtype == Q8_0:
        _put_u16(blocks, 0, _f16_bits(np.abs(s.normal(nblk)) * 0.01))
        blocks[:, 2:34] = s.ints(nblk * 32, -127, 127).astype(np.int8).view(np.uint8).reshape(nblk, 32)
    elif wtype == Q4_K:
        _put_u16(blocks, 0, _f16_bits(np.abs(s.normal(nblk)) * 0.01))
        _put_u16(blocks, 2, _f16_bits(np.abs(s.normal(nblk)) * 0.01))
    elif wtype == Q6_K:
        blocks[:, 192:208] = s.ints(nblk * 16, -64, 63).astype(np.int8).view(np.uint8).reshape(nblk, 16)
        _put_u16(blocks, 208, _f16_bits(np.abs(s.normal(nblk)) * 0.001))
    elif wtype == Q5_0:
        _put_u16(blocks, 0, _f16_bits(np.abs(s.normal(nblk)) * 0.01))
    else:
        raise ValueError(f"unknown weight type {wtype}")
    return blocks.reshape(rows, (k // per) * nbytes)


def activations(rows: int, cols: int, seed: int) -> np.ndarray:
    """``rows x cols`` float32 ~ N(0, 1)."""
    return Stream(seed).normal(rows * cols).astype(np.float32).reshape(rows, cols)


def row_bytes(wtype: int, k: int) -> int:
    per, nbytes = BLOCK[wtype]
    return (k // per) * nbytes


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: weight type, shape, strides and the m set."""

    name: str
    wtype: int
    n: int
    k: int
    batch: int
    ms: Tuple[int, ...]
    index: int
    grouped: bool = False
    experts: int = 0  # > 0: gathered product, batch entry b uses weight set ids[b] of `experts`
    fused_norm: bool = False  # input produced by the fused add + RMS norm (x + r, weight g)

    @property
    def w_seed(self) -> int:
        return 1000 + self.index

    @property
    def x_seed(self) -> int:
        return 2000 + self.index

    def strides(self, m: int) -> Tuple[int, int, int, int]:
        """(x_row, x_batch, y_row, y_batch) in elements."""
        if self.grouped:
            return (self.batch * self.k, self.k, self.batch * self.n, self.n)
        if self.experts:
            # every selected expert multiplies the same tokens; y token-major [m, batch * n]
            return (self.k, 0, self.batch * self.n, self.n)
        return (self.k, 0, self.n, 0)

    @property
    def weight_bytes(self) -> int:
        """Weight bytes one call reads."""
        return row_bytes(self.wtype, self.k) * self.n * self.batch

    @property
    def stored_weight_bytes(self) -> int:
        """Weight bytes held (every expert's set for a gathered product)."""
        return row_bytes(self.wtype, self.k) * self.n * (self.experts or self.batch)

    def make_weights(self) -> np.ndarray:
        return weights(self.wtype, self.n * (self.experts or self.batch), self.k, self.w_seed)

    def make_residual(self, m: int = 8) -> np.ndarray:
        """r for the fused add + RMS norm, shaped like make_x (seed 4000 + index)."""
        cols = self.batch * self.k if self.grouped else self.k
        return activations(8, cols, 4000 + self.index)[:m].copy()

    def make_norm_weight(self) -> np.ndarray:
        """g for the fused add + RMS norm: 1 + 0.1 N(0, 1), float32 (seed 5000 + index)."""
        return (1.0 + 0.1 * Stream(5000 + self.index).normal(self.k)).astype(np.float32)

    def make_ids(self) -> np.ndarray:
        """The batch entries' distinct expert ids (seeded), int32."""
        u = Stream(3000 + self.index).uniform(self.experts)
        return np.argsort(u, kind="stable")[:self.batch].astype(np.int32)

    def make_x(self, m: int = 8) -> np.ndarray:
        """x for ``m`` rows (drawn as 8 rows; an m-row run uses rows 0..m-1).

        Contiguous layout: shape ``[m, k]``.  Grouped token-major layout:
        shape ``[m, batch * k]``.
        """
        cols = self.batch * self.k if self.grouped else self.k
        return activations(8, cols, self.x_seed)[:m].copy()


# The workload configurations of the row-exact mat-vec (index = seed offset).
WORKLOADS: List[Workload] = [
    Workload("f16_256x512", F16, 256, 512, 1, tuple(range(1, 9)), 0),
    Workload("q8_0_4096x4096", Q8_0, 4096, 4096, 1, (1, 4, 8), 1),
    Workload("q4_k_14336x4096", Q4_K, 14336, 4096, 1, tuple(range(1, 9)), 2),
    Workload("q6_k_4096x14336", Q6_K, 4096, 14336, 1, (1, 8), 3),
    Workload("q6_k_128256x4096", Q6_K, 128256, 4096, 1, (1, 8), 4),
    Workload("q5_0_16x1024x4096_grouped", Q5_0, 1024, 4096, 16, (8,), 5, grouped=True),
    # dense weights under the same contract (a 4096 x 4096 projection)
    Workload("f32_4096x4096", F32, 4096, 4096, 1, (1, 4, 8), 6),
    Workload("bf16_4096x4096", BF16, 4096, 4096, 1, (1, 4, 8), 7),
    # mixture-of-experts decode: 8 of 64 Q4_K experts (1408 x 2048) for the same tokens
    Workload("q4_k_moe_64x1408x2048_top8", Q4_K, 1408, 2048, 8, (1, 4, 8), 8, experts=64),
    # the Q8_0 projection with its input made by the fused add + RMS norm (eps 1e-5)
    Workload("q8_0_4096x4096_add_rmsnorm", Q8_0, 4096, 4096, 1, (1, 4, 8), 9, fused_norm=True),
    # held-out shapes: never used to tune the schedule chooser; the decode
    # shapes the row-exact page reports measurements for (Q4_K 1024 x 2816,
    # Q8_0 2816 x 2112, rows x k, m = 1..4)
    Workload("q4_k_1024x2816", Q4_K, 1024, 2816, 1, (1, 2, 3, 4), 10),
    Workload("q8_0_2816x2112", Q8_0, 2816, 2112, 1, (1, 2, 3, 4), 11),
]
# skinny outputs (few rows, long rows): the reduction split across waves
# (k_split > 1) against single-wave rows; a router-like F16 64 x 4096, a
# single-output F16 head, and quantized projections of 32..128 rows
SKINNY_WORKLOADS: List[Workload] = [
    Workload("f16_64x4096", F16, 64, 4096, 1, (1, 4, 8), 12),
    Workload("f16_1x8192", F16, 1, 8192, 1, (1, 4, 8), 13),
    Workload("bf16_128x8192", BF16, 128, 8192, 1, (1, 4, 8), 14),
    Workload("q8_0_128x16384", Q8_0, 128, 16384, 1, (1, 4, 8), 15),
    Workload("q4_k_64x14336", Q4_K, 64, 14336, 1, (1, 4, 8), 16),
    Workload("q6_k_32x14336", Q6_K, 32, 14336, 1, (1, 4, 8), 17),
]
WORKLOADS += SKINNY_WORKLOADS
# Rows whose last 64-lane wave step is at most half full (64 s + r pieces,
# 0 < r <= 32): the block types take 32 lanes per row there, the dense ones
# keep 64 (bench.py --lane-sweep times both maps).
LANE_MAP_WORKLOADS: List[Workload] = [
    Workload("q8_0_4096x3072", Q8_0, 4096, 3072, 1, (1, 2, 4, 8), 18),
    Workload("q8_0_4096x11008", Q8_0, 4096, 11008, 1, (1, 2, 4, 8), 19),
    Workload("q4_k_4096x4352", Q4_K, 4096, 4352, 1, (1, 2, 4, 8), 20),
    Workload("q6_k_4096x6144", Q6_K, 4096, 6144, 1, (1, 2, 4, 8), 21),
    Workload("q5_0_16x1024x11008_grouped", Q5_0, 1024, 11008, 16, (1, 2, 4, 8), 22, grouped=True),
    Workload("f16_4096x1792", F16, 4096, 1792, 1, (1, 2, 4, 8), 23),
]
WORKLOADS += LANE_MAP_WORKLOADS
HELD_OUT = ("q4_k_1024x2816", "q8_0_2816x2112")
# Large inputs at m = 1 and 2 for the chooser's rules on few input rows
# (bench.py --schedule-sweep checks it on them; not full-size parity cases):
# staged x leaving room for one or two workgroups per CU, with enough rows for
# two per wave on every wave of one workgroup per CU; and rows that would give
# each of 32 waves per CU between one and two rows.
LARGE_WORKLOADS: List[Workload] = [
    Workload("q8_0_16384x11008", Q8_0, 16384, 11008, 1, (1, 2), 24),
    Workload("q6_k_16384x14336", Q6_K, 16384, 14336, 1, (1, 2), 25),
    Workload("q4_k_14336x14336", Q4_K, 14336, 14336, 1, (1, 2), 26),
    Workload("q8_0_4096x8192", Q8_0, 4096, 8192, 1, (1, 2), 27),
    Workload("q4_k_14336x8192", Q4_K, 14336, 8192, 1, (1, 2), 28),
    Workload("q8_0_14336x4096", Q8_0, 14336, 4096, 1, (1, 2), 29),
    Workload("q6_k_14336x8192", Q6_K, 14336, 8192, 1, (1, 2), 30),
    Workload("q4_k_14336x6144", Q4_K, 14336, 6144, 1, (1, 2), 31),
]
LARGE = ("q5_0_16x1024x11008_grouped",) + tuple(w.name for w in LARGE_WORKLOADS)
SKINNY = tuple(w.name for w in SKINNY_WORKLOADS)
LANE_MAP = ("q6_k_4096x14336",) + tuple(w.name for w in LANE_MAP_WORKLOADS)
BY_NAME: Dict[str, Workload] = {w.name: w for w in WORKLOADS + LARGE_WORKLOADS}


def get(name: str) -> Workload:
    return BY_NAME[name]


def scaled(w: Workload, n: Optional[int] = None, k: Optional[int] = None,
           batch: Optional[int] = None) -> Workload:
    """Same recipe and seeds at a different size (for oracle-sized tests)."""
    return dataclasses.replace(w, name=w.name + "_scaled", n=n or w.n, k=k or w.k,
                               batch=batch or w.batch)
