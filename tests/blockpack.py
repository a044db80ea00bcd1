"""Test-side block *encoders*: integer fields -> block bytes.

They run in the packing direction (field -> byte and bit position), the
inverse of the oracle's per-value decoders, so a wrong index, shift or mask
in a decoder does not cancel against them.  Each encoder also returns the
exact value of every weight as a ``fractions.Fraction`` computed from the
integer fields, which the tests compare with the oracle's float32 output.

Layouts: the GGML blocks the weight types are named after (field offsets as
in the oracle's header comment); byte sizes from the mlx-native
``row_exact_matvec`` page (block constants).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np


def f16_bits(value: float) -> int:
    return int(np.array([value], dtype=np.float16).view(np.uint16)[0])


def f16_frac(bits: int) -> Fraction:
    """Exact value of a (finite) half bit pattern, via numpy's decoder."""
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def _u16(b: bytearray, off: int, v: int) -> None:
    b[off] = v & 0xFF
    b[off + 1] = (v >> 8) & 0xFF


def enc_q8_0(d_bits: int, q: Sequence[int]) -> Tuple[bytes, List[Fraction]]:
    assert len(q) == 32
    b = bytearray(34)
    _u16(b, 0, d_bits)
    for i, v in enumerate(q):
        b[2 + i] = v & 0xFF
    d = f16_frac(d_bits)
    return bytes(b), [d * v for v in q]


def enc_q5_0(d_bits: int, q: Sequence[int]) -> Tuple[bytes, List[Fraction]]:
    """q: 32 five-bit quants in [0, 31]."""
    assert len(q) == 32 and all(0 <= v < 32 for v in q)
    b = bytearray(22)
    _u16(b, 0, d_bits)
    qh = 0
    for i, v in enumerate(q):
        qh |= ((v >> 4) & 1) << i
    for pos in range(4):
        b[2 + pos] = (qh >> (8 * pos)) & 0xFF
    for byte in range(16):
        b[6 + byte] = (q[byte] & 15) | ((q[byte + 16] & 15) << 4)
    d = f16_frac(d_bits)
    return bytes(b), [d * (v - 16) for v in q]


def pack_q4_k_scales(sc: Sequence[int], mn: Sequence[int]) -> bytes:
    """Eight 6-bit scales and eight 6-bit mins into 12 bytes.

    Bytes 0-3: low 6 bits = sc[0..3], top 2 bits = bits 4-5 of sc[4..7].
    Bytes 4-7: low 6 bits = mn[0..3], top 2 bits = bits 4-5 of mn[4..7].
    Bytes 8-11: low nibble = bits 0-3 of sc[4..7], high nibble = bits 0-3 of mn[4..7].
    """
    assert len(sc) == 8 and len(mn) == 8
    S = bytearray(12)
    for s in range(4):
        S[s] = (sc[s] & 63) | ((sc[s + 4] >> 4) << 6)
        S[s + 4] = (mn[s] & 63) | ((mn[s + 4] >> 4) << 6)
        S[s + 8] = (sc[s + 4] & 15) | ((mn[s + 4] & 15) << 4)
    return bytes(S)


def enc_q4_k(d_bits: int, dmin_bits: int, sc: Sequence[int], mn: Sequence[int],
             q: Sequence[int]) -> Tuple[bytes, List[Fraction]]:
    """q: 256 four-bit quants; sub-block s = v // 32 uses sc[s], mn[s]."""
    assert len(q) == 256
    b = bytearray(144)
    _u16(b, 0, d_bits)
    _u16(b, 2, dmin_bits)
    b[4:16] = pack_q4_k_scales(sc, mn)
    for c in range(4):
        for l in range(32):
            b[16 + 32 * c + l] = (q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4)
    d, dmin = f16_frac(d_bits), f16_frac(dmin_bits)
    vals = [d * sc[v // 32] * q[v] - dmin * mn[v // 32] for v in range(256)]
    return bytes(b), vals


def enc_q6_k(d_bits: int, sc: Sequence[int], q: Sequence[int]) -> Tuple[bytes, List[Fraction]]:
    """q: 256 six-bit quants in [0, 63]; sc: 16 int8 scales (one per 16 values)."""
    assert len(q) == 256 and len(sc) == 16
    b = bytearray(210)
    for h in range(2):
        for l in range(32):
            q0, q1, q2, q3 = (q[128 * h + 32 * t + l] for t in range(4))
            b[64 * h + l] = (q0 & 15) | ((q2 & 15) << 4)
            b[64 * h + 32 + l] = (q1 & 15) | ((q3 & 15) << 4)
            b[128 + 32 * h + l] = (q0 >> 4) | ((q1 >> 4) << 2) | ((q2 >> 4) << 4) | ((q3 >> 4) << 6)
    for g in range(16):
        b[192 + g] = sc[g] & 0xFF
    _u16(b, 208, d_bits)
    d = f16_frac(d_bits)
    return bytes(b), [d * sc[v // 16] * (q[v] - 32) for v in range(256)]


def enc_f16(bits: Sequence[int]) -> Tuple[bytes, List[Fraction]]:
    b = bytearray(2 * len(bits))
    for i, v in enumerate(bits):
        _u16(b, 2 * i, v)
    return bytes(b), [f16_frac(v) for v in bits]


def round_f32(value: Fraction) -> float:
    """Round an exact rational to the nearest float32, ties to even."""
    if value == 0:
        return 0.0
    sign = -1 if value < 0 else 1
    a = abs(value)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, -149)
    n = round(a / Fraction(2) ** q)  # Fraction rounds half to even
    return sign * float(n * Fraction(2) ** q)
