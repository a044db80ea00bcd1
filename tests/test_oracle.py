"""Pins for the oracle (CPU only).

Each test checks the oracle against something other than itself: the page's
printed constants, hand-worked blocks, test-side encoders that run in the
packing direction, numpy's half decoder, exact rational arithmetic, and
closed forms (unit vectors, constant weights, grouped == per-group).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from blockpack import (enc_f16, enc_q4_k, enc_q5_0, enc_q6_k, enc_q8_0, f16_bits, round_f32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TYPES = {"F16": wl.F16, "Q8_0": wl.Q8_0, "Q4_K": wl.Q4_K, "Q6_K": wl.Q6_K, "Q5_0": wl.Q5_0,
         "F32": wl.F32, "BF16": wl.BF16}


def _bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- constants

def test_row_bytes_match_page_constants():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    for name, blk in g["blocks"].items():
        if name.startswith("_"):
            continue
        for nblk in (1, 2, 7, 16, 56):
            k = blk["values"] * nblk
            assert oracle.row_bytes(TYPES[name], k) == blk["bytes"] * nblk
    for k in (4, 8, 512, 4096):
        assert oracle.row_bytes(wl.F16, k) == g["f16_bytes_per_value"]["value"] * k
        assert oracle.row_bytes(wl.F32, k) == 4 * k and oracle.row_bytes(wl.BF16, k) == 2 * k


@pytest.mark.parametrize("name", ["F16", "Q8_0", "Q4_K", "Q6_K", "Q5_0", "F32", "BF16"])
def test_row_locality(name):
    """Row r decodes from bytes [r*rb, (r+1)*rb) only: the parser consumes
    exactly row_bytes per row."""
    t = TYPES[name]
    k = 64 if t in wl.DENSE else 512
    rows = 4
    W = wl.weights(t, rows, k, seed=11)
    full = oracle.dequant(t, W, rows, k)
    rb = oracle.row_bytes(t, k)
    flat = W.ravel()
    for r in range(rows):
        alone = oracle.dequant(t, flat[r * rb:(r + 1) * rb].copy(), 1, k)
        assert np.array_equal(_bits32(alone[0]), _bits32(full[r]))
    # A byte change inside row 2 changes row 2 only.
    W2 = flat.copy()
    W2[2 * rb + rb // 2] ^= 0x5A
    d2 = oracle.dequant(t, W2, rows, k)
    for r in range(rows):
        same = np.array_equal(_bits32(d2[r]), _bits32(full[r]))
        assert same == (r != 2)


# ---------------------------------------------------------------- half floats

def test_f16_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(_bits32(ours[~nan]), _bits32(ref[~nan]))


def test_bf16_exhaustive_against_bit_widening():
    """bfloat16 is the upper half of a binary32: numpy's reinterpretation of
    the widened bits is the reference for all 65536 patterns."""
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_to_f32(bits)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(_bits32(ours[~nan]), _bits32(ref[~nan]))
    # a few by hand: 1.0, -2.0, pi rounded, the smallest subnormal, -0
    hand = oracle.bf16_to_f32(np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x8000], np.uint16))
    assert hand[:3].tolist() == [1.0, -2.0, 3.140625] and hand[3] == 2.0 ** -133
    assert _bits32(hand[4]) == 0x80000000


def test_f32_decode_against_numpy():
    rng = np.random.default_rng(5)
    bits = np.concatenate([rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32),
                           np.array([0, 1, 0x80000000, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x3F800000,
                                     0xFF7FFFFF, 0x7F800000, 0xFF800000], np.uint32)])
    ours = oracle.f32_from_bits(bits)
    ref = bits.view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(_bits32(ours[~nan]), _bits32(ref[~nan]))


def test_dense_weights_decode_as_numpy_views():
    """F32 rows are float32 values as stored; BF16 rows widen bit for bit."""
    for t in (wl.F32, wl.BF16):
        W = wl.weights(t, 3, 36, seed=71)
        d = oracle.dequant(t, W, 3, 36)
        if t == wl.F32:
            ref = W.ravel().view(np.float32).reshape(3, 36)
        else:
            ref = (W.ravel().view(np.uint16).astype(np.uint32) << 16).view(np.float32).reshape(3, 36)
        assert np.array_equal(_bits32(d), _bits32(ref))


def test_bf16_generator_rounds_to_nearest_even():
    """The BF16 recipe rounds float32 to the nearest bfloat16, ties to even."""
    from workloads import _bf16_bits
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20],
                 np.float64)
    got = (_bf16_bits(f).astype(np.uint32) << 16).view(np.float32)
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -1.0, 1.0 + 2 ** -7]


# ---------------------------------------------------------------- hand-worked blocks

def test_hand_worked_blocks():
    g = json.load(open(os.path.join(GOLDEN, "hand_blocks.json")))
    for case in g["cases"]:
        t = TYPES[case["type"]]
        raw = np.frombuffer(bytes.fromhex(case["hex"]), dtype=np.uint8)
        got = oracle.dequant(t, raw, 1, case["k"])[0]
        for idx, want in case["expect"].items():
            v = got[int(idx)]
            assert v == want and np.signbit(v) == np.signbit(want), (case["type"], idx, v, want)


# ---------------------------------------------------------------- encoders (packing direction)

def _check(t, raw, exact, k):
    got = oracle.dequant(t, np.frombuffer(raw, dtype=np.uint8), 1, k)[0]
    want = np.array([round_f32(v) for v in exact], dtype=np.float32)
    # Fractions carry no sign of zero; zeros are compared by value here and
    # their sign is pinned by test_sign_of_zero.
    bad = np.nonzero((_bits32(got) != _bits32(want)) & ~((got == 0) & (want == 0)))[0]
    assert bad.size == 0, (t, bad[:8], got[bad[:8]], want[bad[:8]])


def test_q8_0_roundtrip():
    rng = np.random.default_rng(1)
    for trial in range(20):
        q = rng.integers(-128, 128, 32).tolist()
        d = f16_bits(float(rng.standard_normal()) * 0.03)
        raw, exact = enc_q8_0(d, q)
        _check(wl.Q8_0, raw, exact, 32)


def test_q5_0_roundtrip():
    rng = np.random.default_rng(2)
    for trial in range(20):
        q = rng.integers(0, 32, 32).tolist()
        d = f16_bits(abs(float(rng.standard_normal())) * 0.01)
        raw, exact = enc_q5_0(d, q)
        _check(wl.Q5_0, raw, exact, 32)


def test_q4_k_roundtrip():
    rng = np.random.default_rng(3)
    for trial in range(20):
        sc = rng.integers(0, 64, 8).tolist()
        mn = rng.integers(0, 64, 8).tolist()
        q = rng.integers(0, 16, 256).tolist()
        d = f16_bits(abs(float(rng.standard_normal())) * 0.01)
        dm = f16_bits(abs(float(rng.standard_normal())) * 0.01)
        raw, exact = enc_q4_k(d, dm, sc, mn, q)
        _check(wl.Q4_K, raw, exact, 256)


def test_q4_k_single_rounding():
    """d*sc*q - dmin*mn is rounded once: pick fields whose exact difference
    needs more than 24 bits, so a two-rounding evaluation would differ."""
    d = f16_bits(1.0 + 2.0 ** -10)      # 11 significant bits
    dm = f16_bits(2.0 ** -14 * 1.5)     # tiny min: the difference spans > 24 bits
    sc = [63] * 8
    mn = [63] * 8
    q = [15] * 256
    raw, exact = enc_q4_k(d, dm, sc, mn, q)
    assert any(Fraction(round_f32(v)) != v for v in exact)
    _check(wl.Q4_K, raw, exact, 256)


def test_q6_k_roundtrip():
    rng = np.random.default_rng(4)
    for trial in range(20):
        sc = rng.integers(-128, 128, 16).tolist()
        q = rng.integers(0, 64, 256).tolist()
        d = f16_bits(abs(float(rng.standard_normal())) * 0.001)
        raw, exact = enc_q6_k(d, sc, q)
        _check(wl.Q6_K, raw, exact, 256)


def test_f16_roundtrip():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 65536, 64).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00].tolist()  # finite only
    bits = bits[: len(bits) // 4 * 4]                  # k must be a multiple of 4
    raw, exact = enc_f16(bits)
    _check(wl.F16, raw, exact, len(bits))


# ---------------------------------------------------------------- special cases that reduce to integers

def test_special_integer_cases():
    one = f16_bits(1.0)
    # Q8_0, d = 1: weights are the int8 quants.
    q = list(range(-16, 16))
    raw, _ = enc_q8_0(one, q)
    assert oracle.dequant(wl.Q8_0, np.frombuffer(raw, np.uint8), 1, 32)[0].tolist() == q
    # Q5_0, d = 1, high bits clear: nibble - 16; all set: nibble.
    nib = [i % 16 for i in range(32)]
    raw, _ = enc_q5_0(one, nib)
    assert oracle.dequant(wl.Q5_0, np.frombuffer(raw, np.uint8), 1, 32)[0].tolist() == [v - 16 for v in nib]
    raw, _ = enc_q5_0(one, [v + 16 for v in nib])
    assert oracle.dequant(wl.Q5_0, np.frombuffer(raw, np.uint8), 1, 32)[0].tolist() == nib
    # Q4_K, d = 1, dmin = 0, scale s+1, every quant 1: value = sub-block + 1.
    raw, _ = enc_q4_k(one, 0, [s + 1 for s in range(8)], [0] * 8, [1] * 256)
    got = oracle.dequant(wl.Q4_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert got.tolist() == [v // 32 + 1 for v in range(256)]
    # ... and d = 0, dmin = 1, min s+1: value = -(s+1)  (mins use the same packing).
    raw, _ = enc_q4_k(0, one, [0] * 8, [s + 33 for s in range(8)], [5] * 256)
    got = oracle.dequant(wl.Q4_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert got.tolist() == [-(v // 32 + 33) for v in range(256)]
    # Q6_K, d = 1, scale g+1: (q - 32) * (v // 16 + 1).
    qq = [(7 * v) % 64 for v in range(256)]
    raw, _ = enc_q6_k(one, [g + 1 for g in range(16)], qq)
    got = oracle.dequant(wl.Q6_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert got.tolist() == [(qq[v] - 32) * (v // 16 + 1) for v in range(256)]


def test_sign_of_zero():
    """Integer offsets come first, then the float product: the sign of a zero
    weight is the XOR of the factor signs."""
    one, neg = f16_bits(1.0), f16_bits(-1.0)
    raw, _ = enc_q6_k(one, [-3] * 16, [32] * 256)          # sc < 0, q - 32 = 0 -> -0
    got = oracle.dequant(wl.Q6_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert np.all(got == 0) and np.all(np.signbit(got))
    raw, _ = enc_q8_0(neg, [0] * 32)                         # d < 0, q = 0 -> -0
    got = oracle.dequant(wl.Q8_0, np.frombuffer(raw, np.uint8), 1, 32)[0]
    assert np.all(np.signbit(got))
    raw, _ = enc_q5_0(0, [3] * 32)                           # d = +0, q - 16 < 0 -> -0
    got = oracle.dequant(wl.Q5_0, np.frombuffer(raw, np.uint8), 1, 32)[0]
    assert np.all(np.signbit(got))
    raw, _ = enc_q4_k(one, one, [0] * 8, [0] * 8, [0] * 256)  # +0 - +0 = +0
    got = oracle.dequant(wl.Q4_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
    assert np.all(got == 0) and not np.any(np.signbit(got))


# ---------------------------------------------------------------- single-bit probes

def _probe(t, k, raw, expected_values):
    """Flip every bit of ``raw``; ``expected_values(byte, bit)`` returns the set
    of value indices allowed to change (a quant bit must change exactly that
    one value)."""
    base = oracle.dequant(t, np.frombuffer(raw, np.uint8), 1, k)[0]
    arr = np.frombuffer(raw, np.uint8).copy()
    for byte in range(arr.size):
        for bit in range(8):
            a2 = arr.copy()
            a2[byte] ^= 1 << bit
            got = oracle.dequant(t, a2, 1, k)[0]
            changed = set(np.nonzero(_bits32(got) != _bits32(base))[0].tolist())
            exp, exact = expected_values(byte, bit)
            if exact:
                assert changed == exp, (t, byte, bit, sorted(changed)[:6], sorted(exp)[:6])
            else:
                assert changed and changed <= exp, (t, byte, bit, sorted(changed)[:6])


def test_bit_probes_q8_0():
    raw, _ = enc_q8_0(f16_bits(0.75), [(5 * i) % 200 - 100 for i in range(32)])
    _probe(wl.Q8_0, 32, raw,
           lambda byte, bit: (set(range(32)), False) if byte < 2 else ({byte - 2}, True))


def test_bit_probes_q5_0():
    raw, _ = enc_q5_0(f16_bits(0.75), [(7 * i) % 32 for i in range(32)])

    def exp(byte, bit):
        if byte < 2:
            return set(range(32)), False
        if byte < 6:
            return {8 * (byte - 2) + bit}, True
        i = byte - 6
        return ({i} if bit < 4 else {i + 16}), True
    _probe(wl.Q5_0, 32, raw, exp)


def test_bit_probes_q4_k():
    qv = [(3 * v) % 16 for v in range(256)]
    raw, _ = enc_q4_k(f16_bits(0.5), f16_bits(0.25), [s * 7 + 3 for s in range(8)],
                      [s * 5 + 2 for s in range(8)], qv)

    def sub(s, scale):
        # a scale bit moves the values of sub-block s whose quant is non-zero;
        # a min bit moves all of them
        return {v for v in range(32 * s, 32 * s + 32) if not scale or qv[v] != 0}

    def exp(byte, bit):
        if byte < 4:
            return set(range(256)), False
        if byte < 16:
            j = byte - 4                                  # packed scale byte j
            if j < 4:                                     # sc[j] low 6 bits / sc[j+4] bits 4-5
                return sub(j if bit < 6 else j + 4, True), True
            if j < 8:                                     # mn[j-4] low 6 bits / mn[j] bits 4-5
                return sub(j - 4 if bit < 6 else j, False), True
            return sub(j - 4, bit < 4), True              # low nibble sc[j-4], high nibble mn[j-4]
        b = byte - 16
        c, l = b // 32, b % 32
        return ({64 * c + l} if bit < 4 else {64 * c + 32 + l}), True
    _probe(wl.Q4_K, 256, raw, exp)


def test_bit_probes_q6_k():
    raw, _ = enc_q6_k(f16_bits(0.5), [g - 8 if g != 8 else 9 for g in range(16)],
                      [(11 * v + 5) % 64 for v in range(256)])

    def exp(byte, bit):
        if byte < 128:
            h, r = byte // 64, byte % 64
            t = (r // 32) + (2 if bit >= 4 else 0)
            return {128 * h + 32 * t + r % 32}, True
        if byte < 192:
            h, l = (byte - 128) // 32, (byte - 128) % 32
            return {128 * h + 32 * (bit // 2) + l}, True
        if byte < 208:
            g = byte - 192
            return set(range(16 * g, 16 * g + 16)), False
        return set(range(256)), False
    _probe(wl.Q6_K, 256, raw, exp)


# ---------------------------------------------------------------- products

def _exact_dot(wd_row, x_row):
    return sum((Fraction(float(w)) * Fraction(float(v)) for w, v in zip(wd_row, x_row)), Fraction(0))


@pytest.mark.parametrize("name", ["F16", "Q8_0", "Q4_K", "Q6_K", "Q5_0", "F32", "BF16"])
def test_matvec_brute_force_strided_batched(name):
    """Exact rational dot on tiny strided, batched inputs: the oracle's float64
    sum is within k * 2^-53 * sum|w x| of the exact value, and |w x| sums
    likewise.  Junk in the stride gaps must not leak in."""
    t = TYPES[name]
    k = {wl.F16: 12, wl.Q8_0: 64, wl.Q5_0: 64, wl.Q4_K: 256, wl.Q6_K: 256, wl.F32: 12, wl.BF16: 20}[t]
    n, m, batch = 3, 3, 2
    xrs, xbs = k + 8, 3 * (k + 8) + 4
    W = wl.weights(t, n * batch, k, seed=21)
    xbuf = wl.activations(1, (batch - 1) * xbs + (m - 1) * xrs + k + 16, seed=22)[0]
    y, a = oracle.matvec(t, W, xbuf, n, k, m, batch, xrs, xbs)
    wd = oracle.dequant(t, W, n * batch, k)
    for b in range(batch):
        for j in range(m):
            xr = xbuf[b * xbs + j * xrs: b * xbs + j * xrs + k]
            for i in range(n):
                ex = _exact_dot(wd[b * n + i], xr)
                exa = sum((abs(Fraction(float(w)) * Fraction(float(v))) for w, v in zip(wd[b * n + i], xr)),
                          Fraction(0))
                bound = k * 2.0 ** -53 * float(exa)
                assert abs(Fraction(y[b, j, i]) - ex) <= Fraction(bound)
                assert abs(Fraction(a[b, j, i]) - exa) <= Fraction(bound)


def test_matvec_unit_vectors_extract_columns():
    t, n, k = wl.Q4_K, 5, 512
    W = wl.weights(t, n, k, seed=31)
    wd = oracle.dequant(t, W, n, k)
    for col in (0, 1, 255, 256, 511):
        x = np.zeros(k, np.float32)
        x[col] = 1.0
        y, a = oracle.matvec(t, W, x, n, k, 1)
        assert np.array_equal(y[0, 0], wd[:, col].astype(np.float64))
        assert np.array_equal(a[0, 0], np.abs(wd[:, col]).astype(np.float64))


def test_matvec_constant_weights():
    """F16 weights all c: y = c * sum(x) (exactly, for c a power of two and
    small integer x)."""
    n, k = 4, 64
    W = np.full((n, k), f16_bits(0.25), dtype=np.uint16).view(np.uint8)
    x = np.arange(-32, 32, dtype=np.float32).reshape(1, k) + 0.5
    y, _ = oracle.matvec(wl.F16, W, x, n, k, 1)
    assert np.all(y == 0.25 * float(x.sum()))


def test_grouped_token_major_equals_per_group():
    """grouped_token_major: y[j, g*n + i] = W[g*n + i, :] . x[j, g*k:(g+1)*k]
    (RowExactMatvecShape::grouped_token_major)."""
    t, G, n, k, m = wl.Q5_0, 4, 6, 64, 3
    W = wl.weights(t, G * n, k, seed=41)
    x = wl.activations(m, G * k, seed=42)
    y, _ = oracle.matvec(t, W, x, n, k, m, batch=G, x_row_stride=G * k, x_batch_stride=k)
    rb = oracle.row_bytes(t, k)
    for g in range(G):
        Wg = W.ravel()[g * n * rb:(g + 1) * n * rb]
        xg = np.ascontiguousarray(x[:, g * k:(g + 1) * k])
        yg, _ = oracle.matvec(t, Wg, xg, n, k, m)
        assert np.array_equal(y[g], yg[0])


def test_matvec_rows_independent_of_m():
    """Row j of an m-row call equals the 1-row call on row j (trivially, by
    construction; kept as the oracle-side statement of row exactness)."""
    t, n, k = wl.Q6_K, 7, 256
    W = wl.weights(t, n, k, seed=51)
    x = wl.activations(8, k, seed=52)
    y8, _ = oracle.matvec(t, W, x, n, k, 8)
    for j in range(8):
        y1, _ = oracle.matvec(t, W, x[j], n, k, 1)
        assert np.array_equal(y8[0, j], y1[0, 0])


def test_matvec_vs_numpy_float64_dot():
    """A library dot of the dequantized weights agrees to float64 rounding."""
    t, n, k, m = wl.Q8_0, 33, 1024, 4
    W = wl.weights(t, n, k, seed=61)
    x = wl.activations(m, k, seed=62)
    y, a = oracle.matvec(t, W, x, n, k, m)
    wd = oracle.dequant(t, W, n, k).astype(np.float64)
    ref = x.astype(np.float64) @ wd.T
    assert np.all(np.abs(y[0] - ref) <= 2 * k * 2.0 ** -53 * a[0])


def test_gather_identity_and_selection():
    """ids = 0..batch-1 is the plain batched product; a repeated id equals
    the product with that weight set; an id out of range gives NaN only for
    its own batch entry."""
    t, E, n, k, m = wl.Q4_K, 5, 6, 256, 2
    W = wl.weights(t, E * n, k, seed=81)
    x = wl.activations(1, 4 * (m * k + 8), seed=82)[0]
    xrs, xbs = k, m * k + 8
    y, a = oracle.matvec(t, W, x, n, k, m, batch=4, x_row_stride=xrs, x_batch_stride=xbs)
    yg, ag = oracle.matvec_gather(t, W, E, np.arange(4), x, n, k, m, 4, xrs, xbs)
    assert np.array_equal(y, yg) and np.array_equal(a, ag)
    rb = oracle.row_bytes(t, k)
    ids = np.array([3, 3, -1, 4], np.int32)
    yg, _ = oracle.matvec_gather(t, W, E, ids, x, n, k, m, 4, xrs, xbs)
    for b, e in enumerate(ids):
        if e < 0:
            assert np.all(np.isnan(yg[b]))
            continue
        We = W.ravel()[e * n * rb:(e + 1) * n * rb]
        ye, _ = oracle.matvec(t, We, x[b * xbs:], n, k, m, x_row_stride=xrs)
        assert np.array_equal(yg[b], ye[0])
    yg, _ = oracle.matvec_gather(t, W, E, np.array([0, 5, 1, 2], np.int32), x, n, k, m, 4, xrs, xbs)
    assert np.all(np.isnan(yg[1])) and not np.any(np.isnan(yg[[0, 2, 3]]))


def test_residual_rmsnorm_reduces_and_normalises():
    """With x = 0 the residual form is the add form (x := h, r := 0, g := w2,
    eps := eps2) bit for bit; with h = 0, w = 1, no scaling and eps = 0 its
    first normalisation alone has mean square 1 and is float32 x / rms in
    float64; scaling x by 4 leaves it unchanged; the scaling c multiplies the
    float32 sum after rounding; with w2 = 1, eps2 = 0 the second
    normalisation has mean square 1; the product is a library float64 dot of
    the dequantized weights with xn."""
    t, n, k, m = wl.Q8_0, 5, 64, 3
    W = wl.weights(t, n, k, seed=191)
    h = wl.activations(m, k, seed=192)
    x = wl.activations(m, k, seed=193)
    w = (1.0 + wl.activations(1, k, seed=194)[0] * 0.1).astype(np.float32)
    c = (0.5 + wl.activations(1, k, seed=195)[0] * 0.05).astype(np.float32)
    w2 = (1.0 + wl.activations(1, k, seed=196)[0] * 0.1).astype(np.float32)
    zero = np.zeros_like(x)
    hs, xn, y, a = oracle.mv_residual_rmsnorm(t, W, h, zero, w, None, w2, 1e-3, 1e-5, n, k, m)
    h2, xn2, y2, a2 = oracle.mv_add_rmsnorm(t, W, h, zero, w2, 1e-5, n, k, m)
    assert np.array_equal(_bits32(hs), _bits32(h2)) and np.array_equal(xn, xn2)
    assert np.array_equal(y, y2) and np.array_equal(a, a2)
    # the first normalisation alone
    hs, xn, _, _ = oracle.mv_residual_rmsnorm(t, W, zero, x, None, None, None, 0.0, 0.0, n, k, m)
    x64 = x.astype(np.float64)
    rms = np.sqrt((x64 ** 2).sum(axis=1, keepdims=True) / k)
    assert np.max(np.abs(hs.reshape(m, k).astype(np.float64) - x64 / rms)) <= 2.0 ** -24 * 4
    assert np.allclose((hs.reshape(m, k).astype(np.float64) ** 2).mean(axis=1), 1.0, rtol=1e-6)
    hs4, _, _, _ = oracle.mv_residual_rmsnorm(t, W, zero, 4 * x, None, None, None, 0.0, 0.0, n, k, m)
    assert np.array_equal(_bits32(hs4), _bits32(hs))
    # the scaling acts on the rounded sum
    hs_c, _, _, _ = oracle.mv_residual_rmsnorm(t, W, h, x, w, c, None, 1e-5, 1e-5, n, k, m)
    hs_1, _, _, _ = oracle.mv_residual_rmsnorm(t, W, h, x, w, None, None, 1e-5, 1e-5, n, k, m)
    assert np.array_equal(_bits32(hs_c), _bits32((hs_1.reshape(m, k) * c).ravel()))
    # the second normalisation and the product
    hs, xn, y, a = oracle.mv_residual_rmsnorm(t, W, h, x, w, c, None, 1e-5, 0.0, n, k, m)
    assert np.allclose((xn[0] ** 2).mean(axis=1), 1.0, rtol=1e-14, atol=0)
    wd = oracle.dequant(t, W, n, k).astype(np.float64)
    assert np.all(np.abs(y[0] - xn[0] @ wd.T) <= 2 * k * 2.0 ** -53 * a[0])


def test_add_rmsnorm_sum_and_normalisation():
    """h is numpy's float32 sum; with eps = 0 and g = 1 every normalised row
    has mean square 1; a constant row c normalises to c / sqrt(c^2 + eps);
    scaling h by 4 leaves xn unchanged (eps = 0, exact in float64); the
    product is a library float64 dot of the dequantized weights with xn."""
    t, n, k, m = wl.Q8_0, 5, 64, 3
    W = wl.weights(t, n, k, seed=91)
    x = wl.activations(m, k, seed=92)
    r = wl.activations(m, k, seed=93)
    g = (1.0 + wl.activations(1, k, seed=94)[0] * 0.1).astype(np.float32)
    h, xn, y, a = oracle.mv_add_rmsnorm(t, W, x, r, None, 0.0, n, k, m)
    assert np.array_equal(_bits32(h), _bits32((x + r).ravel()))
    assert np.allclose((xn[0] ** 2).mean(axis=1), 1.0, rtol=1e-14, atol=0)
    _, xn4, _, _ = oracle.mv_add_rmsnorm(t, W, 4 * x, 4 * r, None, 0.0, n, k, m)
    assert np.array_equal(xn4, xn)
    c, eps = np.float32(0.75), 1e-3
    _, xc, _, _ = oracle.mv_add_rmsnorm(t, W, np.full((1, k), c, np.float32), np.zeros((1, k), np.float32), g, eps,
                                        n, k, 1)
    assert np.allclose(xc[0, 0], float(c) / np.sqrt(float(c) ** 2 + eps) * g.astype(np.float64), rtol=1e-15)
    h, xn, y, a = oracle.mv_add_rmsnorm(t, W, x, r, g, 1e-5, n, k, m)
    wd = oracle.dequant(t, W, n, k).astype(np.float64)
    ref = xn[0] @ wd.T
    assert np.all(np.abs(y[0] - ref) <= 2 * k * 2.0 ** -53 * a[0])
    assert np.all(np.abs(a[0] - np.abs(xn[0]) @ np.abs(wd).T) <= 2 * k * 2.0 ** -53 * a[0])


# ---------------------------------------------------------------- generator

def test_generator_deterministic_and_distributed():
    a = wl.weights(wl.Q6_K, 8, 512, seed=7)
    b = wl.weights(wl.Q6_K, 8, 512, seed=7)
    c = wl.weights(wl.Q6_K, 8, 512, seed=8)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    z = wl.Stream(3).normal(200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    q = wl.weights(wl.Q8_0, 64, 1024, seed=9).reshape(-1, 34)
    qs = q[:, 2:].view(np.int8)
    assert qs.min() == -127 and qs.max() == 127
    s6 = wl.weights(wl.Q6_K, 64, 1024, seed=9).reshape(-1, 210)[:, 192:208].view(np.int8)
    assert s6.min() == -64 and s6.max() == 63
    # splitmix64 reference values for seed 0 (outputs of the published algorithm)
    assert wl.splitmix64(0, 3).tolist() == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
