// Device code of the row-exact few-row mat-vec (gfx950, wave64).
//
// Product (mlx-native 0.18.0, src/ops/row_exact_matvec.rs, module docs):
//   y[b][j][i] = sum_kk W[b*n + i][kk] * x[b][j][kk],  1 <= m <= 8.
//
// Work decomposition
//   - A weight row is cut into "pieces": per-lane work items whose bytes sit
//     together in the row (F16: 8 values; Q8_0 / Q5_0: one block; Q4_K: 32
//     nibble bytes, two sub-blocks, of a super-block; Q6_K: a quarter
//     super-block).  A row has 64 lanes of a wave, or 32 / 16 (two / four
//     rows per wave) for rows of at most 32 / 16 pieces and, for the
//     block-quantized types, unsplit rows whose last 64-lane step would be
//     at most half full.  Lane L of the row's L_row lanes takes pieces L,
//     L + L_row, L + 2 L_row, ... in that order, so each load instruction of
//     a wave covers adjacent bytes of each of its rows.
//   - A wave streams rows_per_wave (NR) rows at once: every input value read
//     from LDS feeds all NR weight rows (the page's nr0 packing).
//   - The m input rows of the batch are staged once per pass into LDS
//     (padded so that the lanes' 16-byte reads hit distinct banks).
//
// Numerics (module docs, "Row exactness")
//   - Every weight is decoded exactly in registers.  Dense weights (F16,
//     BF16, F32) are decoded to their float32 value w.  Q8_0, Q5_0 and Q6_K
//     weights are s * q with an integer-valued q and a scale s shared by a
//     segment of values (a block; 16 values for Q6_K); Q4_K weights are
//     s * q - o with a scale and an offset shared by a 32-value sub-block:
//     they are decoded to q, exactly.
//   - For each (row, input row) a lane keeps one accumulator and folds its
//     pieces into it with an explicit fmaf chain, in piece order and, inside
//     a piece, in a fixed value order: acc = fma(w, x, acc) per value, or,
//     per scaled segment, part = q*x then fma(q, x, part) over its values,
//     acc = fma(s, part, acc) and, for Q4_K, acc = fma(-o, sum_x, acc) with
//     the segment's sum of x, which each workgroup forms once per input row
//     in a fixed order.  Nothing about those chains depends on m or on the
//     packing (NR, waves per workgroup, grid).
//   - The 64 lane partials of an output are added by one fixed tree: lanes
//     (L, L^32), then (L, L^16), then within each row of 16 lanes: rotate-8,
//     half-row mirror, xor 2, xor 1 (rows on 32 or 16 lanes: the same tree
//     without its first one or two levels).  The first two levels are done with the
//     gfx950 permlane32/permlane16 swaps and, when a lane holds several
//     outputs, transposed (each swap hands half of the outputs to the other
//     half of the wave, so no work is duplicated); the rest with DPP.  IEEE
//     addition is commutative, so whichever lane performs a given pairwise
//     add produces the same bits: every output gets the same tree for every
//     m and every packing.
#pragma once

#include <mutex>

#include "re_internal.h"

// Code-generation knobs (measured defaults; variants with other values,
// and with register caps for more waves per SIMD, measured no faster): the
// smallest m whose piece loop gets a scheduling barrier per group, the
// register budget that allows two items of loads in flight, the largest m
// whose x is requested ahead of the weights, the smallest m at which half
// of a workgroup's waves request their weights after the x staging, and the
// smallest m from which waves of three or more items take x ahead instead.
#ifndef REX_SCHED_BARRIER_MIN_M
#define REX_SCHED_BARRIER_MIN_M 4
#endif
#ifndef REX_DEPTH_BUDGET
#define REX_DEPTH_BUDGET 120
#endif
#ifndef REX_X_FIRST_MAX_M
#define REX_X_FIRST_MAX_M 4
#endif
#ifndef REX_LATE_HALF_MIN_M
#define REX_LATE_HALF_MIN_M 5
#endif
#ifndef REX_X_FIRST_UNC_MIN_M
#define REX_X_FIRST_UNC_MIN_M 6
#endif

// 1: single-pass instances of types with a fixed load count per piece stage
// x with loads that write LDS directly (see stage_x_dma).
#ifndef REX_X_DMA
#define REX_X_DMA 1
#endif


namespace rex {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Exact widening of an IEEE half (subnormals included).
__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Hides a value from the optimizer so that byte-parallel (SWAR) code stays
// byte-parallel instead of being folded back into per-value bit extracts.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// ({hi, lo} >> 8*sh)[31:0]
__device__ __forceinline__ uint32_t abyte(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// Loads below take a wave-uniform row base R (4-byte aligned; 16-byte for
// Q4_K, 8-byte for F16) and a per-lane 32-bit byte offset, so they compile
// to global loads with a scalar base.
template <class V> __device__ __forceinline__ V ldv(const uint8_t *R, uint32_t off) {
    return *(const V *)(R + off);
}
__device__ __forceinline__ uint32_t ld16(const uint8_t *R, uint32_t off) { return *(const uint16_t *)(R + off); }

// The same 16 bytes with one 2-byte-aligned dwordx4 load (the HSA runtime
// runs the GPU in unaligned-access mode).  Measured: faster than the aligned
// loads + realignment for Q6_K's three 16-byte fields (fewer VALU and
// memory instructions), slower for Q8_0 and Q5_0 blocks, which keep
// aligned loads (realigned at multiply time).
__device__ __forceinline__ void load16_u(const uint8_t *R, uint32_t o, uint32_t (&out)[4]) {
    const u32x4a2 r = ldv<u32x4a2>(R, o);
    out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}

template <int T> struct Tr;

// Each Tr<T> gives, for piece p of a row:
//   load(R, o0, p)  raw bytes (o0 = offset of the row from R)
//   prep(raw, p)    per-piece scales
//   deq(raw, pre, g, w)  exact float32 values of the piece's group g (4 values)
//   vpos(p, g)      index in the row of the group's first value
//   xoff(p) + goff(g) == vpos(p, g) - vb padded for LDS (xoff relative to the
//                   pass's first value vb, which is a wave-step multiple)

// ---------------------------------------------------------------- F16
// Piece p: values 8p..8p+7 (16 bytes).  k % 8 == 4 leaves a half piece.
template <> struct Tr<kF16> : Geo<kF16> {
    static constexpr int SEG = 0;  // no scale: the fma chain runs on w
    static constexpr int LOADS = 0;  // x staged in registers (a piece takes 1 or 2 loads)
    static constexpr int ITEM_DWORDS = 4;
    struct Raw { uint32_t w[4]; };
    struct Pre {};
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t k) {
        Raw r;
        const uint32_t o = o0 + 16 * p;
        if (8 * p + 8 <= k) {
            const u32x4a4 v = ldv<u32x4a4>(R, o);
            r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
        } else {
            const u32x2a4 v = ldv<u32x2a4>(R, o);
            r.w[0] = v.x; r.w[1] = v.y; r.w[2] = 0; r.w[3] = 0;
        }
        return r;
    }
    static __device__ __forceinline__ Pre prep(const Raw &, uint32_t) { return {}; }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &, int g, float (&w)[4]) {
        w[0] = h2f(r.w[2 * g] & 0xffffu);
        w[1] = h2f(r.w[2 * g] >> 16);
        w[2] = h2f(r.w[2 * g + 1] & 0xffffu);
        w[3] = h2f(r.w[2 * g + 1] >> 16);
    }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) { return 8 * p + 4 * g; }
    // 4 pad floats after every Geo PADP values (PADP / 8 pieces)
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) {
        const uint32_t q = p - vb / 8;
        return 8 * q + 4 * (q / (Geo<kF16>::PADP / 8));
    }
    static constexpr uint32_t goff(int g) { return 4 * g; }
    static __device__ __forceinline__ bool group_valid(uint32_t p, int g, uint32_t k) {
        return g == 0 || 8 * p + 4 < k;
    }
};

// ---------------------------------------------------------------- BF16
// Piece p: values 8p..8p+7 (16 bytes), as F16.  A bfloat16 is the upper half
// of a float32, so the exact widening is a 16-bit shift.
template <> struct Tr<kBF16> : Geo<kBF16> {
    static constexpr int SEG = 0;
    static constexpr int LOADS = 0;  // as F16
    static constexpr int ITEM_DWORDS = 4;
    struct Raw { uint32_t w[4]; };
    struct Pre {};
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t k) {
        const auto h = Tr<kF16>::load(R, o0, p, k);
        Raw r;
        r.w[0] = h.w[0]; r.w[1] = h.w[1]; r.w[2] = h.w[2]; r.w[3] = h.w[3];
        return r;
    }
    static __device__ __forceinline__ Pre prep(const Raw &, uint32_t) { return {}; }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &, int g, float (&w)[4]) {
        w[0] = __uint_as_float(r.w[2 * g] << 16);
        w[1] = __uint_as_float(r.w[2 * g] & 0xffff0000u);
        w[2] = __uint_as_float(r.w[2 * g + 1] << 16);
        w[3] = __uint_as_float(r.w[2 * g + 1] & 0xffff0000u);
    }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) { return Tr<kF16>::vpos(p, g); }
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) { return Tr<kF16>::xoff(p, vb); }
    static constexpr uint32_t goff(int g) { return 4 * g; }
    static __device__ __forceinline__ bool group_valid(uint32_t p, int g, uint32_t k) {
        return Tr<kF16>::group_valid(p, g, k);
    }
};

// ---------------------------------------------------------------- F32
// Piece p: values 4p..4p+3 (16 bytes, 16-byte aligned: W is, and a row is
// 4k bytes with k % 4 == 0).
template <> struct Tr<kF32> : Geo<kF32> {
    static constexpr int SEG = 0;
    static constexpr int LOADS = 0;  // x staged in registers (see stage_x_dma)
    static constexpr int ITEM_DWORDS = 4;
    struct Raw { uint32_t w[4]; };
    struct Pre {};
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        const u32x4 v = ldv<u32x4>(R, o0 + 16 * p);
        Raw r;
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
        return r;
    }
    static __device__ __forceinline__ Pre prep(const Raw &, uint32_t) { return {}; }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &, int, float (&w)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(r.w[i]);
    }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int) { return 4 * p; }
    // 4 pad floats after every Geo PADP values (PADP / 4 pieces)
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) {
        const uint32_t q = p - vb / 4;
        return 4 * q + 4 * (q / (Geo<kF32>::PADP / 4));
    }
    static constexpr uint32_t goff(int) { return 0; }
    static __device__ __forceinline__ bool group_valid(uint32_t, int, uint32_t) { return true; }
};

// ---------------------------------------------------------------- Q8_0
// Piece p: block p (34 bytes: f16 d, 32 int8).  w = d * q.
template <> struct Tr<kQ8_0> : Geo<kQ8_0> {
    static constexpr int SEG = 8;  // one scale per piece
    static constexpr int LOADS = 0;  // x staged in registers (see stage_x_dma)
    static constexpr int ITEM_DWORDS = 9;
    // Raw: the quants' bytes as loaded (eight aligned dwords around them, the
    // last two bytes, the byte shift) and d.  They are realigned where they
    // are multiplied: realigned at load time, the compiler waits for a
    // piece's loads right after issuing them, before the multiply they were
    // meant to overlap.
    struct Raw { uint32_t w[9]; uint32_t sh; uint32_t d; };
    struct Pre { float d; };
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        Raw r;
        const uint32_t B = o0 + 34 * p;
        r.d = ld16(R, B);
        const uint32_t F = B + 2;  // quants
        r.sh = F & 3u;
        const u32x4a4 r0 = ldv<u32x4a4>(R, F - r.sh), r1 = ldv<u32x4a4>(R, F - r.sh + 16);
        r.w[0] = r0.x; r.w[1] = r0.y; r.w[2] = r0.z; r.w[3] = r0.w;
        r.w[4] = r1.x; r.w[5] = r1.y; r.w[6] = r1.z; r.w[7] = r1.w;
        r.w[8] = ld16(R, F + 30);
        return r;
    }
    // quant bytes 4g..4g+3
    static __device__ __forceinline__ uint32_t qword(const Raw &r, int g) { return abyte(r.w[g + 1], r.w[g], r.sh); }
    static __device__ __forceinline__ Pre prep(const Raw &r, uint32_t) { return {h2f(r.d)}; }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &pr, int g, float (&w)[4]) {
        const uint32_t q4 = qword(r, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pr.d * (float)(int8_t)(q4 >> (8 * i));
    }
    static __device__ __forceinline__ void deqi(const Raw &r, const Pre &, int g, float (&q)[4]) {
        const uint32_t q4 = qword(r, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)(int8_t)(q4 >> (8 * i));
    }
    static __device__ __forceinline__ float scale(const Pre &pr, int) { return pr.d; }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) { return 32 * p + 4 * g; }
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) { return 36 * (p - vb / 32); }
    static constexpr uint32_t goff(int g) { return 4 * g; }
    static __device__ __forceinline__ bool group_valid(uint32_t, int, uint32_t) { return true; }
};

// ---------------------------------------------------------------- Q5_0
// Piece p: block p (22 bytes: f16 d, u32 high bits, 16 nibble bytes).
// Value i < 16: low nibble of byte i; i >= 16: high nibble of byte i - 16;
// bit i of the high bits is bit 4.  w = d * (q - 16).
// Four values at a time: byte i of a dword becomes the int8 8*(q_i - 16)
// (nibble in bits 3..6, inverted high bit as the sign bit), converted with
// one signed-byte convert and scaled by d/8 (exact).
template <> struct Tr<kQ5_0> : Geo<kQ5_0> {
    static constexpr int SEG = 8;  // one scale per piece
    static constexpr int LOADS = 0;  // x staged in registers (see stage_x_dma)
    static constexpr int ITEM_DWORDS = 6;
    // Raw: the block's bytes as loaded (the aligned dwords around its first
    // 8 bytes, around the 16 nibble bytes plus their last two bytes, the
    // byte shift of the block); realigned where they are multiplied (see
    // Q8_0), into d and the inverted high bits in prep, the nibble bytes in
    // bytes8.
    struct Raw { uint32_t e[3]; uint32_t q[5]; uint32_t sh; };
    struct Pre { float d8; uint32_t nqh; };
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        Raw r;
        const uint32_t B = o0 + 22 * p;
        r.sh = B & 3u;
        const u32x3a4 e = ldv<u32x3a4>(R, B - r.sh);  // covers bytes 0..7 of the block
        r.e[0] = e.x; r.e[1] = e.y; r.e[2] = e.z;
        // the 16 nibble bytes at B + 6: the aligned dwords around them and
        // their last two bytes (nothing past the block is read)
        const uint32_t o = B + 6, shq = o & 3u;
        const u32x4a4 q = ldv<u32x4a4>(R, o - shq);
        r.q[0] = q.x; r.q[1] = q.y; r.q[2] = q.z; r.q[3] = q.w;
        r.q[4] = ld16(R, o + 14);
        return r;
    }
    static __device__ __forceinline__ Pre prep(const Raw &r, uint32_t) {
        const uint32_t b0 = abyte(r.e[1], r.e[0], r.sh);  // d | qh.lo << 16
        const uint32_t b1 = abyte(r.e[2], r.e[1], r.sh);  // qh.hi | qs[0..1] << 16
        return {h2f(b0 & 0xffffu) * 0.125f, ~abyte(b1, b0, 2)};
    }
    // nibble bytes 4i..4i+3 (the shift of B + 6 is that of B plus 2)
    static __device__ __forceinline__ uint32_t qword(const Raw &r, int i) {
        return abyte(r.q[i + 1], r.q[i], (r.sh + 2u) & 3u);
    }
    static __device__ __forceinline__ uint32_t bytes8(const Raw &r, const Pre &pr, int g) {
        const uint32_t qw = qword(r, g & 3);
        const uint32_t lo = g < 4 ? ((qw << 3) & 0x78787878u) : ((qw >> 1) & 0x78787878u);
        // bits 4g..4g+3 of ~qh -> bit 7 of bytes 0..3 (t * 0x204081 puts bit i at 8i, no carries)
        const uint32_t t = (pr.nqh >> (4 * g)) & 15u;
        return ((opaque(__umul24(t, 0x204081u)) << 7) & 0x80808080u) | lo;
    }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &pr, int g, float (&w)[4]) {
        const uint32_t b = bytes8(r, pr, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (float)(int8_t)(b >> (8 * i)) * pr.d8;
    }
    static __device__ __forceinline__ void deqi(const Raw &r, const Pre &pr, int g, float (&q)[4]) {
        const uint32_t b = bytes8(r, pr, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)(int8_t)(b >> (8 * i));
    }
    static __device__ __forceinline__ float scale(const Pre &pr, int) { return pr.d8; }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) { return 32 * p + 4 * g; }
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) { return 36 * (p - vb / 32); }
    static constexpr uint32_t goff(int g) { return 4 * g; }
    static __device__ __forceinline__ bool group_valid(uint32_t, int, uint32_t) { return true; }
};

// ---------------------------------------------------------------- Q4_K
// Piece p: super-block p/4, nibble chunk c = p%4 (bytes 32c..32c+31 of its
// 128): low nibbles are values 64c + 0..31 of sub-block 2c, high nibbles
// values 64c + 32..63 of sub-block 2c+1.
// The weight value (row_exact_dequant) is w = fma(d*sc, q, -(dmin*mn)): one
// rounding of the exact value; the mat-vec applies d*sc and dmin*mn per
// sub-block instead (see SEG).
template <> struct Tr<kQ4K> : Geo<kQ4K> {
    // One scale and one offset per 32 values (groups 8e..8e+7, sub-block
    // 2c+e): the segment contributes d*sc * sum(q*x) - dmin*mn * sum(x).
    static constexpr int SEG = 8;
    static constexpr int LOADS = 0;  // x staged in registers (see stage_x_dma)
    static constexpr int ITEM_DWORDS = 12;
    struct Raw { uint32_t qs[8]; uint32_t h[4]; };
    struct Pre { float dsc[2], dmn[2]; };
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        Raw r;
        const uint32_t B = o0 + 144 * (p >> 2);
        const u32x4 hv = ldv<u32x4>(R, B);
        const u32x4 q0 = ldv<u32x4>(R, B + 16 + 32 * (p & 3));
        const u32x4 q1 = ldv<u32x4>(R, B + 32 + 32 * (p & 3));
        r.h[0] = hv.x; r.h[1] = hv.y; r.h[2] = hv.z; r.h[3] = hv.w;
        r.qs[0] = q0.x; r.qs[1] = q0.y; r.qs[2] = q0.z; r.qs[3] = q0.w;
        r.qs[4] = q1.x; r.qs[5] = q1.y; r.qs[6] = q1.z; r.qs[7] = q1.w;
        return r;
    }
    // Scales and mins of sub-blocks 2c and 2c+1 as byte pairs.  With the 12
    // packed bytes S in h[1] (S0..3), h[2] (S4..7), h[3] (S8..11):
    //   s < 4 : sc = S[s] & 63,                     mn = S[s+4] & 63
    //   s >= 4: sc = (S[s+4] & 15) | (S[s-4] >> 6) << 4,
    //           mn = (S[s+4] >> 4) | (S[s] >> 6) << 4
    static __device__ __forceinline__ Pre prep(const Raw &r, uint32_t p) {
        Pre pr;
        const uint32_t c = p & 3;
        const bool hi = c >= 2;
        const uint32_t sh = 16 * (c & 1);
        const uint32_t top = sh + (hi ? 2u : 0u);
        const uint32_t scp = (((hi ? r.h[3] : r.h[1]) >> sh) & 0x0F0Fu) | ((r.h[1] >> top) & 0x3030u);
        const uint32_t mnp = (((hi ? r.h[3] : r.h[2]) >> (sh + (hi ? 4u : 0u))) & 0x0F0Fu) | ((r.h[2] >> top) & 0x3030u);
        const float d = h2f(r.h[0] & 0xffffu), dmin = h2f(r.h[0] >> 16);
        pr.dsc[0] = d * (float)(scp & 0xffu);       // exact
        pr.dsc[1] = d * (float)(scp >> 8);
        pr.dmn[0] = dmin * (float)(mnp & 0xffu);
        pr.dmn[1] = dmin * (float)(mnp >> 8);
        return pr;
    }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &pr, int g, float (&w)[4]) {
        const int e = g >= 8 ? 1 : 0;
        const uint32_t dw = r.qs[g & 7];
        const uint32_t q4 = opaque(e ? ((dw >> 4) & 0x0F0F0F0Fu) : (dw & 0x0F0F0F0Fu));
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_fmaf(pr.dsc[e], (float)((q4 >> (8 * i)) & 0xffu), -pr.dmn[e]);
    }
    static __device__ __forceinline__ void deqi(const Raw &r, const Pre &, int g, float (&q)[4]) {
        const uint32_t dw = r.qs[g & 7];
        const uint32_t q4 = opaque(g >= 8 ? ((dw >> 4) & 0x0F0F0F0Fu) : (dw & 0x0F0F0F0Fu));
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)((q4 >> (8 * i)) & 0xffu);
    }
    static __device__ __forceinline__ float scale(const Pre &pr, int e) { return pr.dsc[e]; }
    static __device__ __forceinline__ float offset(const Pre &pr, int e) { return pr.dmn[e]; }
    // index of the piece's first segment among the pass's segment sums
    static __device__ __forceinline__ uint32_t sxoff(uint32_t p, uint32_t vb) { return 2 * p - vb / 32; }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) {
        return 256 * (p >> 2) + 64 * (p & 3) + (g >= 8 ? 32 : 0) + 4 * (g & 7);
    }
    // PADP 64: pad index = 4*(super-block) + chunk
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) {
        return 272 * ((p >> 2) - vb / 256) + 68 * (p & 3);
    }
    static constexpr uint32_t goff(int g) { return (g >= 8 ? 32 : 0) + 4 * (g & 7); }
    static __device__ __forceinline__ bool group_valid(uint32_t, int, uint32_t) { return true; }
};

// ---------------------------------------------------------------- Q6_K
// Piece p: super-block p/4, half hh = (p/2)%2, lane column block l0 = 16(p%2):
// values 128hh + 32t + l0 + 0..15 for t = 0..3.  Low 4 bits from
// ql[64hh + 32(t&1) + l] (low nibble for t < 2, high for t >= 2), high 2 bits
// from bits 2t..2t+1 of qh[32hh + l], scale sc[8hh + 2t + l0/16].
// w = (d * sc) * (q - 32), exact.
template <> struct Tr<kQ6K> : Geo<kQ6K> {
    static constexpr int SEG = 4;  // one scale per 16 values (groups 4t..4t+3)
    static constexpr int LOADS = 5;  // 3 x 16 bytes, 8 scale bytes, d
    static constexpr int ITEM_DWORDS = 14;
    // Raw: the piece's bytes as loaded (low bits, high bits, the eight scales
    // of its half, d); Pre (at multiply time): d*sc/4 of its four 16-value
    // segments and the high bits with the top bit of each 2-bit part inverted.
    struct Raw { uint32_t ql0[4], ql1[4], qh[4], sc[2], d; };
    struct Pre { float ds4[4]; uint32_t qhx[4]; };
    // Piece `pos` (0..3) of super-block sb of a row.
    static __device__ __forceinline__ Raw load_at(const uint8_t *R, uint32_t o0, uint32_t sb, uint32_t pos) {
        Raw r;
        const uint32_t hh = pos >> 1, l0 = 16 * (pos & 1);
        // offsets inside the super-block (fixed per lane in the walks), then
        // its start: sb < 2^24 (k < 2^32), so a full-rate 24-bit multiply
        const uint32_t oql = 64 * hh + l0, oqh = 128 + 32 * hh + l0, osc = 192 + 8 * hh;
        const uint32_t B = o0 + __umul24(sb, 210u);
        load16_u(R, B + oql, r.ql0);
        load16_u(R, B + (oql + 32), r.ql1);
        load16_u(R, B + oqh, r.qh);
        const u32x2a2 v = ldv<u32x2a2>(R, B + osc);  // sc[8hh .. 8hh+7]
        r.sc[0] = v.x;
        r.sc[1] = v.y;
        r.d = ld16(R, B + 208);
        return r;
    }
    static __device__ __forceinline__ Raw load(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        return load_at(R, o0, p >> 2, p & 3);
    }
    // The mat-vec walks: every piece whose values are used has p % 4 == lane % 4
    // (a lane's pieces are lane + (a multiple of the lanes per row)), so the
    // position inside the super-block comes from the lane and its offsets
    // stay fixed across the walk; other loads (clamped or past the last item)
    // stay inside the super-block p / 4 and are never used.
    static __device__ __forceinline__ Raw load_walk(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t) {
        return load_at(R, o0, p >> 2, threadIdx.x & 3u);
    }
    // p: the piece (its position in the super-block, p % 4, decides which
    // four of the eight scales are its own).
    static __device__ __forceinline__ Pre prep(const Raw &r, uint32_t p) {
        Pre pr;
        // scale bytes (p & 1) + 0, 2, 4, 6 of the eight (v_perm_b32: selector 0-3 = sc[0], 4-7 = sc[1])
        const uint32_t s4 = __builtin_amdgcn_perm(r.sc[1], r.sc[0], 0x06040200u + 0x01010101u * (p & 1));
        const float d4 = h2f(r.d) * 0.25f;  // exact (a power of two, far from underflow)
#pragma unroll
        for (int t = 0; t < 4; ++t) pr.ds4[t] = d4 * (float)(int8_t)(s4 >> (8 * t));  // exact: d*sc/4
#pragma unroll
        for (int i = 0; i < 4; ++i) pr.qhx[i] = r.qh[i] ^ 0xAAAAAAAAu;  // invert bit 1 of every 2-bit high part
        return pr;
    }
    // Four values at a time: byte i becomes the int8 4*(q_i - 32) (low 4
    // bits in bits 2..5, high 2 bits in bits 6..7 with the top one inverted),
    // converted with one signed-byte convert and scaled by d*sc/4: exactly
    // d*sc*(q-32), sign of zero included.
    static __device__ __forceinline__ uint32_t bytes4(const Raw &r, const Pre &pr, int g) {
        const int t = g >> 2, G = g & 3;
        const uint32_t src = (t & 1) ? r.ql1[G] : r.ql0[G];
        const uint32_t lo = t < 2 ? ((src << 2) & 0x3C3C3C3Cu) : ((src >> 2) & 0x3C3C3C3Cu);
        return ((pr.qhx[G] << (6 - 2 * t)) & 0xC0C0C0C0u) | lo;
    }
    static __device__ __forceinline__ void deq(const Raw &r, const Pre &pr, int g, float (&w)[4]) {
        const uint32_t b = bytes4(r, pr, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (float)(int8_t)(b >> (8 * i)) * pr.ds4[g >> 2];
    }
    static __device__ __forceinline__ void deqi(const Raw &r, const Pre &pr, int g, float (&q)[4]) {
        const uint32_t b = bytes4(r, pr, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)(int8_t)(b >> (8 * i));
    }
    static __device__ __forceinline__ float scale(const Pre &pr, int seg) { return pr.ds4[seg]; }
    static __device__ __forceinline__ uint32_t vpos(uint32_t p, int g) {
        return 256 * (p >> 2) + 128 * ((p >> 1) & 1) + 32 * (g >> 2) + 16 * (p & 1) + 4 * (g & 3);
    }
    // PADP 128: pad index = 2*(super-block) + hh
    static __device__ __forceinline__ uint32_t xoff(uint32_t p, uint32_t vb) {
        const uint32_t sb = (p >> 2) - vb / 256, hh = (p >> 1) & 1;
        return 264 * sb + 132 * hh + 16 * (p & 1);
    }
    static constexpr uint32_t goff(int g) { return 32 * (g >> 2) + 4 * (g & 3); }
    static __device__ __forceinline__ bool group_valid(uint32_t, int, uint32_t) { return true; }
};

template <int T>
__device__ __forceinline__ typename Tr<T>::Raw load_walk(const uint8_t *R, uint32_t o0, uint32_t p, uint32_t k) {
    if constexpr (T == kQ6K)
        return Tr<T>::load_walk(R, o0, p, k);
    else
        return Tr<T>::load(R, o0, p, k);
}

// Per-row output scale of the fused normalisation: either the four
// float64 group sums of each input row's statistic in LDS (part, the
// single-kernel form), or each row's inverse RMS formed from the same sums
// by norm_rows_kernel (inv, one double per input row of the batch entry).
// Both give (float)((double)v * inv) with the same inv; neither: v.
struct RowScale {
    const double *part;
    const double *inv;
    uint32_t k;
    float eps;
    __device__ __forceinline__ float apply(float v, uint32_t j) const {
        if (inv) return (float)((double)v * inv[j]);
        if (!part) return v;
        return (float)((double)v * inv_rms(part + 4 * j, k, eps));
    }
    // 1 / sqrt(mean + eps) from the four group sums, added as (s0 + s1) + (s2 + s3).
    static __device__ __forceinline__ double inv_rms(const double *p4, uint32_t k, float eps) {
        const double s = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        return 1.0 / __builtin_sqrt(s / (double)k + (double)eps);
    }
};

// ---------------------------------------------------------------- reduction

template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Lanes (L, L^32): X keeps lanes 0..31 of X and receives Y's lanes 0..31 in
// its upper half; Y receives X's upper half in its lower half.  X' + Y' is
// X[L] + X[L+32] on lanes 0..31 and Y[L-32] + Y[L] on lanes 32..63.
__device__ __forceinline__ float swap32_add(float x, float y) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// Lanes (L, L^16): rows 0 and 2 get X's row pair sum, rows 1 and 3 Y's.
__device__ __forceinline__ float swap16_add(float x, float y) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

constexpr int pow2ceil(int v) { return v <= 1 ? 1 : 2 * pow2ceil((v + 1) / 2); }

// Sum each of the NR*M accumulators over the L lanes of its row with the
// fixed tree; the lane holding output o = r*M + j of slot `slot` (rows
// slot*NR + r of the wave's group) calls emit(slot, o, sum).
template <int M, int NR, int L, typename Emit>
__device__ __forceinline__ void reduce_tree(const float (&acc)[NR][M], uint32_t lane, Emit &&emit) {
    // L lanes per weight row: slot lane / L of the wave holds rows
    // row0 + slot*NR + r.  The tree over a slot's lanes is the last log2(L)
    // levels of the 64-lane tree.
    constexpr int NA = NR * M;
    constexpr int A = pow2ceil(NA);
    float v[A];
#pragma unroll
    for (int a = 0; a < A; ++a) v[a] = a < NA ? acc[a / M][a % M] : 0.0f;

    // level 1: (L, L^32), 64-lane rows only
    constexpr int A1 = L < 64 ? A : (A >= 2 ? A / 2 : 1);
    if constexpr (L == 64) {
        if constexpr (A >= 2) {
#pragma unroll
            for (int a = 0; a < A1; ++a) v[a] = swap32_add(v[a], v[a + A1]);
        } else {
            v[0] = swap32_add(v[0], v[0]);
        }
    }
    // level 2: (L, L^16), 64- and 32-lane rows
    constexpr int A2 = L < 32 ? A1 : (A1 >= 2 ? A1 / 2 : 1);
    if constexpr (L >= 32) {
        if constexpr (A1 >= 2) {
#pragma unroll
            for (int a = 0; a < A2; ++a) v[a] = swap16_add(v[a], v[a + A2]);
        } else {
            v[0] = swap16_add(v[0], v[0]);
        }
    }
    // levels 3..6 inside each row of 16 lanes
    constexpr int AN = L < 32 ? NA : A2;
#pragma unroll
    for (int a = 0; a < AN; ++a) {
        v[a] = v[a] + dpp_mov<0x128>(v[a]);  // row_ror:8     (L, L^8)
        v[a] = v[a] + dpp_mov<0x141>(v[a]);  // row_half_mirror (L, 7-L)
        v[a] = v[a] + dpp_mov<0x4E>(v[a]);   // quad_perm 2,3,0,1
        v[a] = v[a] + dpp_mov<0xB1>(v[a]);   // quad_perm 1,0,3,2
    }

    // Which lanes hold which outputs of their slot.  L == 64: A >= 4: row
    // R = lane/16 holds outputs R*A2 + a; A == 2: lanes 0..31 output 0,
    // lanes 32..63 output 1; A == 1: lane 0.  L == 32: A >= 2: the 16-lane
    // row R of the slot holds outputs R*A2 + a; A == 1: the slot's first lane.
    // L == 16: the row's first lane holds all outputs.
    uint32_t base, slot;
    bool holder;
    if constexpr (L == 64) {
        slot = 0;
        if constexpr (A >= 4) {
            holder = (lane & 15) == 0;
            base = (lane >> 4) * A2;
        } else if constexpr (A == 2) {
            holder = (lane & 31) == 0;
            base = lane >> 5;
        } else {
            holder = lane == 0;
            base = 0;
        }
    } else if constexpr (L == 32) {
        slot = lane >> 5;
        if constexpr (A >= 2) {
            holder = (lane & 15) == 0;
            base = ((lane >> 4) & 1) * A2;
        } else {
            holder = (lane & 31) == 0;
            base = 0;
        }
    } else {
        slot = lane >> 4;
        holder = (lane & 15) == 0;
        base = 0;
    }
    if (holder) {
#pragma unroll
        for (int a = 0; a < AN; ++a) {
            const uint32_t o = base + a;
            if (o < (uint32_t)NA) emit(slot, o, v[a]);
        }
    }
}

// The tree, then output (r, j) of slot s to y[j*yrs + row0 + s*NR + r] when
// that row is < n.
template <int M, int NR, int L>
__device__ __forceinline__ void reduce_store(const float (&acc)[NR][M], float *__restrict__ yb, uint32_t yrs,
                                             uint32_t n, uint32_t row0, uint32_t lane, const RowScale &sc) {
    reduce_tree<M, NR, L>(acc, lane, [&](uint32_t slot, uint32_t o, float v) {
        const uint32_t r = o / M, j = o % M;
        const uint32_t row = row0 + slot * NR + r;
        if (row < n) yb[(uint64_t)j * yrs + row] = sc.apply(v, j);
    });
}

// K-split reduction (K waves per row group): each wave's 64-lane tree sums
// go to LDS (kp[wave][o], 32 floats per wave), and after a barrier the
// group's first wave adds the K partials of each output by a fixed pairwise
// tree over the split index, ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 +
// p7)) truncated to K terms, then stores.  Every wave of the workgroup must
// call it (it holds two barriers).
template <int M, int NR>
__device__ __forceinline__ void reduce_store_split(const float (&acc)[NR][M], float *__restrict__ kp, uint32_t K,
                                                   uint32_t wave, uint32_t ws, bool active, float *__restrict__ yb,
                                                   uint32_t yrs, uint32_t n, uint32_t row0, uint32_t lane,
                                                   const RowScale &sc) {
    constexpr int NA = NR * M;
    static_assert(NA <= 32, "32 partials per wave");
    reduce_tree<M, NR, 64>(acc, lane, [&](uint32_t, uint32_t o, float v) { kp[wave * 32 + o] = v; });
    __syncthreads();
    if (active && ws == 0 && lane < (uint32_t)NA) {
        const float *p = kp + wave * 32 + lane;
        float s;
        if (K == 2) {
            s = p[0] + p[32];
        } else if (K == 4) {
            s = (p[0] + p[32]) + (p[64] + p[96]);
        } else {
            s = ((p[0] + p[32]) + (p[64] + p[96])) + ((p[128] + p[160]) + (p[192] + p[224]));
        }
        const uint32_t r = lane / M, j = lane % M;
        const uint32_t row = row0 + r;
        if (row < n) yb[(uint64_t)j * yrs + row] = sc.apply(s, j);
    }
    __syncthreads();
}

// ---------------------------------------------------------------- x staging

// Float offset, in a staged input row of an M-row product, of value lv (a
// multiple of 4, counted from the pass' first value): value order with 4 pad
// floats after every Geo<T>::PADP values, or, piece-major (piece_major:
// Q6_K from M = 2), piece q's 64 values (its four 16-value runs, in order)
// at 68 q, followed by 4 pad floats.
template <int T, int M> __device__ __forceinline__ uint32_t lpos(uint32_t lv) {
    if constexpr (piece_major(T, M)) {
        const uint32_t r = lv & 255u;  // value in its super-block
        const uint32_t piece = 4 * (lv >> 8) + 2 * (r >> 7) + ((r >> 4) & 1u);
        return 68 * piece + 16 * ((r >> 5) & 3u) + (r & 15u);
    } else {
        return lv + 4 * (lv / Geo<T>::PADP);
    }
}

// Data slots (16 bytes) per pad period of a staged row.
template <int T, int M> constexpr uint32_t slots_per_period() { return piece_major(T, M) ? 16u : Geo<T>::PADP / 4; }

// The 4-value chunk of the input row (its first value / 4, from the pass'
// first value) held by data slot r of pad period per of a staged row: the
// inverse of lpos on 16-byte slots.
template <int T, int M> __device__ __forceinline__ uint32_t slot_chunk(uint32_t per, uint32_t r) {
    if constexpr (piece_major(T, M)) {
        // per = piece (super-block per / 4, quarter per % 4), r = 4 t + w4
        return 64 * (per >> 2) + 32 * ((per >> 1) & 1u) + 8 * (r >> 2) + 4 * (per & 1u) + (r & 3u);
    } else {
        return per * slots_per_period<T, M>() + r;
    }
}

// LDS offset of piece p's staged values (pass' first value vb) and of its
// group g: the type's value-order offsets, or, piece-major, 68 (p - vb / 64)
// and 4 g (sixteen consecutive pieces then start on sixteen distinct 4-bank
// groups of the 64 LDS banks, so a wave's reads of one group do not
// conflict).
template <int T, int M> __device__ __forceinline__ uint32_t xoff_of(uint32_t p, uint32_t vb) {
    if constexpr (piece_major(T, M)) return 68 * (p - vb / 64);
    else return Tr<T>::xoff(p, vb);
}
template <int T, int M> __device__ __forceinline__ constexpr uint32_t goff_of(int g) {
    if constexpr (piece_major(T, M)) return 4 * g;
    else return Tr<T>::goff(g);
}

// Stage values [v0, v1) of the m input rows into LDS.
template <int T, int M>
__device__ __forceinline__ void stage_x(float *__restrict__ xs, const float *__restrict__ xb, uint32_t xrs,
                                        uint32_t v0, uint32_t v1, uint32_t XS) {
    // Up to 8 float4 loads per thread in flight before the LDS writes.
    constexpr int U = M >= 8 ? 1 : 8 / M;
    const uint32_t n4 = (v1 - v0) >> 2;
    const uint32_t nt = blockDim.x;
    for (uint32_t q0 = threadIdx.x; q0 < n4; q0 += U * nt) {
        f32x4 v[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t q = q0 + u * nt;
            if (q < n4) {
#pragma unroll
                for (int j = 0; j < M; ++j) v[u][j] = *(const f32x4 *)(xb + (uint64_t)j * xrs + v0 + 4 * q);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t q = q0 + u * nt;
            if (q < n4) {
                const uint32_t lv = 4 * q;
                const uint32_t d = lpos<T, M>(lv);
#pragma unroll
                for (int j = 0; j < M; ++j) *(f32x4 *)(xs + j * XS + d) = v[u][j];
            }
        }
    }
}

// The same for few input rows, with `between` run once after the first
// batch of loads is issued and before any of it is written to LDS (the
// caller issues its first weight loads there): x is then a few loads per
// thread that arrive well before the weights, and the barrier after the
// staging does not wait for every wave's weights.
template <int T, int M, typename F>
__device__ __forceinline__ void stage_x_first(float *__restrict__ xs, const float *__restrict__ xb, uint32_t xrs,
                                              uint32_t k, uint32_t XS, F &&between) {
    // Chunks per thread requested ahead of the weights: at 512 threads, all
    // of x up to k = 4096 (m = 1, m >= 5) or 8192 (m = 2..4).  The rest goes
    // behind the weights, and the staging barrier then waits for them too.
    // At m = 2..4 a whole k = 4096 row ahead measured 2-12% faster than half
    // of it; at m = 1 more chunks ahead cost occupancy (the staging
    // registers exceed the walk's) and measured 15-75% slower.
    constexpr int U = (M >= 2 && M <= 4) ? 4 : 2;
    const uint32_t n4 = k >> 2;
    const uint32_t nt = blockDim.x;
    f32x4 v[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t q = threadIdx.x + u * nt;
        if (q < n4) {
#pragma unroll
            for (int j = 0; j < M; ++j) v[u][j] = *(const f32x4 *)(xb + (uint64_t)j * xrs + 4 * q);
        }
    }
    between();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t q = threadIdx.x + u * nt;
        if (q < n4) {
            const uint32_t lv = 4 * q;
            const uint32_t d = lpos<T, M>(lv);
#pragma unroll
            for (int j = 0; j < M; ++j) *(f32x4 *)(xs + j * XS + d) = v[u][j];
        }
    }
    // the rest (k > 4 U nt), behind the weights
    for (uint32_t q = threadIdx.x + U * nt; q < n4; q += nt) {
        const uint32_t lv = 4 * q;
        const uint32_t d = lpos<T, M>(lv);
#pragma unroll
        for (int j = 0; j < M; ++j) *(f32x4 *)(xs + j * XS + d) = *(const f32x4 *)(xb + (uint64_t)j * xrs + lv);
    }
}

// x staged by loads that write LDS directly (gfx950 global_load_lds_dwordx4:
// lane L of a wave writes the 16 bytes it reads to lds + 16 L, no VGPRs), so
// all of x can be requested ahead of the weights whatever its size.  Used
// where x is larger than the register staging requests ahead of the weights
// (see the host's x_dma), for the types whose Tr<T>::LOADS gives the fixed
// number of load instructions of a piece (Q6_K); the others keep the
// register staging: the extra code path cost them 1-9% at m = 1 on MI355X.  Each wave
// instruction fills 64 consecutive 16-byte slots of one staged row (pad
// periods of Geo<T>::PADP / 4 data slots and one pad slot); a lane reads the
// x chunk its slot holds (slot_chunk), pad slots and slots past the row are
// masked off.
// Completion is counted by vmcnt with the other loads, in issue order: the
// caller waits with barrier_after_loads, never with __syncthreads.
__device__ __forceinline__ void lds_dma16(const float *src, float *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

template <int T, int M>
__device__ __forceinline__ void stage_x_dma(float *__restrict__ xs, const float *__restrict__ xb, uint32_t xrs,
                                            uint32_t k, uint32_t XS, uint32_t wave, uint32_t nwaves, uint32_t lane) {
    constexpr uint32_t P = slots_per_period<T, M>();  // data slots per pad period
    const uint32_t S = XS / 4;                 // slots per staged row
    const uint32_t bpr = (S + 63) >> 6;        // 64-slot blocks per row
    const uint32_t n4 = k >> 2;
    for (uint32_t t = wave; t < (uint32_t)M * bpr; t += nwaves) {
        const uint32_t j = t / bpr, b = t - j * bpr;
        const uint32_t s = (b << 6) + lane;
        const uint32_t per = s / (P + 1), r = s - per * (P + 1);
        const uint32_t d = slot_chunk<T, M>(per, r);
        if (r < P && d < n4) lds_dma16(xb + (uint64_t)j * xrs + 4 * d, xs + j * XS + (b << 8));
    }
}

// s_waitcnt immediate (gfx9 layout): vmcnt n, expcnt and lgkmcnt not waited on.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Barrier after this wave's loads issued before its last N load
// instructions have completed: loads complete in issue order, so the x
// chunks staged ahead of N weight loads are in LDS, while those weight loads
// stay in flight.  N must be the exact number of load instructions issued
// after the staging (fewer would wait for weights; more would let the
// barrier pass before x is in LDS: a CPU test reads the count out of the
// built code).  The fence after the barrier is acquire-only: a release
// fence would make the compiler wait for every load in flight (it counts
// the LDS-writing loads as outstanding LDS stores), and without any fence it
// was free to regroup the walk's weight loads ahead of their multiplies
// (then each step waited for all of them).
template <int N> __device__ __forceinline__ void barrier_after_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
    __builtin_amdgcn_s_waitcnt(vmcnt_only(N));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Segment sums of the staged input (offset types): sx[j*SXS + s] = the sum
// of staged values 32s .. 32s+31 of input row j by one fixed pairwise tree
// (each 4 values as (a+b)+(c+d), then the 8 sums pairwise, in order), the
// same steps for every m and every packing.  Needs the staged values
// written (a barrier) and a barrier before use.
template <int T, int M>
__device__ __forceinline__ void stage_sx(const float *__restrict__ xs, uint32_t XS, float *__restrict__ sx,
                                         uint32_t SXS, uint32_t nvals) {
    static_assert(Geo<T>::PADP % 32 == 0, "a segment must not straddle a pad");
    const uint32_t nseg = nvals / 32;
    for (uint32_t i = threadIdx.x; i < M * nseg; i += blockDim.x) {
        const uint32_t j = i / nseg, sg = i - j * nseg;
        const uint32_t lv = 32 * sg;
        const float *__restrict__ src = xs + j * XS + lpos<T, M>(lv);
        f32x4 v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = *(const f32x4 *)(src + 4 * c);
        float t[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) t[c] = (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
        sx[j * SXS + sg] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    }
}

// ---------------------------------------------------------------- fused add + RMS norm
//
// nuvec-core 0.6.0, src/gpu.rs, add_rms_norm (FastOp::AddRmsNorm): the sum
// h = x + r and its RMS normalisation h / sqrt(mean(h^2) + eps) * g, here
// fused into the mat-vec.  The normalisation is linear in h per input row, so
// the kernel stages u = h * g (one float32 rounding), runs the row-exact fma
// chains and reduction on u, and scales each output once by the row's inverse
// RMS: y = (float)((double)sum * inv).
//
// The statistic of input row j is summed in float64 in one fixed order: the
// row's float4 chunks q are split over 256 virtual lanes (q mod 256), each
// summing the squares of its chunks' h values in increasing q; each group of
// 64 virtual lanes is reduced by a fixed xor tree, and the four group sums
// are added as (s0 + s1) + (s2 + s3).  Workgroups with any number of waves
// compute the same value (a wave takes whole 64-lane groups), and the single-
// and multi-pass paths take the same steps, so outputs stay row-exact.
//
// LDS layout after the staged x: part[M][4] (double).

__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, mask, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), mask, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double fold4(double ss, f32x4 h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = __builtin_fma((double)h[i], (double)h[i], ss);
    return ss;
}

__device__ __forceinline__ f32x4 times_g(f32x4 h, const float *__restrict__ g, uint32_t v) {
    if (!g) return h;
    const f32x4 gv = *(const f32x4 *)(g + v);
    f32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = h[i] * gv[i];
    return u;
}

// The four group sums of every input row into part[j*4 + group], with
// h = x + r read from memory; h is also written to hb (when not NULL; every
// chunk is visited exactly once) and, with TO_LDS, u = h * g staged into xs
// in the padded x layout (single pass).
//
// Work is dealt as pairs (row j, virtual lane v).  With a multiple of 256
// threads a thread keeps v = tid mod 256 and takes rows tid/256, tid/256 +
// nt/256, ...; otherwise it takes v = tid, tid + nt, ... < 256 for every
// row.  Either way the 64 lanes of a wave hold the 64 virtual lanes of one
// group of one row, so the group's xor tree runs inside the wave.  The loads
// of JB rows x CB chunks are issued together (at k <= 4096 and 8 waves: two
// batches for m <= 2, where registers buy occupancy; one for m = 3, 4; two
// for m > 4), g once per chunk for the JB rows when JB > 1.  The caller's
// weight loads go out first: loads complete in issue order, and x / r / g
// requested ahead of them delayed the weights more than it saved.
template <int T, int M, bool TO_LDS>
__device__ __forceinline__ void norm_partials(double *part, float *__restrict__ xs, uint32_t XS,
                                              const float *__restrict__ xb, const float *__restrict__ rb,
                                              const float *__restrict__ g, float *__restrict__ hb, uint32_t xrs,
                                              uint32_t k, uint32_t wave, uint32_t nwaves, uint32_t lane) {
    // rows per batch: from m = 4, half the rows (with 256-thread row
    // groups, a thread's rows of one parity in one batch: one round trip
    // for x and r instead of two; fused Q8_0 4096 x 4096 at m = 5..8: -2
    // to -6% against two rows per batch)
    constexpr int JB = M >= 4 ? (M + 1) / 2 : 1;
    // chunks per row per batch (few rows: registers for occupancy; 4 at m <= 2
    // measured 3% slower on fused Q8_0 4096 x 4096)
    constexpr int CB = M <= 2 ? 2 : 4;
    const uint32_t n4 = k >> 2;
    const uint32_t nt = nwaves << 6, tid = (wave << 6) + lane;
    const bool wide = (nt & 255u) == 0;
    const uint32_t v_step = wide ? 256u : nt;
    const uint32_t j_first = wide ? (tid >> 8) : 0u, j_step = wide ? (nt >> 8) : 1u;
    const float *__restrict__ gg = TO_LDS ? g : nullptr;
    for (uint32_t v = wide ? (tid & 255u) : tid; v < 256u; v += v_step) {
        const uint32_t v0 = v & ~63u;  // the wave's first virtual lane (loop bounds stay wave-uniform)
        for (uint32_t jb = j_first; jb < (uint32_t)M; jb += JB * j_step) {
            double ss[JB];
#pragma unroll
            for (int i = 0; i < JB; ++i) ss[i] = 0.0;
            for (uint32_t c0 = 0; v0 + 256u * c0 < n4; c0 += CB) {
                // chunks q = v + 256 c, c = c0 .. c0 + CB - 1, of rows jb + i * j_step
                f32x4 xv[JB][CB], rv[JB][CB], gv[CB];
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    const uint32_t q = v + 256u * (c0 + c);
                    if (q < n4) {
                        if (JB > 1 && gg) gv[c] = *(const f32x4 *)(gg + 4 * q);
#pragma unroll
                        for (int i = 0; i < JB; ++i) {
                            const uint32_t j = jb + i * j_step;
                            if (j < M) {
                                xv[i][c] = *(const f32x4 *)(xb + (uint64_t)j * xrs + 4 * q);
                                rv[i][c] = *(const f32x4 *)(rb + (uint64_t)j * xrs + 4 * q);
                            }
                        }
                    }
                }
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    const uint32_t q = v + 256u * (c0 + c);
                    if (q < n4) {
                        if (JB == 1 && gg) gv[c] = *(const f32x4 *)(gg + 4 * q);
#pragma unroll
                        for (int i = 0; i < JB; ++i) {
                            const uint32_t j = jb + i * j_step;
                            if (j < M) {
                                f32x4 h;
#pragma unroll
                                for (int e = 0; e < 4; ++e) h[e] = xv[i][c][e] + rv[i][c][e];
                                if (hb) *(f32x4 *)(hb + (uint64_t)j * xrs + 4 * q) = h;
                                if constexpr (TO_LDS) {
                                    const uint32_t lv = 4 * q;
                                    f32x4 u = h;
                                    if (gg) {
#pragma unroll
                                        for (int e = 0; e < 4; ++e) u[e] = h[e] * gv[c][e];
                                    }
                                    *(f32x4 *)(xs + j * XS + lpos<T, M>(lv)) = u;
                                }
                                ss[i] = fold4(ss[i], h);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int msk = 32; msk >= 1; msk >>= 1) {
#pragma unroll
                for (int i = 0; i < JB; ++i) ss[i] += shfl_xor_d(ss[i], msk);
            }
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < JB; ++i) {
                    const uint32_t j = jb + i * j_step;
                    if (j < M) part[4 * j + (v >> 6)] = ss[i];
                }
            }
        }
    }
}

// Multi-pass: stage values [v0, v1) of u = (x + r) * g.
template <int T, int M>
__device__ __forceinline__ void stage_u(float *__restrict__ xs, const float *__restrict__ xb,
                                        const float *__restrict__ rb, const float *__restrict__ g, uint32_t xrs,
                                        uint32_t v0, uint32_t v1, uint32_t XS) {
    const uint32_t n4 = (v1 - v0) >> 2;
    for (uint32_t q = threadIdx.x; q < n4; q += blockDim.x) {
        const uint32_t v = v0 + 4 * q;
        const uint32_t lv = 4 * q;
        const uint32_t d = lpos<T, M>(lv);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const f32x4 xv = *(const f32x4 *)(xb + (uint64_t)j * xrs + v);
            const f32x4 rv = *(const f32x4 *)(rb + (uint64_t)j * xrs + v);
            f32x4 h;
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = xv[i] + rv[i];
            *(f32x4 *)(xs + j * XS + d) = times_g(h, g, v);
        }
    }
}


// ---------------------------------------------------------------- one piece

// Types whose segments carry an offset term (- offset * sum of the
// segment's x) besides the scale.
template <int T> constexpr bool kOffsets = T == kQ4K;

template <int T, int M, int NR>
__device__ __forceinline__ void compute_piece(float (&acc)[NR][M], const typename Tr<T>::Raw (&raw)[NR], uint32_t p,
                                              uint32_t vb, const float *__restrict__ xs, uint32_t XS, uint32_t k,
                                              const float *__restrict__ sx, uint32_t SXS) {
    using TR = Tr<T>;
    typename TR::Pre pre[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) pre[r] = TR::prep(raw[r], p);
    const float *__restrict__ xp = xs + xoff_of<T, M>(p, vb);
    if constexpr (TR::SEG == 0) {
        // unscaled: acc = fma(w, x, acc) value by value
#pragma unroll
        for (int g = 0; g < TR::NG; ++g) {
            if (!TR::group_valid(p, g, k)) continue;
            f32x4 xv[M];
#pragma unroll
            for (int j = 0; j < M; ++j) xv[j] = *(const f32x4 *)(xp + j * XS + goff_of<T, M>(g));
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float w[4];
                TR::deq(raw[r], pre[r], g, w);
#pragma unroll
                for (int j = 0; j < M; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[r][j] = __builtin_fmaf(w[i], xv[j][i], acc[r][j]);
                }
            }
        }
    } else {
        // scaled: a segment's values share one scale s, so the segment
        // contributes s * sum(q * x); the inner chain multiplies the exact
        // integer-valued q, and one fma folds the segment into acc.  The x
        // values of group g+1 are read while group g is multiplied, and the
        // scheduler is kept from hoisting further reads (register pressure).
        f32x4 xv[2][M];
#pragma unroll
        for (int j = 0; j < M; ++j) xv[0][j] = *(const f32x4 *)(xp + j * XS + goff_of<T, M>(0));
        float part[NR][M];
        // the sums of x over the piece's two segments (offset types)
        f32x2 sv[M];
        if constexpr (kOffsets<T>) {
#pragma unroll
            for (int j = 0; j < M; ++j) sv[j] = *(const f32x2 *)(sx + j * SXS + TR::sxoff(p, vb));
        }
#pragma unroll
        for (int g = 0; g < TR::NG; ++g) {
            const int gg = g % TR::SEG, cb = g & 1;
            if (g + 1 < TR::NG) {
#pragma unroll
                for (int j = 0; j < M; ++j) xv[cb ^ 1][j] = *(const f32x4 *)(xp + j * XS + goff_of<T, M>(g + 1));
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float q[4];
                TR::deqi(raw[r], pre[r], g, q);
#pragma unroll
                for (int j = 0; j < M; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part[r][j] = (gg == 0 && i == 0) ? q[0] * xv[cb][j][0]
                                                         : __builtin_fmaf(q[i], xv[cb][j][i], part[r][j]);
                }
            }
            if (gg == TR::SEG - 1) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float sc = TR::scale(pre[r], g / TR::SEG);
#pragma unroll
                    for (int j = 0; j < M; ++j) acc[r][j] = __builtin_fmaf(sc, part[r][j], acc[r][j]);
                    if constexpr (kOffsets<T>) {
                        const float of = TR::offset(pre[r], g / TR::SEG);
#pragma unroll
                        for (int j = 0; j < M; ++j) acc[r][j] = __builtin_fmaf(-of, sv[j][g / TR::SEG], acc[r][j]);
                    }
                }
            }
            if (M >= REX_SCHED_BARRIER_MIN_M) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Pieces pb + lane, pb + lane + stride, ... below pe of the NR rows (lane:
// the lane's index in its row slot; stride: the lanes per row, or 64 K for
// the K-split, whose wave ws starts at pb + 64 ws), with the next piece's
// loads issued before the current piece's math.
template <int T, int M, int NR>
__device__ __forceinline__ void accumulate(float (&acc)[NR][M], const uint8_t *const (&R)[NR],
                                           const uint32_t (&o0)[NR], uint32_t pb, uint32_t pe, uint32_t vb,
                                           const float *__restrict__ xs, uint32_t XS, uint32_t k, uint32_t lane,
                                           const float *__restrict__ sx, uint32_t SXS, uint32_t stride) {
    using TR = Tr<T>;
    using Raw = typename TR::Raw;
    uint32_t p = pb + lane;
    if (p >= pe) return;
    Raw A[NR], B[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) A[r] = load_walk<T>(R[r], o0[r], p, k);
    while (true) {
        const uint32_t p1 = p + stride;
        const bool m1 = p1 < pe;
#pragma unroll
        for (int r = 0; r < NR; ++r) B[r] = load_walk<T>(R[r], o0[r], m1 ? p1 : p, k);
        compute_piece<T, M, NR>(acc, A, p, vb, xs, XS, k, sx, SXS);
        if (!m1) break;
        const uint32_t p2 = p1 + stride;
        const bool m2 = p2 < pe;
#pragma unroll
        for (int r = 0; r < NR; ++r) A[r] = load_walk<T>(R[r], o0[r], m2 ? p2 : p1, k);
        compute_piece<T, M, NR>(acc, B, p1, vb, xs, XS, k, sx, SXS);
        if (!m2) break;
        p = p2;
    }
}

// Wave-uniform base of a row that starts at rp and the row's offset from it:
// rp aligned down to 4 bytes, unless that falls before the first weight byte
// Wlo: then rp itself.  W and every row start are 2-byte aligned, so that
// happens exactly for the first row of a W 2 bytes past a 4-byte boundary
// (a scalar 64-bit equality; an ordered 64-bit compare would take vector
// instructions).  The block loads read at or after base + offset - 2 only
// where the base is 4-byte aligned (Q5_0's header dwords; see
// Tr<kQ5_0>::load), so nothing before W is read.
__device__ __forceinline__ void row_base(const uint8_t *Wlo, const uint8_t *rp, const uint8_t *&R, uint32_t &o0) {
    const uint32_t lo = (uint32_t)(uintptr_t)rp & 3u;
    o0 = rp == Wlo ? 0u : lo;
    R = rp - o0;
}

// Wave-uniform base and per-lane byte offset of each of a lane's rows: row0 +
// r for the wave's first slot, plus slot_rows for the lane's slot (short
// rows; slot_rows = 0 with 64 lanes per row).  Rows past n are clamped to
// n - 1 (read, never stored).
template <int NR>
__device__ __forceinline__ void row_bases(const uint8_t *Wlo, const uint8_t *Wb, uint64_t row_bytes, uint32_t n,
                                          uint32_t row0, bool sub_wave, uint32_t slot_rows, const uint8_t *(&R)[NR],
                                          uint32_t (&o0)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const uint32_t row = min(row0 + r, n - 1);
        row_base(Wlo, Wb + (uint64_t)row * row_bytes, R[r], o0[r]);
        if (sub_wave) o0[r] += (uint32_t)((min(row0 + slot_rows + r, n - 1) - row) * row_bytes);
    }
}

// log2 of the lanes per row: 6 for the 64-lane instances, a.lpr_log2 (5 or
// 4) for the short-row instances.
template <bool SUB> __device__ __forceinline__ uint32_t lpr_of(const MvArgs &a) { return SUB ? a.lpr_log2 : 6u; }

template <int T, int NR, bool SUB>
__device__ __forceinline__ void load_item(const uint8_t *Wb, const MvArgs &a, uint32_t g, uint32_t p,
                                          uint32_t slot, typename Tr<T>::Raw (&raw)[NR]) {
    const uint8_t *R[NR];
    uint32_t o0[NR];
    row_bases<NR>(a.W, Wb, a.row_bytes, a.n, (g * NR) << (6 - lpr_of<SUB>(a)), SUB, slot * NR, R, o0);
#pragma unroll
    for (int r = 0; r < NR; ++r) raw[r] = load_walk<T>(R[r], o0[r], p, a.k);
}

// The group's outputs, with the tree for the lanes-per-row of this k.
template <int M, int NR, bool SUB>
__device__ __forceinline__ void store_group(const MvArgs &a, const float (&acc)[NR][M], float *__restrict__ yb,
                                            uint32_t g, uint32_t lane, const RowScale &sc) {
    const uint32_t row0 = (g * NR) << (6 - lpr_of<SUB>(a));
    if constexpr (!SUB)
        reduce_store<M, NR, 64>(acc, yb, a.yrs, a.n, row0, lane, sc);
    else if (a.lpr_log2 == 5)
        reduce_store<M, NR, 32>(acc, yb, a.yrs, a.n, row0, lane, sc);
    else
        reduce_store<M, NR, 16>(acc, yb, a.yrs, a.n, row0, lane, sc);
}

template <int M, int NR> __device__ __forceinline__ void zero(float (&acc)[NR][M]) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int j = 0; j < M; ++j) acc[r][j] = 0.0f;
}

// Items in flight ahead of the one being multiplied (1 or 2), chosen so the
// buffers of 1 + DEPTH items stay within the register budget (a third item
// in flight measured no faster at m <= 2).  ITEM_DWORDS: a piece's decoded
// size in dwords (the budget was measured with the pieces held decoded).
template <int T, int M, int NR> struct Depth {
    static constexpr int raw_dwords = Tr<T>::ITEM_DWORDS * NR;
    static constexpr int value = (raw_dwords * 3 + 2 * NR * M <= REX_DEPTH_BUDGET) ? 2 : 1;
};

// Loads the item at the load cursor (lg, ls) into dst and advances the
// cursor.  UNC: the loads are issued even past the wave's last item (then
// every lane reads piece 0 of the workgroup's last group, one line), so the
// code is straight-line and the compiler's wait before a multiply covers
// exactly the item being multiplied; with the loads under a branch it has to
// assume either path and waits for the items still in flight as well.  The
// branch form is kept for waves with at most DEPTH items, where the extra
// loads would cost more than the waits.
template <int T, int NR, bool SUB, bool UNC>
__device__ __forceinline__ void fetch_item(const uint8_t *__restrict__ Wb, const MvArgs &a, uint32_t &lg, uint32_t &ls,
                                           uint32_t g1, uint32_t gstride, uint32_t S, uint32_t li, uint32_t slot,
                                           typename Tr<T>::Raw (&dst)[NR]) {
    const bool have = lg < g1;
    if (UNC || have)
        load_item<T, NR, SUB>(Wb, a, have ? lg : g1 - 1,
                              have ? min((ls << lpr_of<SUB>(a)) + li, a.pieces - 1) : 0u, slot, dst);
    if (have && ++ls == S) {
        ls = 0;
        lg += gstride;
    }
}

// One step of the single-pass walk.  Items are (row group g, step s):
// pieces L*s + li of the group's rows, for the lane's index li < L in its
// row slot (L lanes per row; L = 64: one slot of NR rows).  The load cursor (lg, ls) runs
// DEPTH items ahead of the compute cursor (cg, cs): the step loads the item
// at the load cursor into `nxt`, multiplies `cur`, and stores a group's
// outputs after its last step.  Returns whether items remain.
template <int T, int M, int NR, bool SUB, bool UNC>
__device__ __forceinline__ bool walk_step(const MvArgs &a, const uint8_t *__restrict__ Wb, float *__restrict__ yb,
                                          const float *__restrict__ xs, uint32_t XS, uint32_t &lg, uint32_t &ls,
                                          uint32_t &cg, uint32_t &cs, uint32_t gstride, uint32_t g1, uint32_t S,
                                          uint32_t lane, uint32_t li, uint32_t slot, const RowScale &sc,
                                          const typename Tr<T>::Raw (&cur)[NR], typename Tr<T>::Raw (&nxt)[NR],
                                          float (&acc)[NR][M]) {
    fetch_item<T, NR, SUB, UNC>(Wb, a, lg, ls, g1, gstride, S, li, slot, nxt);
    const uint32_t pc = (cs << lpr_of<SUB>(a)) + li;
    if (pc < a.pieces)
        compute_piece<T, M, NR>(acc, cur, pc, 0, xs, XS, a.k, (const float *)((const uint8_t *)xs + a.sx_offset),
                                a.sx_stride);
    if (cs == S - 1) {
        store_group<M, NR, SUB>(a, acc, yb, cg, lane, sc);
        zero<M, NR>(acc);
    }
    if (++cs == S) {
        cs = 0;
        cg += gstride;
    }
    return cg < g1;
}

// ---------------------------------------------------------------- kernels

// SUB: instances for short rows (32 or 16 lanes per row, a.lpr_log2 5 / 4);
// the others have 64 lanes per row as compile-time constants.  NORM: the
// instances with the fused add + RMS normalisation (a.r != NULL); kept apart
// so that its prologue's registers do not cost the plain product occupancy.
template <int T, int M, int NR, bool SUB, bool NORM, bool UNC>
__global__ void __launch_bounds__(512) mv_kernel(const MvArgs a) {
    extern __shared__ float xs[];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nwaves = blockDim.x >> 6;
    // Batch-fastest flattening: workgroup w of batch entry b is w*batch + b.
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its
    // own L2), so with a batch that is a multiple of 8 every entry's
    // workgroups share one XCD and its x is fetched into one L2 instead of
    // all eight (16 grouped entries at m = 8: -7.6%; batch-1 launches
    // unaffected).
    const uint32_t w = blockIdx.x / a.batch;
    const uint32_t b = blockIdx.x - w * a.batch;
    const float *__restrict__ xb = a.x + b * a.xbs;
    float *__restrict__ yb = a.y + b * a.ybs;
    const uint32_t g0 = w * a.groups_per_wg;
    const uint32_t g1 = min(g0 + a.groups_per_wg, a.groups_per_batch);
    // Weight set of this batch entry: b, or ids[b] for a gathered product.
    // An id outside [0, num_experts) reads nothing and yields NaN outputs.
    uint64_t wsel = b;
    if (a.ids) {
        const int32_t e = a.ids[b];
        if (e < 0 || (uint32_t)e >= a.num_experts) {
            const uint32_t r1 = min((g1 * NR) << (6 - lpr_of<SUB>(a)), a.n);
            for (uint32_t row = ((g0 * NR) << (6 - lpr_of<SUB>(a))) + threadIdx.x; row < r1; row += blockDim.x) {
#pragma unroll
                for (int j = 0; j < M; ++j) yb[(uint64_t)j * a.yrs + row] = __builtin_nanf("");
            }
            return;
        }
        wsel = (uint32_t)e;
    }
    const uint8_t *__restrict__ Wb = a.W + wsel * a.batch_bytes;
    const uint32_t XS = a.xs_stride;

    if (a.nchunks == 1 && a.k_split == 1) {
        // Single pass: the wave walks (row group, wave step) items of its
        // groups g0+wave, g0+wave+nwaves, ... with DEPTH items of loads in
        // flight.  The first DEPTH items are requested before x is staged.
        using Raw = typename Tr<T>::Raw;
        constexpr int DEPTH = Depth<T, M, NR>::value;
        const uint32_t lpr = lpr_of<SUB>(a);
        const uint32_t li = lane & ((1u << lpr) - 1), slot = lane >> lpr;
        const uint32_t S = (a.pieces + (1u << lpr) - 1) >> lpr;
        uint32_t lg = g0 + wave, ls = 0;
        const uint32_t gfirst = lg;
        Raw A[NR], B[NR], C[NR];
        double *part = (double *)((uint8_t *)xs + a.norm_offset);
        const RowScale sc{NORM ? part : nullptr, a.row_scale ? a.row_scale + (uint64_t)b * a.row_scale_stride : nullptr,
                          a.k, a.eps};
        // The first DEPTH items' loads: straight-line (see fetch_item) for
        // the unconditional walk and for x staged ahead of them (so that the
        // x loads can be waited for without them); under a branch otherwise
        // (measured faster for waves of one or two items at m >= 3).
        // x ahead of the weights: up to REX_X_FIRST_MAX_M input rows, and
        // from REX_X_FIRST_UNC_MIN_M on in the unconditional walk (three or
        // more items per wave: the walk staggers the later items' loads
        // itself, and the barrier should not wait behind the first ones;
        // m = 6 / 8: BF16 -3%, Q4_K -1% / -5%, F32 -1% / -2%; at m = 5 it
        // measured mixed, up to +4%); waves of one or two items take the
        // late half-workgroup issue below instead.
        constexpr bool XF = M <= REX_X_FIRST_MAX_M || (UNC && M >= REX_X_FIRST_UNC_MIN_M);
        // x by LDS DMA ahead of the first items' weights (types whose pieces
        // take a fixed number of load instructions), chosen by the host where
        // x exceeds what the register staging requests ahead (a.x_dma)
        constexpr bool DMA = !NORM && REX_X_DMA && Tr<T>::LOADS > 0 && M == 1;
        constexpr bool UP = UNC || XF || DMA;
        auto prefetch_first = [&] {
            fetch_item<T, NR, SUB, UP>(Wb, a, lg, ls, g1, nwaves, S, li, slot, A);
            if (DEPTH == 2) fetch_item<T, NR, SUB, UP>(Wb, a, lg, ls, g1, nwaves, S, li, slot, B);
        };
        if constexpr (NORM) {
            // at every m, the upper half of the waves request their first
            // items after the normalisation prologue (as the plain product
            // does from REX_LATE_HALF_MIN_M input rows on): the prologue's x
            // and r loads then wait behind half of the weights (fused Q8_0
            // 4096 x 4096: m = 1..4 -4 to -8%, m = 5..8 -2 to -4%)
            const bool late = nwaves >= 2 && wave >= (nwaves >> 1);
            if (!late) prefetch_first();
            norm_partials<T, M, true>(part, xs, XS, xb, a.r + b * a.xbs, a.g,
                                      (a.h && w == 0) ? a.h + b * a.xbs : nullptr, a.xrs, a.k, wave, nwaves, lane);
            __syncthreads();
            if (late) prefetch_first();
        } else if (DMA && a.x_dma) {
            stage_x_dma<T, M>(xs, xb, a.xrs, a.k, XS, wave, nwaves, lane);
            __builtin_amdgcn_sched_barrier(0);
            prefetch_first();
            __builtin_amdgcn_sched_barrier(0);
            barrier_after_loads<DEPTH * NR * (DMA ? Tr<T>::LOADS : 0)>();
        } else if constexpr (XF) {
            // x is a few loads per thread, requested ahead of the weights, so
            // the barrier does not wait for every wave's weights
            stage_x_first<T, M>(xs, xb, a.xrs, a.k, XS, prefetch_first);
            __syncthreads();
        } else {
            // From REX_LATE_HALF_MIN_M input rows on, the upper half of the
            // workgroup's waves request their first items only after the
            // staging barrier: the lower half's weights then arrive sooner
            // and their multiply overlaps the later loads (Q8_0 4096 x 4096
            // at m = 6 / 8: -4.9% / -3.6%, BF16 -2.5% / -1.6%, Q4_K and
            // Q6_K unchanged; mixed at m = 4).
            const bool late = M >= REX_LATE_HALF_MIN_M && nwaves >= 2 && wave >= (nwaves >> 1);
            if (!late) prefetch_first();
            stage_x<T, M>(xs, xb, a.xrs, 0, a.k, XS);
            __syncthreads();
            if (late) prefetch_first();
        }

        if constexpr (kOffsets<T>) {
            stage_sx<T, M>(xs, XS, (float *)((uint8_t *)xs + a.sx_offset), a.sx_stride, a.k);
            __syncthreads();
        }
        if (gfirst < g1) {
            constexpr bool U = UNC;
            float acc[NR][M];
            zero<M, NR>(acc);
            uint32_t cg = gfirst, cs = 0;
            if constexpr (DEPTH == 2) {
                while (walk_step<T, M, NR, SUB, U>(a, Wb, yb, xs, XS, lg, ls, cg, cs, nwaves, g1, S, lane, li, slot, sc, A, C, acc) &&
                       walk_step<T, M, NR, SUB, U>(a, Wb, yb, xs, XS, lg, ls, cg, cs, nwaves, g1, S, lane, li, slot, sc, B, A, acc) &&
                       walk_step<T, M, NR, SUB, U>(a, Wb, yb, xs, XS, lg, ls, cg, cs, nwaves, g1, S, lane, li, slot, sc, C, B, acc)) {
                }
            } else {
                while (walk_step<T, M, NR, SUB, U>(a, Wb, yb, xs, XS, lg, ls, cg, cs, nwaves, g1, S, lane, li, slot, sc, A, B, acc) &&
                       walk_step<T, M, NR, SUB, U>(a, Wb, yb, xs, XS, lg, ls, cg, cs, nwaves, g1, S, lane, li, slot, sc, B, A, acc)) {
                }
            }
        }
    } else {
        // Several LDS passes over K, or a K split (64 lanes per row only):
        // every K waves of the workgroup work on one row group per round
        // (wave ws of the K takes the row's wave steps ws, ws + K, ws + 2K,
        // ..., in that order across the passes, so a pass of fewer than K
        // steps leaves some of the K waves without work) and all waves stage
        // each pass together.  With L < 64 lanes per row (no split) a lane
        // takes pieces li, li + L, ... of the row in its slot, in the order
        // of the single pass.
        const uint32_t K = SUB ? 1u : a.k_split;
        const uint32_t lpr = lpr_of<SUB>(a);
        const uint32_t li = lane & ((1u << lpr) - 1), slot = lane >> lpr;
        const uint32_t slots = nwaves / K;               // row groups per round
        const uint32_t gs = wave / K, ws = wave - gs * K;  // group slot, split index
        float *kp = (float *)((uint8_t *)xs + a.kp_offset);
        double *part = (double *)((uint8_t *)xs + a.norm_offset);
        const RowScale sc{NORM ? part : nullptr, a.row_scale ? a.row_scale + (uint64_t)b * a.row_scale_stride : nullptr,
                          a.k, a.eps};
        const float *rb = NORM ? a.r + b * a.xbs : nullptr;
        if constexpr (NORM)  // the pass loop's first barrier orders these writes before any store
            norm_partials<T, M, false>(part, nullptr, XS, xb, rb, a.g, (a.h && w == 0) ? a.h + b * a.xbs : nullptr,
                                       a.xrs, a.k, wave, nwaves, lane);
        for (uint32_t base = g0; base < g1; base += slots) {
            const uint32_t g = base + gs;
            const bool active = g < g1;
            float acc[NR][M];
            zero<M, NR>(acc);
            const uint8_t *R[NR];
            uint32_t o0[NR];
            row_bases<NR>(a.W, Wb, a.row_bytes, a.n, (g * NR) << (6 - lpr), SUB, slot * NR, R, o0);
            for (uint32_t c = 0; c < a.nchunks; ++c) {
                const uint32_t pb = c * a.pieces_per_chunk;
                const uint32_t pe = min(pb + a.pieces_per_chunk, a.pieces);
                const uint32_t vb = pb * Geo<T>::PV;
                const uint32_t ve = min(a.k, vb + a.kchunk);
                __syncthreads();
                if constexpr (NORM)
                    stage_u<T, M>(xs, xb, rb, a.g, a.xrs, vb, ve, XS);
                else
                    stage_x<T, M>(xs, xb, a.xrs, vb, ve, XS);
                __syncthreads();
                if constexpr (kOffsets<T>) {
                    stage_sx<T, M>(xs, XS, (float *)((uint8_t *)xs + a.sx_offset), a.sx_stride, ve - vb);
                    __syncthreads();
                }
                // the wave's first step in this pass: the first of the
                // pass' wave steps s0, s0 + 1, ... with s = ws (mod K)
                const uint32_t s0 = pb >> 6;
                const uint32_t first = s0 + ((ws - s0) & (K - 1));
                if (active)
                    accumulate<T, M, NR>(acc, R, o0, 64 * first, pe, vb, xs, XS, a.k, li,
                                         (const float *)((const uint8_t *)xs + a.sx_offset), a.sx_stride, K << lpr);
            }
            if constexpr (SUB) {
                if (active) store_group<M, NR, true>(a, acc, yb, g, lane, sc);
            } else if (K == 1) {
                if (active) reduce_store<M, NR, 64>(acc, yb, a.yrs, a.n, g * NR, lane, sc);
            } else {
                reduce_store_split<M, NR>(acc, kp, K, wave, ws, active, yb, a.yrs, a.n, g * NR, lane, sc);
            }
        }
        // The walk leaves its last (unused) prefetch in flight; drain it
        // here, where nothing follows, so that the compiler's wait
        // bookkeeping does not carry it into the single-pass code (the two
        // branches share a join block, and a load pending there forces a
        // full wait ahead of the single pass' first weight loads).
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    }
}

// out[r*k + v] = weight v of row r, one thread per (row, piece).
template <int T>
__global__ void __launch_bounds__(256) dq_kernel(const DqArgs a) {
    using TR = Tr<T>;
    const uint64_t gid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (uint64_t)a.rows * a.pieces) return;
    const uint32_t r = (uint32_t)(gid / a.pieces), p = (uint32_t)(gid % a.pieces);
    const uint8_t *R;
    uint32_t o0;
    row_base(a.W, a.W + (uint64_t)r * a.row_bytes, R, o0);
    const typename TR::Raw raw = TR::load(R, o0, p, a.k);
    const typename TR::Pre pre = TR::prep(raw, p);
    float *o = a.out + (uint64_t)r * a.k;
#pragma unroll
    for (int g = 0; g < TR::NG; ++g) {
        if (!TR::group_valid(p, g, a.k)) continue;
        float w[4];
        TR::deq(raw, pre, g, w);
        const uint32_t v = TR::vpos(p, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[v + i] = w[i];
    }
}

// ---------------------------------------------------------------- launchers

// Raises fn's dynamic-LDS limit to lds_max once per process (the first launch
// of an instance that needs more than 64 KB), so that concurrent launches of
// one instance never lower it under each other.
template <int T, int M, int NR, bool SUB, bool NORM, bool UNC>
hipError_t allow_lds(size_t lds, size_t lds_max) {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    if (lds <= 65536) return hipSuccess;
    std::call_once(once, [&] {
        err = hipFuncSetAttribute((const void *)mv_kernel<T, M, NR, SUB, NORM, UNC>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
    });
    return err;
}

template <int T, int M, int NR, bool SUB, bool NORM, bool UNC>
hipError_t launch_instance(const MvArgs &a, dim3 grid, dim3 block, size_t lds, size_t lds_max, hipStream_t s) {
    const hipError_t e = allow_lds<T, M, NR, SUB, NORM, UNC>(lds, lds_max);
    if (e != hipSuccess) return e;
    MvArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)mv_kernel<T, M, NR, SUB, NORM, UNC>, grid, block, args, lds, s);
}

template <int T, int M, int NR>
hipError_t launch_one(const MvArgs &a, dim3 grid, dim3 block, size_t lds, size_t lds_max, hipStream_t s) {
    // Unconditional-load walks (see fetch_item) only for the plain
    // (unnormalised) instances, where waves hold many items on the large
    // shapes.
    if (a.lpr_log2 < 6) {
        if (a.r) return launch_instance<T, M, NR, true, true, false>(a, grid, block, lds, lds_max, s);
        if (a.walk_unconditional) return launch_instance<T, M, NR, true, false, true>(a, grid, block, lds, lds_max, s);
        return launch_instance<T, M, NR, true, false, false>(a, grid, block, lds, lds_max, s);
    }
    if (a.r) return launch_instance<T, M, NR, false, true, false>(a, grid, block, lds, lds_max, s);
    if (a.walk_unconditional) return launch_instance<T, M, NR, false, false, true>(a, grid, block, lds, lds_max, s);
    return launch_instance<T, M, NR, false, false, false>(a, grid, block, lds, lds_max, s);
}

template <int T, int M, int NR>
hipError_t attributes_one(hipFuncAttributes *attr) {
    return hipFuncGetAttributes(attr, (const void *)mv_kernel<T, M, NR, false, false, false>);
}

template <int T, int M>
hipError_t attributes_m(uint32_t nr, hipFuncAttributes *attr) {
    switch (nr) {
    case 1: return attributes_one<T, M, 1>(attr);
    case 2: return attributes_one<T, M, 2>(attr);
    case 4: return attributes_one<T, M, 4>(attr);
    default: return hipErrorInvalidValue;
    }
}

template <int T>
hipError_t attributes_mv(uint32_t m, uint32_t nr, hipFuncAttributes *attr) {
    switch (m) {
    case 1: return attributes_m<T, 1>(nr, attr);
    case 2: return attributes_m<T, 2>(nr, attr);
    case 3: return attributes_m<T, 3>(nr, attr);
    case 4: return attributes_m<T, 4>(nr, attr);
    case 5: return attributes_m<T, 5>(nr, attr);
    case 6: return attributes_m<T, 6>(nr, attr);
    case 7: return attributes_m<T, 7>(nr, attr);
    case 8: return attributes_m<T, 8>(nr, attr);
    default: return hipErrorInvalidValue;
    }
}

template <int T, int M>
hipError_t launch_m(const MvArgs &a, uint32_t nr, dim3 grid, dim3 block, size_t lds, size_t lds_max, hipStream_t s) {
    switch (nr) {
    case 1: return launch_one<T, M, 1>(a, grid, block, lds, lds_max, s);
    case 2: return launch_one<T, M, 2>(a, grid, block, lds, lds_max, s);
    case 4: return launch_one<T, M, 4>(a, grid, block, lds, lds_max, s);
    default: return hipErrorInvalidValue;
    }
}

template <int T>
hipError_t launch_mv(const MvArgs &a, uint32_t m, uint32_t nr, dim3 grid, dim3 block, size_t lds, size_t lds_max,
                     hipStream_t s) {
    switch (m) {
    case 1: return launch_m<T, 1>(a, nr, grid, block, lds, lds_max, s);
    case 2: return launch_m<T, 2>(a, nr, grid, block, lds, lds_max, s);
    case 3: return launch_m<T, 3>(a, nr, grid, block, lds, lds_max, s);
    case 4: return launch_m<T, 4>(a, nr, grid, block, lds, lds_max, s);
    case 5: return launch_m<T, 5>(a, nr, grid, block, lds, lds_max, s);
    case 6: return launch_m<T, 6>(a, nr, grid, block, lds, lds_max, s);
    case 7: return launch_m<T, 7>(a, nr, grid, block, lds, lds_max, s);
    case 8: return launch_m<T, 8>(a, nr, grid, block, lds, lds_max, s);
    default: return hipErrorInvalidValue;
    }
}

template <int T>
hipError_t launch_dq(const DqArgs &a, hipStream_t s) {
    const uint64_t total = (uint64_t)a.rows * a.pieces;
    const dim3 grid((uint32_t)((total + 255) / 256));
    DqArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)dq_kernel<T>, grid, dim3(256), args, 0, s);
}

}  // namespace rex
