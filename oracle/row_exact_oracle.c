/*
 * Oracle for the row-exact few-row mat-vec  y[b][j][i] = sum_kk Wd[b*n+i][kk] * x[b][j][kk].
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct CPU code.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or constant with the HIP library, and
 * neither includes the other.
 *
 * What it follows (mlx-native 0.18.0, src/ops/row_exact_matvec.rs):
 *   - module docs: y[j,:] = W . x[j,:], F16 / Q8_0 / Q4_K / Q6_K / Q5_0 weights,
 *     F32 input and output, 1 <= m <= 8 rows;
 *   - "Batched / grouped products": batch b reads weight rows at
 *     b * n * row_bytes, input at b * x_batch_stride, output at
 *     b * y_batch_stride;
 *   - the block constants (32 values / 34 bytes, 256 / 144, 256 / 210,
 *     32 / 22) and RowExactWeight::row_bytes.
 * Dense float32 and bfloat16 weights follow the same product (nuvec-core
 * 0.6.0, src/gpu.rs: the matmul's "a few rows" route to gemv_rows and its
 * row-independence contract); their values are decoded from the IEEE fields.
 *
 * The pages give block byte sizes only.  The bit layout inside each block is
 * the plain reading of the GGML types the enum is named after; every value is
 * decoded on its own, from its index, straight from that layout.
 *
 * Weights are decoded to their exact float32 value (every product of block
 * fields is exact in float32 except Q4_K's final difference, which is rounded
 * once, to nearest even).  Products Wd * x are exact in float64 and summed in
 * float64 in index order; the sum of their absolute values is returned too.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_Q8_0 = 1, OR_Q4_K = 2, OR_Q6_K = 3, OR_Q5_0 = 4, OR_F32 = 5, OR_BF16 = 6 };

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static uint32_t rd_u32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* IEEE 754 binary16 -> float, from the definition: sign, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 is zero/subnormal (f * 2^-24),
 * exponent 31 is infinity/NaN. */
float oracle_f16_to_f32(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return (float)(sign ? -v : v);
}

/* bfloat16 -> float, from the definition: sign, 8-bit exponent (bias 127),
 * 7-bit fraction; exponent 0 is zero/subnormal (f * 2^-133), exponent 255 is
 * infinity/NaN. */
float oracle_bf16_to_f32(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 7) & 255;
    int f = h & 127;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);
    }
    return (float)(sign ? -v : v);
}

/* IEEE 754 binary32 bit pattern -> float, from the definition: sign, 8-bit
 * exponent (bias 127), 23-bit fraction; exponent 0 is zero/subnormal
 * (f * 2^-149), exponent 255 is infinity/NaN. */
float oracle_f32_from_bits(uint32_t u) {
    int sign = (int)(u >> 31);
    int e = (int)((u >> 23) & 255u);
    uint32_t f = u & 0x7FFFFFu;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -149);
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(0x800000u + f), e - 150);
    }
    return (float)(sign ? -v : v);
}

/* Bytes per row of k values (RowExactWeight::row_bytes). */
uint64_t oracle_row_bytes(int type, uint32_t k) {
    switch (type) {
    case OR_F16: return (uint64_t)k * 2;
    case OR_Q8_0: return (uint64_t)(k / 32) * 34;
    case OR_Q4_K: return (uint64_t)(k / 256) * 144;
    case OR_Q6_K: return (uint64_t)(k / 256) * 210;
    case OR_Q5_0: return (uint64_t)(k / 32) * 22;
    case OR_F32: return (uint64_t)k * 4;
    case OR_BF16: return (uint64_t)k * 2;
    default: return 0;
    }
}

/* Q8_0 block (34 bytes): d f16 at 0, 32 int8 quants at 2.  w = d * q. */
static float value_q8_0(const uint8_t *row, uint32_t v) {
    const uint8_t *blk = row + 34 * (size_t)(v / 32);
    float d = oracle_f16_to_f32(rd_u16(blk));
    int8_t q = (int8_t)blk[2 + v % 32];
    return d * (float)q;
}

/* Q5_0 block (22 bytes): d f16 at 0, 32 high bits (u32) at 2, 16 bytes of
 * nibbles at 6.  Value i < 16 takes the low nibble of byte i, value i >= 16
 * the high nibble of byte i - 16; bit i of the high bits is bit 4 of the
 * 5-bit quant.  w = d * (q - 16). */
static float value_q5_0(const uint8_t *row, uint32_t v) {
    const uint8_t *blk = row + 22 * (size_t)(v / 32);
    uint32_t i = v % 32;
    float d = oracle_f16_to_f32(rd_u16(blk));
    uint32_t qh = rd_u32(blk + 2);
    uint32_t lo = i < 16 ? (blk[6 + i] & 15u) : (blk[6 + i - 16] >> 4);
    uint32_t hb = (qh >> i) & 1u;
    int q = (int)(lo | (hb << 4));
    return d * (float)(q - 16);
}

/* Q4_K super-block (144 bytes): d f16 at 0, dmin f16 at 2, 12 bytes of packed
 * 6-bit scales and mins at 4, 128 bytes of nibbles at 16.  Sub-block s (32
 * values) has scale sc_s and min mn_s:
 *   s < 4 : sc = S[s] & 63,                      mn = S[s+4] & 63
 *   s >= 4: sc = (S[s+4] & 15) | (S[s-4] >> 6) << 4,
 *           mn = (S[s+4] >> 4) | (S[s] >> 6) << 4
 * Value v: chunk c = v / 64 uses bytes 32c..32c+31; t = v % 64 takes the low
 * nibble of byte 32c + t for t < 32 and the high nibble of byte 32c + t - 32
 * otherwise.  w = (d * sc) * q - dmin * mn, one rounding. */
static float value_q4_k(const uint8_t *row, uint32_t v) {
    const uint8_t *blk = row + 144 * (size_t)(v / 256);
    uint32_t i = v % 256;
    double d = oracle_f16_to_f32(rd_u16(blk));
    double dmin = oracle_f16_to_f32(rd_u16(blk + 2));
    const uint8_t *S = blk + 4;
    const uint8_t *qs = blk + 16;
    uint32_t s = i / 32;
    uint32_t sc, mn;
    if (s < 4) {
        sc = S[s] & 63u;
        mn = S[s + 4] & 63u;
    } else {
        sc = (S[s + 4] & 15u) | ((uint32_t)(S[s - 4] >> 6) << 4);
        mn = (uint32_t)(S[s + 4] >> 4) | ((uint32_t)(S[s] >> 6) << 4);
    }
    uint32_t c = i / 64, t = i % 64;
    uint32_t byte = qs[32 * c + t % 32];
    uint32_t q = t < 32 ? (byte & 15u) : (byte >> 4);
    /* Both products and their difference are exact in double. */
    return (float)(d * (double)sc * (double)q - dmin * (double)mn);
}

/* Q6_K super-block (210 bytes): 128 bytes of low nibbles at 0, 64 bytes of
 * 2-bit high parts at 128, 16 int8 scales at 192, d f16 at 208.  Value v:
 * h = v / 128, r = v % 128, t = r / 32, l = r % 32; the low 4 bits are the
 * low (t < 2) or high (t >= 2) nibble of ql[64h + l + 32 (t & 1)], the high
 * 2 bits are bits 2t..2t+1 of qh[32h + l]; the scale is sc[v / 16].
 * w = d * sc * (q - 32). */
static float value_q6_k(const uint8_t *row, uint32_t v) {
    const uint8_t *blk = row + 210 * (size_t)(v / 256);
    uint32_t i = v % 256;
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    float d = oracle_f16_to_f32(rd_u16(blk + 208));
    uint32_t h = i / 128, r = i % 128, t = r / 32, l = r % 32;
    uint32_t lob = ql[64 * h + l + 32 * (t & 1)];
    uint32_t lo = t < 2 ? (lob & 15u) : (lob >> 4);
    uint32_t hi = (qh[32 * h + l] >> (2 * t)) & 3u;
    int q = (int)(lo | (hi << 4));
    return d * (float)sc[i / 16] * (float)(q - 32);
}

static float value_f16(const uint8_t *row, uint32_t v) { return oracle_f16_to_f32(rd_u16(row + 2 * (size_t)v)); }

static float value_f32(const uint8_t *row, uint32_t v) { return oracle_f32_from_bits(rd_u32(row + 4 * (size_t)v)); }

static float value_bf16(const uint8_t *row, uint32_t v) { return oracle_bf16_to_f32(rd_u16(row + 2 * (size_t)v)); }

/* Exact float32 value of weight v of one row. */
float oracle_weight(int type, const uint8_t *row, uint32_t v) {
    switch (type) {
    case OR_F16: return value_f16(row, v);
    case OR_Q8_0: return value_q8_0(row, v);
    case OR_Q4_K: return value_q4_k(row, v);
    case OR_Q6_K: return value_q6_k(row, v);
    case OR_Q5_0: return value_q5_0(row, v);
    case OR_F32: return value_f32(row, v);
    case OR_BF16: return value_bf16(row, v);
    default: return NAN;
    }
}

static int k_ok(int type, uint32_t k) {
    switch (type) {
    case OR_F16: case OR_F32: case OR_BF16: return k % 4 == 0;
    case OR_Q8_0: case OR_Q5_0: return k % 32 == 0;
    case OR_Q4_K: case OR_Q6_K: return k % 256 == 0;
    default: return 0;
    }
}

/* out[r * k + v] = exact value of weight v of row r, for rows consecutive
 * rows of k values starting at W.  Returns 0, or -1 on a bad type or k. */
int oracle_dequant(int type, const uint8_t *W, uint32_t rows, uint32_t k, float *out) {
    if (!k_ok(type, k)) return -1;
    uint64_t rb = oracle_row_bytes(type, k);
    for (uint32_t r = 0; r < rows; ++r) {
        const uint8_t *row = W + rb * r;
        for (uint32_t v = 0; v < k; ++v) out[(size_t)r * k + v] = oracle_weight(type, row, v);
    }
    return 0;
}

/* Reference product.  For every batch b < batch, row j < m, output i < n:
 *   y[(b*m + j)*n + i] = sum_kk Wd[b*n + i][kk] * x[b*xbs + j*xrs + kk]
 *   a[(b*m + j)*n + i] = sum_kk |Wd[b*n + i][kk] * x[b*xbs + j*xrs + kk]|
 * in float64, kk in increasing order.  Weight row b*n + i starts at byte
 * (b*n + i) * row_bytes (batch b at b * n * row_bytes).  Outputs are dense
 * [batch][m][n] whatever the device output strides are.  Rows i in
 * [i0, i1) only (pass 0, n for all); other outputs are left untouched. */
int oracle_matvec_rows(int type, const uint8_t *W, const float *x, uint32_t n, uint32_t k, uint32_t m,
                       uint32_t batch, uint32_t xrs, uint32_t xbs, uint32_t i0, uint32_t i1, double *y,
                       double *a) {
    if (!k_ok(type, k) || m == 0 || n == 0 || batch == 0) return -1;
    uint64_t rb = oracle_row_bytes(type, k);
    float *wd = (float *)malloc(sizeof(float) * k);
    if (!wd) return -2;
    for (uint32_t b = 0; b < batch; ++b) {
        for (uint32_t i = i0; i < i1 && i < n; ++i) {
            const uint8_t *row = W + rb * ((uint64_t)b * n + i);
            for (uint32_t v = 0; v < k; ++v) wd[v] = oracle_weight(type, row, v);
            for (uint32_t j = 0; j < m; ++j) {
                const float *xr = x + (uint64_t)b * xbs + (uint64_t)j * xrs;
                double s = 0.0, sa = 0.0;
                for (uint32_t v = 0; v < k; ++v) {
                    double p = (double)wd[v] * (double)xr[v];
                    s += p;
                    sa += fabs(p);
                }
                size_t o = ((size_t)b * m + j) * n + i;
                y[o] = s;
                a[o] = sa;
            }
        }
    }
    free(wd);
    return 0;
}

int oracle_matvec(int type, const uint8_t *W, const float *x, uint32_t n, uint32_t k, uint32_t m,
                  uint32_t batch, uint32_t xrs, uint32_t xbs, double *y, double *a) {
    return oracle_matvec_rows(type, W, x, n, k, m, batch, xrs, xbs, 0, n, y, a);
}

/* Gathered product (per-expert weight selection: nuvec-core 0.6.0,
 * src/gpu.rs, GatherQmm / GatherMm).  As oracle_matvec_rows, except that
 * batch entry b takes its weight rows from set ids[b] of num_experts sets
 * (set e at byte e * n * row_bytes); an id outside [0, num_experts) gives NaN
 * for all of that entry's outputs (and its absolute sums). */
int oracle_matvec_gather(int type, const uint8_t *W, uint32_t num_experts, const int32_t *ids, const float *x,
                         uint32_t n, uint32_t k, uint32_t m, uint32_t batch, uint32_t xrs, uint32_t xbs,
                         double *y, double *a) {
    if (!k_ok(type, k) || m == 0 || n == 0 || batch == 0 || num_experts == 0) return -1;
    uint64_t rb = oracle_row_bytes(type, k);
    for (uint32_t b = 0; b < batch; ++b) {
        size_t o = (size_t)b * m * n;
        if (ids[b] < 0 || (uint32_t)ids[b] >= num_experts) {
            for (size_t q = 0; q < (size_t)m * n; ++q) {
                y[o + q] = NAN;
                a[o + q] = NAN;
            }
            continue;
        }
        const uint8_t *We = W + rb * (uint64_t)n * (uint32_t)ids[b];
        int rc = oracle_matvec_rows(type, We, x + (uint64_t)b * xbs, n, k, m, 1, xrs, 0, 0, n, y + o, a + o);
        if (rc) return rc;
    }
    return 0;
}

/* The product with a residual RMS normalisation producing its input
 * (nuvec-core 0.6.0, src/gpu.rs, residual_rms_norm: the residual stream plus
 * the RMS normalisation of a layer output, optionally scaled, then that sum's
 * own RMS normalisation for the next projection).  For every batch b and
 * input row j, over the k values v of the row (h, x and hout share the
 * layout b*xbs + j*xrs + v):
 *   s1      = sum_v x[v]^2                                  (float64, v in order)
 *   t[v]    = x[v] / sqrt(s1 / k + eps) * w[v]              (float64, rounded once to float32; w NULL: 1)
 *   hs[v]   = h[v] + t[v]                                   (float32 addition)
 *   hs[v]   = hs[v] * c[v]                                  (float32 multiplication; c NULL: skipped)
 *   s2      = sum_v hs[v]^2                                 (float64, v in order)
 *   xn[v]   = hs[v] / sqrt(s2 / k + eps2) * w2[v]           (float64; w2 NULL: 1)
 *   y[(b*m + j)*n + i] = sum_v Wd[b*n + i][v] * xn[v]       (float64)
 *   a[...]             = sum_v |Wd[b*n + i][v] * xn[v]|
 * hout (= hs) is written in x's layout, xn dense [batch][m][k]. */
int oracle_mv_residual_rmsnorm(int type, const uint8_t *W, const float *h, const float *x, const float *w,
                               const float *c, const float *w2, float eps, float eps2, uint32_t n, uint32_t k,
                               uint32_t m, uint32_t batch, uint32_t xrs, uint32_t xbs, float *hout, double *xn,
                               double *y, double *a) {
    if (!k_ok(type, k) || m == 0 || n == 0 || batch == 0) return -1;
    uint64_t rb = oracle_row_bytes(type, k);
    float *wd = (float *)malloc(sizeof(float) * k);
    if (!wd) return -2;
    for (uint32_t b = 0; b < batch; ++b) {
        for (uint32_t j = 0; j < m; ++j) {
            size_t off = (size_t)b * xbs + (size_t)j * xrs;
            double *xr = xn + ((size_t)b * m + j) * k;
            double s1 = 0.0;
            for (uint32_t v = 0; v < k; ++v) s1 += (double)x[off + v] * (double)x[off + v];
            double rms1 = sqrt(s1 / (double)k + (double)eps);
            double s2 = 0.0;
            for (uint32_t v = 0; v < k; ++v) {
                float t = (float)((double)x[off + v] / rms1 * (w ? (double)w[v] : 1.0));
                float hs = h[off + v] + t;
                if (c) hs = hs * c[v];
                hout[off + v] = hs;
                s2 += (double)hs * (double)hs;
            }
            double rms2 = sqrt(s2 / (double)k + (double)eps2);
            for (uint32_t v = 0; v < k; ++v) xr[v] = (double)hout[off + v] / rms2 * (w2 ? (double)w2[v] : 1.0);
        }
        for (uint32_t i = 0; i < n; ++i) {
            const uint8_t *row = W + rb * ((uint64_t)b * n + i);
            for (uint32_t v = 0; v < k; ++v) wd[v] = oracle_weight(type, row, v);
            for (uint32_t j = 0; j < m; ++j) {
                const double *xr = xn + ((size_t)b * m + j) * k;
                double sy = 0.0, sa = 0.0;
                for (uint32_t v = 0; v < k; ++v) {
                    double p = (double)wd[v] * xr[v];
                    sy += p;
                    sa += fabs(p);
                }
                y[((size_t)b * m + j) * n + i] = sy;
                a[((size_t)b * m + j) * n + i] = sa;
            }
        }
    }
    free(wd);
    return 0;
}

/* The product with a fused add + RMS normalisation of its input (nuvec-core
 * 0.6.0, src/gpu.rs, add_rms_norm: the sum x + r and its RMS normalisation
 * with weight g).  For every batch b and input row j, over the k values v of
 * the row (x, r and h share the layout b*xbs + j*xrs + v):
 *   h[v]  = x[v] + r[v]                                  (float32 addition)
 *   s     = sum_v h[v]^2                                 (float64, v in order)
 *   xn[v] = h[v] / sqrt(s / k + eps) * g[v]              (float64; g NULL: 1)
 *   y[(b*m + j)*n + i] = sum_v Wd[b*n + i][v] * xn[v]    (float64)
 *   a[...]             = sum_v |Wd[b*n + i][v] * xn[v]|
 * h is written in x's layout, xn dense [batch][m][k]. */
int oracle_mv_add_rmsnorm(int type, const uint8_t *W, const float *x, const float *r, const float *g, float eps,
                          uint32_t n, uint32_t k, uint32_t m, uint32_t batch, uint32_t xrs, uint32_t xbs,
                          float *h, double *xn, double *y, double *a) {
    if (!k_ok(type, k) || m == 0 || n == 0 || batch == 0) return -1;
    uint64_t rb = oracle_row_bytes(type, k);
    float *wd = (float *)malloc(sizeof(float) * k);
    if (!wd) return -2;
    for (uint32_t b = 0; b < batch; ++b) {
        for (uint32_t j = 0; j < m; ++j) {
            size_t off = (size_t)b * xbs + (size_t)j * xrs;
            double *xr = xn + ((size_t)b * m + j) * k;
            double s = 0.0;
            for (uint32_t v = 0; v < k; ++v) {
                float hv = x[off + v] + r[off + v];
                h[off + v] = hv;
                s += (double)hv * (double)hv;
            }
            double rms = sqrt(s / (double)k + (double)eps);
            for (uint32_t v = 0; v < k; ++v) xr[v] = (double)h[off + v] / rms * (g ? (double)g[v] : 1.0);
        }
        for (uint32_t i = 0; i < n; ++i) {
            const uint8_t *row = W + rb * ((uint64_t)b * n + i);
            for (uint32_t v = 0; v < k; ++v) wd[v] = oracle_weight(type, row, v);
            for (uint32_t j = 0; j < m; ++j) {
                const double *xr = xn + ((size_t)b * m + j) * k;
                double sy = 0.0, sa = 0.0;
                for (uint32_t v = 0; v < k; ++v) {
                    double p = (double)wd[v] * xr[v];
                    sy += p;
                    sa += fabs(p);
                }
                y[((size_t)b * m + j) * n + i] = sy;
                a[((size_t)b * m + j) * n + i] = sa;
            }
        }
    }
    free(wd);
    return 0;
}
