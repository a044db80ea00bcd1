// The add + RMS statistics of the fused normalisation as a kernel of its own
// (nuvec-core 0.6.0, src/gpu.rs, add_rms_norm: the sum h = x + r and its RMS
// normalisation with weight g), the first of the two launches of
// row_exact_mv_add_rmsnorm: it writes h, u = h * g and each input row's
// inverse RMS; the plain mat-vec then multiplies u and scales every output
// once by its row's value.
//
// The statistic is summed in float64 in the order the single-kernel form
// uses (norm_partials in re_kernels.h), so both forms give every output the
// same bits: virtual lane v (here thread v of 256) sums the squares of the
// h values of chunks q = v, v + 256, v + 512, ... (four values each, in
// order, by fma); each wave's 64 lanes are added by the xor tree over masks
// 32, 16, ..., 1; the four wave sums as (s0 + s1) + (s2 + s3).
#include "re_kernels.h"

namespace rex {

namespace {

// Chunks of a row a thread has in flight at once.
constexpr int kChunksAhead = 4;

__global__ void __launch_bounds__(256) norm_rows_kernel(const NormArgs a) {
    const uint32_t b = blockIdx.x / a.m, j = blockIdx.x - b * a.m;
    const uint32_t v = threadIdx.x, lane = v & 63u, wave = v >> 6;
    const uint64_t o = (uint64_t)b * a.xbs + (uint64_t)j * a.xrs;
    const float *__restrict__ xr = a.x + o;
    const float *__restrict__ rr = a.r + o;
    float *__restrict__ hr = a.h ? a.h + o : nullptr;
    float *__restrict__ ur = a.u + ((uint64_t)b * a.m + j) * a.k;
    const uint32_t n4 = a.k >> 2;
    double ss = 0.0;
    for (uint32_t q0 = v; q0 < n4; q0 += 256u * kChunksAhead) {
        // x, r and g requested together: one memory round trip per batch
        f32x4 xv[kChunksAhead], rv[kChunksAhead], gv[kChunksAhead];
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) {
                xv[c] = *(const f32x4 *)(xr + 4 * q);
                rv[c] = *(const f32x4 *)(rr + 4 * q);
                if (a.g) gv[c] = *(const f32x4 *)(a.g + 4 * q);
            }
        }
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) {
                f32x4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = xv[c][e] + rv[c][e];
                if (hr) *(f32x4 *)(hr + 4 * q) = h;
                ss = fold4(ss, h);
                f32x4 u = h;
                if (a.g) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] = h[e] * gv[c][e];
                }
                *(f32x4 *)(ur + 4 * q) = u;
            }
        }
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) ss += shfl_xor_d(ss, msk);
    __shared__ double part[4];
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    if (v == 0) a.inv[(uint64_t)b * a.m + j] = RowScale::inv_rms(part, a.k, a.eps);
}

// The workgroup's sum of the 256 virtual lanes' float64 partials: each
// wave's 64 by the xor tree over masks 32, 16, ..., 1, the four wave sums as
// (s0 + s1) + (s2 + s3); every thread gets 1 / sqrt(sum / k + eps).
__device__ __forceinline__ double block_inv_rms(double ss, double *part, uint32_t lane, uint32_t wave, uint32_t k,
                                                float eps) {
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) ss += shfl_xor_d(ss, msk);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    const double inv = RowScale::inv_rms(part, k, eps);
    __syncthreads();  // part is reused
    return inv;
}

// The prologue of the residual RMS normalisation (nuvec-core 0.6.0,
// src/gpu.rs, residual_rms_norm: the residual stream plus the RMS
// normalisation of a layer output, optionally scaled, and that sum's own RMS
// normalisation), 256 threads per (batch entry, input row).  Both statistics
// are summed in float64 in the order of norm_rows_kernel.  Per value:
// t = (float)(x * inv1 * w) in float64, hs = h + t and hs = hs * c in
// float32, u = hs * w2 in float32; the product then scales every output by
// the row's inverse RMS of hs.
__global__ void __launch_bounds__(256) residual_rows_kernel(const ResidualArgs a) {
    const uint32_t b = blockIdx.x / a.m, j = blockIdx.x - b * a.m;
    const uint32_t v = threadIdx.x, lane = v & 63u, wave = v >> 6;
    const uint64_t o = (uint64_t)b * a.xbs + (uint64_t)j * a.xrs;
    const float *__restrict__ xr = a.x + o;
    const float *__restrict__ hr = a.h + o;
    float *__restrict__ ho = a.hout ? a.hout + o : nullptr;
    float *__restrict__ ur = a.u + ((uint64_t)b * a.m + j) * a.k;
    const uint32_t n4 = a.k >> 2;
    __shared__ double part[4];
    // With one batch per thread (k <= 4096) every input is requested once,
    // up front, and the second pass works from registers; otherwise each
    // pass requests its batch's inputs together.
    const bool one_batch = n4 <= 256u * kChunksAhead;
    f32x4 xv[kChunksAhead], hv[kChunksAhead], wv[kChunksAhead], cv[kChunksAhead], w2v[kChunksAhead];
    auto load_rest = [&](uint32_t q0) {
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) {
                hv[c] = *(const f32x4 *)(hr + 4 * q);
                wv[c] = a.w ? *(const f32x4 *)(a.w + 4 * q) : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
                if (a.c) cv[c] = *(const f32x4 *)(a.c + 4 * q);
                if (a.w2) w2v[c] = *(const f32x4 *)(a.w2 + 4 * q);
            }
        }
    };
    auto load_x = [&](uint32_t q0) {
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) xv[c] = *(const f32x4 *)(xr + 4 * q);
        }
    };
    double s1 = 0.0;
    for (uint32_t q0 = v; q0 < n4; q0 += 256u * kChunksAhead) {
        load_x(q0);
        if (one_batch) load_rest(q0);
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c)
            if (q0 + 256u * c < n4) s1 = fold4(s1, xv[c]);
    }
    const double inv1 = block_inv_rms(s1, part, lane, wave, a.k, a.eps);
    double s2 = 0.0;
    for (uint32_t q0 = v; q0 < n4; q0 += 256u * kChunksAhead) {
        if (!one_batch) {
            load_x(q0);
            load_rest(q0);
        }
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) {
                f32x4 hs;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = (float)((double)xv[c][e] * inv1 * (double)wv[c][e]);
                    hs[e] = hv[c][e] + t;
                }
                if (a.c) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) hs[e] = hs[e] * cv[c][e];
                }
                if (ho) *(f32x4 *)(ho + 4 * q) = hs;
                s2 = fold4(s2, hs);
                f32x4 u = hs;
                if (a.w2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] = hs[e] * w2v[c][e];
                }
                *(f32x4 *)(ur + 4 * q) = u;
            }
        }
    }
    const double inv2 = block_inv_rms(s2, part, lane, wave, a.k, a.eps2);
    if (v == 0) a.inv[(uint64_t)b * a.m + j] = inv2;
}

}  // namespace

hipError_t launch_residual_rows(const ResidualArgs &a, uint32_t batch, hipStream_t s) {
    ResidualArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)residual_rows_kernel, dim3(batch * a.m), dim3(256), args, 0, s);
}

hipError_t launch_norm_rows(const NormArgs &a, uint32_t batch, hipStream_t s) {
    NormArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)norm_rows_kernel, dim3(batch * a.m), dim3(256), args, 0, s);
}

}  // namespace rex
