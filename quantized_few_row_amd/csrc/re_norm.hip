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
        f32x4 xv[kChunksAhead], rv[kChunksAhead];
#pragma unroll
        for (int c = 0; c < kChunksAhead; ++c) {
            const uint32_t q = q0 + 256u * c;
            if (q < n4) {
                xv[c] = *(const f32x4 *)(xr + 4 * q);
                rv[c] = *(const f32x4 *)(rr + 4 * q);
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
                *(f32x4 *)(ur + 4 * q) = times_g(h, a.g, 4 * q);
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

}  // namespace

hipError_t launch_norm_rows(const NormArgs &a, uint32_t batch, hipStream_t s) {
    NormArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)norm_rows_kernel, dim3(batch * a.m), dim3(256), args, 0, s);
}

}  // namespace rex
