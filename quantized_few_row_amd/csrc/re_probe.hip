// Plain streaming read of a device buffer: the attainable HBM read rate for a
// given size, used by the benchmark as the ceiling a weight-streaming kernel
// can approach.  Each wave reads whole KiB rows of 16-byte chunks (lane L
// takes chunk L), UNROLL of them in flight per lane, grid-stride over the
// buffer; a tail shorter than a KiB is read by the lanes that cover it.
#include <cstdio>

#include "re_internal.h"
#include "row_exact_mv.h"
#include "row_exact_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ p, uint64_t nchunks,
                                                           uint32_t *sink) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t nkib = nchunks >> 6;  // whole KiB rows
    const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x >> 6);
    uint32_t acc = 0;
    uint64_t r = wave;
    for (; r + (UNROLL - 1) * nw < nkib; r += UNROLL * nw) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = p[(r + u * nw) * 64 + lane];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
    }
    for (; r < nkib; r += nw) {
        const u32x4 v = p[r * 64 + lane];
        acc ^= v.x + v.y + v.z + v.w;
    }
    if (wave == 0 && (nkib << 6) + lane < nchunks) {
        const u32x4 v = p[(nkib << 6) + lane];
        acc ^= v.x + v.y + v.z + v.w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

struct Shape {
    uint32_t workgroups;
    int unroll;
};
constexpr Shape kShapes[] = {{1024, 2}, {2048, 4}, {1024, 4}, {2048, 8}, {4096, 4}, {8192, 2}};

}  // namespace

extern "C" uint32_t row_exact_stream_read_shapes(void) { return sizeof kShapes / sizeof kShapes[0]; }

extern "C" int row_exact_stream_read(const void *p, uint64_t bytes, uint32_t *sink, uint32_t shape,
                                     hipStream_t stream) {
    using namespace rex;
    if (!p || !sink) return report_error(ROW_EXACT_EARG, "stream_read: NULL pointer");
    if (bytes < 16 || bytes % 16) return report_error(ROW_EXACT_EARG, "stream_read: bytes must be a positive multiple of 16");
    if (shape >= row_exact_stream_read_shapes()) return report_error(ROW_EXACT_EARG, "stream_read: unknown shape");
    if ((uintptr_t)p % 16) return report_error(ROW_EXACT_EALIGN, "stream_read: buffer must be 16-byte aligned");
    if ((uintptr_t)sink % 4) return report_error(ROW_EXACT_EALIGN, "stream_read: sink must be 4-byte aligned");
    const Shape s = kShapes[shape];
    const uint64_t nchunks = bytes / 16;
    const dim3 grid(s.workgroups), block(256);
    const u32x4 *q = (const u32x4 *)p;
    switch (s.unroll) {
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, stream, q, nchunks, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, stream, q, nchunks, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, stream, q, nchunks, sink); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        char msg[256];
        snprintf(msg, sizeof msg, "stream_read: launch failed: %s", hipGetErrorString(e));
        return report_error(ROW_EXACT_EHIP, msg);
    }
    count_launch();
    return 0;
}
