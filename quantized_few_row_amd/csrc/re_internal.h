// Host/device shared definitions of the row-exact mat-vec library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rex {

enum WeightType : int { kF16 = 0, kQ8_0 = 1, kQ4K = 2, kQ6K = 3, kQ5_0 = 4, kF32 = 5, kBF16 = 6 };
constexpr int kNumTypes = 7;

// Kernel argument block (passed by value).
struct MvArgs {
    const uint8_t *W;
    const float *x;
    float *y;
    uint64_t row_bytes;    // bytes per weight row
    uint64_t batch_bytes;  // n * row_bytes
    uint64_t xbs, ybs;     // batch strides (elements)
    uint32_t n, k;
    uint32_t xrs, yrs;     // row strides (elements)
    uint32_t pieces;            // per-lane work items per weight row
    uint32_t groups_per_batch;  // ceil(n / rows_per_wave)
    uint32_t groups_per_wg;     // row groups one workgroup handles
    uint32_t nchunks;           // LDS passes over K
    uint32_t pieces_per_chunk;  // multiple of 64 (one wave step)
    uint32_t kchunk;            // values per pass
    uint32_t xs_stride;         // floats per staged x row in LDS (padded)
    uint32_t lpr_log2;          // log2 of the lanes per weight row (6, or 5 / 4 for short rows)
    const int32_t *ids;         // per-batch weight selection (NULL: batch b uses weights b)
    uint32_t num_experts;       // number of weight sets ids may select
    // Fused add + RMS normalisation of the input (r != NULL): the product
    // uses x' = (x + r) / sqrt(mean((x + r)^2) + eps) * g per input row; the
    // sum x + r goes to h (if not NULL) from the first workgroup of a batch.
    const float *r;
    const float *g;             // k weights, or NULL for none
    float *h;
    float eps;
    uint32_t norm_offset;       // byte offset in LDS of the m per-row inverse RMS values (double)
    uint32_t walk_unconditional;  // 1: waves hold more items than the load depth (see fetch_item)
    uint32_t batch;               // batch entries (grid = workgroups per entry x batch)
    // Types whose weights carry a per-segment offset (Q4_K: - dmin * mn):
    // the sums of the staged input over each 32-value segment, per input
    // row, at byte offset sx_offset in LDS, sx_stride floats per row.
    uint32_t sx_offset;
    uint32_t sx_stride;
    // 1: stage x with loads that write LDS directly, all of it ahead of the
    // weights (single pass, m = 1, x larger than the register staging
    // requests ahead of them)
    uint32_t x_dma;
    // Each output (b, j, i) scaled by row_scale[b * row_scale_stride + j]
    // (float64, one rounding), or NULL: the product of the two-launch fused
    // add + RMS norm runs on u = (x + r) * g with the rows' inverse RMS here.
    const double *row_scale;
    uint32_t row_scale_stride;
    // Waves whose partial sums form one output (1, 2, 4 or 8; numerics: the
    // row's wave steps are dealt round-robin over them and their sums added
    // in a fixed order), and the LDS byte offset of their partials (32
    // floats per wave) when > 1.
    uint32_t k_split;
    uint32_t kp_offset;
};

// The add + RMS statistics of the fused normalisation (norm_rows_kernel):
// one workgroup of 256 threads per (batch entry, input row).
struct NormArgs {
    const float *x, *r, *g;  // x and r in the product's x layout; g: k weights or NULL
    float *h;                // x + r in the same layout, or NULL
    float *u;                // (x + r) * g, contiguous [batch][m][k]
    double *inv;             // inverse RMS per (batch entry, input row), [batch][m]
    uint64_t xbs;
    uint32_t xrs, k, m;
    float eps;
};
hipError_t launch_norm_rows(const NormArgs &a, uint32_t batch, hipStream_t s);

// The residual RMS normalisation's prologue kernel: per (batch entry, input
// row), hs = (h + rms_norm(x) * w) * c written to hout (or NULL), u = hs * w2
// and the inverse RMS of hs (with eps2).
struct ResidualArgs {
    const float *h, *x;           // the product's x layout
    const float *w, *c, *w2;      // k values each, or NULL (1, no scaling, 1)
    float *hout;                  // hs in the same layout, or NULL
    float *u;                     // contiguous [batch][m][k]
    double *inv;                  // [batch][m]
    uint64_t xbs;
    uint32_t xrs, k, m;
    float eps, eps2;
};
hipError_t launch_residual_rows(const ResidualArgs &a, uint32_t batch, hipStream_t s);

struct DqArgs {
    const uint8_t *W;
    float *out;
    uint64_t row_bytes;
    uint32_t rows, k, pieces;
};

// Per-type static geometry, shared by host (schedule) and device (kernels).
template <int T> struct Geo;
// Pad period of the dense types' staged x: 64 values, so that sixteen
// consecutive pieces of 4 or 8 values start on sixteen distinct 4-bank groups
// of the 64 LDS banks (with 32, six of sixteen F16 / BF16 lanes share a
// group; measured the same speed either way on MI355X, ±1%).
constexpr int kDensePadp = 64;
template <> struct Geo<kF16> {   // piece: 8 consecutive halves (16 bytes)
    static constexpr int PV = 8, NG = 2, PADP = kDensePadp;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return (k + 7) / 8; }
};
template <> struct Geo<kQ8_0> {  // piece: one 34-byte block
    static constexpr int PV = 32, NG = 8, PADP = 32;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return k / 32; }
};
template <> struct Geo<kQ4K> {   // piece: one 32-byte nibble chunk of a super-block (64 values)
    static constexpr int PV = 64, NG = 16, PADP = 64;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return k / 256 * 4; }
};
template <> struct Geo<kQ6K> {   // piece: a quarter super-block (64 values)
    static constexpr int PV = 64, NG = 16, PADP = 128;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return k / 256 * 4; }
};
template <> struct Geo<kQ5_0> {  // piece: one 22-byte block
    static constexpr int PV = 32, NG = 8, PADP = 32;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return k / 32; }
};
template <> struct Geo<kF32> {   // piece: 4 consecutive floats (16 bytes)
    static constexpr int PV = 4, NG = 1, PADP = kDensePadp;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return k / 4; }
};
template <> struct Geo<kBF16> {  // piece: 8 consecutive bfloat16 (16 bytes)
    static constexpr int PV = 8, NG = 2, PADP = kDensePadp;
    __host__ __device__ static constexpr uint32_t pieces(uint32_t k) { return (k + 7) / 8; }
};

// Values covered by one wave step (64 pieces).
inline uint32_t wave_step_values(int t) {
    switch (t) {
    case kF16: return 64 * Geo<kF16>::PV;
    case kQ8_0: return 64 * Geo<kQ8_0>::PV;
    case kQ4K: return 64 * Geo<kQ4K>::PV;
    case kQ6K: return 64 * Geo<kQ6K>::PV;
    case kF32: return 64 * Geo<kF32>::PV;
    case kBF16: return 64 * Geo<kBF16>::PV;
    default: return 64 * Geo<kQ5_0>::PV;
    }
}
inline uint32_t pieces_of(int t, uint32_t k) {
    switch (t) {
    case kF16: return Geo<kF16>::pieces(k);
    case kQ8_0: return Geo<kQ8_0>::pieces(k);
    case kQ4K: return Geo<kQ4K>::pieces(k);
    case kQ6K: return Geo<kQ6K>::pieces(k);
    case kF32: return Geo<kF32>::pieces(k);
    case kBF16: return Geo<kBF16>::pieces(k);
    default: return Geo<kQ5_0>::pieces(k);
    }
}
// Lanes that split one weight row, a function of (type, k) only: 64, or 32 /
// 16 when a row has at most 32 / 16 pieces (a wave then covers 2 / 4 rows at
// once instead of leaving lanes idle).
inline uint32_t lanes_per_row_log2(int t, uint32_t k) {
    const uint32_t p = pieces_of(t, k);
    return p <= 16 ? 4u : p <= 32 ? 5u : 6u;
}
// 1: from m = 2 on, Q6_K's staged x is piece-major (each piece's 64 values
// contiguous in the piece's value order, 4 pad floats after each piece: 68
// floats per piece, the density of a 64-value pad period), so that the
// lanes' reads of one group of sixteen consecutive pieces hit distinct LDS
// banks; at m = 1 it keeps the value order, whose LDS-DMA staging reads x
// contiguously.  A staging layout only: the bits do not depend on it.
#ifndef REX_Q6K_PIECE_MAJOR
#define REX_Q6K_PIECE_MAJOR 1
#endif
__host__ __device__ constexpr bool piece_major(int t, uint32_t m) { return REX_Q6K_PIECE_MAJOR && t == kQ6K && m >= 2; }

inline uint32_t pad_period(int t) {
    switch (t) {
    case kF16: return Geo<kF16>::PADP;
    case kQ8_0: return Geo<kQ8_0>::PADP;
    case kQ4K: return Geo<kQ4K>::PADP;
    case kQ6K: return Geo<kQ6K>::PADP;
    case kF32: return Geo<kF32>::PADP;
    case kBF16: return Geo<kBF16>::PADP;
    default: return Geo<kQ5_0>::PADP;
    }
}
// Values per pad period of a staged x row (piece-major rows: one piece).
inline uint32_t pad_period(int t, uint32_t m) {
    if (piece_major(t, m)) return 64;
    return pad_period(t);
}

// Launchers, one translation unit per weight type.
// lds: dynamic LDS bytes of this launch; lds_max: the device's per-workgroup
// limit (each instance's attribute is raised to it once, on its first launch
// that needs more than 64 KB).
typedef hipError_t (*MvLauncher)(const MvArgs &, uint32_t m, uint32_t nr, dim3 grid, dim3 block, size_t lds,
                                 size_t lds_max, hipStream_t s);
typedef hipError_t (*DqLauncher)(const DqArgs &, hipStream_t s);
typedef hipError_t (*MvAttributes)(uint32_t m, uint32_t nr, hipFuncAttributes *attr);

hipError_t launch_mv_f16(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_q8_0(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_q4_k(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_q6_k(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_q5_0(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_f32(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t launch_mv_bf16(const MvArgs &, uint32_t, uint32_t, dim3, dim3, size_t, size_t, hipStream_t);
hipError_t attributes_mv_f16(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_q8_0(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_q4_k(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_q6_k(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_q5_0(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_f32(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t attributes_mv_bf16(uint32_t, uint32_t, hipFuncAttributes *);
hipError_t launch_dq_f16(const DqArgs &, hipStream_t);
hipError_t launch_dq_q8_0(const DqArgs &, hipStream_t);
hipError_t launch_dq_q4_k(const DqArgs &, hipStream_t);
hipError_t launch_dq_q6_k(const DqArgs &, hipStream_t);
hipError_t launch_dq_q5_0(const DqArgs &, hipStream_t);
hipError_t launch_dq_f32(const DqArgs &, hipStream_t);
hipError_t launch_dq_bf16(const DqArgs &, hipStream_t);

// Error text for row_exact_last_error() (returns code) and the launch
// counter, shared by every host translation unit of the library.
int report_error(int code, const char *msg);
void count_launch();

}  // namespace rex
