// Host side of the row-exact mat-vec C ABI: argument checks, schedule and
// launch.  The argument contract is that of mlx-native 0.18.0
// src/ops/row_exact_matvec.rs, validate() (shape, k multiple, strides,
// pointer alignment, output aliasing, sizes), checked here in this library's
// own order and terms; the schedule is this library's own (wave64 pieces,
// rows per wave, LDS passes).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "re_internal.h"
#include "row_exact_mv.h"

// Waves with at least this many items walk with unconditional loads (more
// than the load depth of 2; measured on MI355X: waves of one or two items are
// faster with the loads under a branch).
#ifndef REX_WALK_UNCONDITIONAL_MIN_ITEMS
#define REX_WALK_UNCONDITIONAL_MIN_ITEMS 3
#endif
// 1: rows whose last 64-lane step is at most half full take 32 lanes per
// row (see lane_map_log2).
#ifndef REX_HALF_STEP_LANES
#define REX_HALF_STEP_LANES 1
#endif

using namespace rex;

namespace {

thread_local std::string g_err;
std::atomic<uint64_t> g_launches{0};

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = std::string("row_exact_mv: ") + buf;
    return code;
}

}  // namespace

// Shared with the other host translation units of the library.
int rex::report_error(int code, const char *msg) { return fail(code, "%s", msg); }
void rex::count_launch() { g_launches.fetch_add(1, std::memory_order_relaxed); }

namespace {

const char *type_name(int t) {
    static const char *names[] = {"F16", "Q8_0", "Q4_K", "Q6_K", "Q5_0", "F32", "BF16"};
    return (t >= 0 && t < kNumTypes) ? names[t] : "?";
}

bool valid_type(int t) { return t >= 0 && t < kNumTypes; }

uint32_t k_multiple(int t) {
    switch (t) {
    case kF16: case kF32: case kBF16: return 4;
    case kQ8_0: case kQ5_0: return 32;
    default: return 256;
    }
}

// Weight pointer alignment (the page's 8 / 2 / 16 / 2 / 2 bytes for its five
// types; F32 rows are read 16 bytes at a time, BF16 as F16).  Q8_0, Q6_K and
// Q5_0 blocks are read with loads that never start before the block (see
// row_base in the kernels), so 2 bytes suffice.
uint32_t w_align(int t) {
    switch (t) {
    case kF16: case kBF16: return 8;
    case kQ4K: case kF32: return 16;
    default: return 2;
    }
}

uint64_t row_bytes_of(int t, uint32_t k) {
    switch (t) {
    case kF16: return (uint64_t)k * 2;
    case kQ8_0: return (uint64_t)(k / 32) * 34;
    case kQ4K: return (uint64_t)(k / 256) * 144;
    case kQ6K: return (uint64_t)(k / 256) * 210;
    case kQ5_0: return (uint64_t)(k / 32) * 22;
    case kF32: return (uint64_t)k * 4;
    case kBF16: return (uint64_t)k * 2;
    default: return 0;
    }
}

struct DevInfo {
    int cus = 0;
    size_t lds_max = 0;
    bool ok = false;
};

int device_info(DevInfo &out) {
    static std::mutex mu;
    static DevInfo cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && cache[dev].ok) {
        out = cache[dev];
        return 0;
    }
    int cus = 0, lds = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "device query: %s", hipGetErrorString(e));
    DevInfo d;
    d.cus = cus > 0 ? cus : 1;
    d.lds_max = (size_t)(lds > 0 ? lds : 65536);
    d.ok = true;
    if (dev >= 0 && dev < 64) cache[dev] = d;
    out = d;
    return 0;
}

// Floats per staged x row for kc values of an m-row product (4 pad floats
// per pad period).
uint32_t xs_stride(int t, uint32_t kc, uint32_t m) {
    const uint32_t padp = pad_period(t, m);
    return kc + 4 * ((kc + padp - 1) / padp);
}

// LDS of a workgroup: the m staged input rows (padded), then 4m doubles for
// the fused normalisation's per-row partial sums.
size_t lds_x_bytes(int t, uint32_t m, uint32_t k, uint32_t k_chunk) {
    const uint32_t kc = k_chunk < k ? k_chunk : k;
    return (size_t)m * xs_stride(t, kc, m) * sizeof(float);
}
// Floats per input row of the segment sums (Q4_K: one per 32 staged values).
uint32_t sx_stride(int t, uint32_t k, uint32_t k_chunk) {
    const uint32_t kc = k_chunk < k ? k_chunk : k;
    return t == kQ4K ? kc / 32 : 0;
}
// LDS layout: staged x (m rows, padded), 4 m doubles of the fused norm's
// statistic, the segment sums (m rows).
size_t lds_sx_offset(int t, uint32_t m, uint32_t k, uint32_t k_chunk) {
    return lds_x_bytes(t, m, k, k_chunk) + (size_t)4 * m * sizeof(double);
}
// Then, for a K split, 32 float partial sums per wave (8 waves).
size_t lds_kp_offset(int t, uint32_t m, uint32_t k, uint32_t k_chunk) {
    return (lds_sx_offset(t, m, k, k_chunk) + (size_t)m * sx_stride(t, k, k_chunk) * sizeof(float) + 15) & ~(size_t)15;
}
size_t lds_bytes(int t, uint32_t m, uint32_t k, uint32_t k_chunk, uint32_t k_split = 1) {
    return lds_kp_offset(t, m, k, k_chunk) + (k_split > 1 ? 8 * 32 * sizeof(float) : 0);
}

typedef unsigned __int128 u128;

// (batch-1)*bs + (rows-1)*rs + cols, the last element + 1 of a strided view.
u128 extent(uint32_t batch, uint64_t bs, uint32_t rows, uint64_t rs, uint64_t cols) {
    return (u128)(batch - 1) * bs + (u128)(rows - 1) * rs + cols;
}

row_exact_strides_t resolve_strides(const row_exact_strides_t *s, uint32_t m, uint32_t n, uint32_t k) {
    if (s) return *s;
    row_exact_strides_t c;
    c.x_row_stride = k;
    c.x_batch_stride = 0;
    c.y_row_stride = n;
    c.y_batch_stride = 0;
    (void)m;
    return c;
}

// Checks every entry point shares: weight type, m, the dimensions and k's
// block multiple.  Rows are counted in 32 bits inside the kernels (row groups
// of up to 16 rows), so n stays below 2^31.
int check_shape(int t, uint32_t n, uint32_t k, uint32_t m, uint32_t batch) {
    if (!valid_type(t)) return fail(ROW_EXACT_EARG, "weight type %d is not one of 0..%d", t, kNumTypes - 1);
    if (m < 1 || m > ROW_EXACT_MAX_ROWS)
        return fail(ROW_EXACT_EARG, "m = %u: a call takes 1 to %d input rows", m, ROW_EXACT_MAX_ROWS);
    if (!n || !k || !batch)
        return fail(ROW_EXACT_EARG, "n = %u, k = %u, batch = %u: every dimension must be at least 1", n, k, batch);
    if (k % k_multiple(t))
        return fail(ROW_EXACT_EARG, "%s weights need k divisible by %u, got k = %u", type_name(t), k_multiple(t), k);
    if (n > 0x7fffffffu) return fail(ROW_EXACT_EEXTENT, "n = %u: at most 2^31 - 1 weight rows per batch entry", n);
    return 0;
}

// Byte extents of W (weight_sets sets of n rows), x and y.
int sizes(int t, uint32_t n, uint32_t k, uint32_t m, uint32_t batch, const row_exact_strides_t &s, uint64_t &wb,
          uint64_t &xb, uint64_t &yb, uint32_t weight_sets = 0) {
    const u128 w = (u128)row_bytes_of(t, k) * n * (weight_sets ? weight_sets : batch);
    const u128 x = extent(batch, s.x_batch_stride, m, s.x_row_stride, k) * 4;
    const u128 y = extent(batch, s.y_batch_stride, m, s.y_row_stride, n) * 4;
    const u128 lim = (u128)1 << 62;
    if (w >= lim || x >= lim || y >= lim)
        return fail(ROW_EXACT_EEXTENT, "W, x or y spans 2^62 bytes or more");
    wb = (uint64_t)w;
    xb = (uint64_t)x;
    yb = (uint64_t)y;
    return 0;
}

bool overlap(uintptr_t a, uint64_t an, uintptr_t b, uint64_t bn) { return a < b + bn && b < a + an; }

// Output element (b, j, i), i < n, sits at b*ybs + j*yrs + i.  Accepted
// layouts nest: of the two strided axes that have more than one entry, the
// one with the smaller stride is the inner one, and each stride reaches past
// everything nested inside it (n values, then the inner axis' whole extent).
// Every nested layout writes each element once; interleaved layouts (which
// can also be free of collisions) are refused, as the page refuses them.
bool outputs_nest(uint32_t n, uint32_t m, uint64_t yrs, uint32_t batch, uint64_t ybs) {
    struct Axis { uint64_t stride; uint32_t count; } ax[2] = {{yrs, m}, {ybs, batch}};
    if (ax[1].stride < ax[0].stride) {
        const Axis t = ax[0];
        ax[0] = ax[1];
        ax[1] = t;
    }
    u128 span = n;
    for (const Axis &a : ax) {
        if (a.count < 2) continue;
        if ((u128)a.stride < span) return false;
        span += (u128)(a.count - 1) * a.stride;
    }
    return true;
}

int validate_mv(int t, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                const row_exact_strides_t &s, uint64_t &wb, uint64_t &xbytes, uint64_t &ybytes,
                const int32_t *ids = nullptr, uint32_t num_experts = 0) {
    int rc = check_shape(t, n, k, m, batch);
    if (rc) return rc;
    if (!W || !x || !y) return fail(ROW_EXACT_EARG, "W, x and y must be non-NULL device pointers");
    if (ids && !num_experts) return fail(ROW_EXACT_EARG, "num_experts is 0: expert_ids has nothing to select");
    const uint32_t wa = w_align(t);
    if ((uintptr_t)W % wa)
        return fail(ROW_EXACT_EALIGN, "%s weights must sit on a %u-byte boundary (W mod %u = %u)", type_name(t), wa,
                    wa, (unsigned)((uintptr_t)W % wa));
    if ((uintptr_t)x % 16)
        return fail(ROW_EXACT_EALIGN, "x must sit on a 16-byte boundary (x mod 16 = %u)", (unsigned)((uintptr_t)x % 16));
    if ((uintptr_t)y % 4) return fail(ROW_EXACT_EALIGN, "y must sit on a 4-byte boundary");
    if (ids && (uintptr_t)ids % 4) return fail(ROW_EXACT_EALIGN, "expert_ids must sit on a 4-byte boundary");
    if ((s.x_row_stride | s.x_batch_stride) & 3u)
        return fail(ROW_EXACT_ESTRIDE, "x strides (row %u, batch %u) must be multiples of 4 elements", s.x_row_stride,
                    s.x_batch_stride);
    if (!outputs_nest(n, m, s.y_row_stride, batch, s.y_batch_stride))
        return fail(ROW_EXACT_EALIAS,
                    "y layout writes some element twice (n %u, m %u at row stride %u, batch %u at batch stride %u)", n,
                    m, s.y_row_stride, batch, s.y_batch_stride);
    rc = sizes(t, n, k, m, batch, s, wb, xbytes, ybytes, ids ? num_experts : 0);
    if (rc) return rc;
    if (row_bytes_of(t, k) > 0x7fffffffull)
        return fail(ROW_EXACT_EEXTENT, "one weight row takes %llu bytes, more than 2^31 - 1",
                    (unsigned long long)row_bytes_of(t, k));
    if (overlap((uintptr_t)y, ybytes, (uintptr_t)W, wb) || overlap((uintptr_t)y, ybytes, (uintptr_t)x, xbytes) ||
        (ids && overlap((uintptr_t)y, ybytes, (uintptr_t)ids, 4ull * batch)))
        return fail(ROW_EXACT_EALIAS, "y overlaps the bytes of W, x or expert_ids");
    return 0;
}

// Reduction split (numerics): the waves whose partial sums form one output,
// 1, 2, 4 or 8, derived from the weight shape alone -- type, k and the rows
// n of one batch entry -- never from m, the batch or the packing (the page
// derives its simdgroup split from (weight, rows, k) the same way; leaving
// the batch out keeps a batched or gathered call bitwise equal to separate
// calls per entry).  Skinny outputs deal each row's wave steps over K
// waves, so that rows times K reach about one wave per SIMD of a 256-CU
// device (1024; a constant, so that the bits do not depend on the device),
// without a wave holding less than one whole wave step: K is the largest
// power of two <= min(1024 / n, 8, whole wave steps of a row).  Rows of at
// most 32 pieces (16 or 32 lanes per row) and rows of fewer than 3 whole
// wave steps are not split: at 2 steps the split measured slower at m <= 4
// (Q8_0 512 x 4096, m = 1: 3.2 us unsplit, 3.7 us split in 2), the one
// wave's single-pass walk being cheaper than the partial-sum exchange.  At
// n >= 1024, K is 1: one wave's 64 lanes per output.
uint32_t derived_k_split(int t, uint32_t k, uint32_t rows) {
    if (lanes_per_row_log2(t, k) < 6) return 1;
    const uint32_t steps = pieces_of(t, k) / 64;
    if (steps < 3) return 1;
    const uint32_t per_row = 1024 / (rows ? rows : 1);
    uint32_t K = 1;
    while (K < 8 && 2 * K <= per_row && 2 * K <= steps) K *= 2;
    return K;
}

// Lanes per row (log2) of the product under reduction split K: 16 or 32
// for rows of at most 16 / 32 pieces; 32 also for unsplit rows of the
// block-quantized types whose last 64-lane wave step would be at most half
// full (64 s + r pieces, 0 < r <= 32; e.g. Q6_K k = 14336: 3.5 steps of 64
// lanes): on 32 lanes, two rows per wave, such a row issues half a 64-lane
// step less; 64 otherwise.  Measured on MI355X, interleaved against 64
// lanes, n = 4096 (Q5_0: 16 x 1024 grouped), m = 1, 2, 4, 8: Q6_K
// 4096 x 14336 -9% at m = 1 and -2% to -8% above; rows of 1.5, 3.5 and
// 5.4 steps of Q4_K, Q6_K, Q5_0 and Q8_0 -4% to -28% with few exceptions;
// rows of about one step (Q8_0 k = 2112 and 3072, Q4_K k = 4352) +4% to +8%
// at m = 1 and 2, -4% to -14% above; the dense types, whose pieces carry
// little vector work per byte, 4-18% slower (half as many waves for the
// same rows), so they keep 64 lanes.  Part of the numerics (the lane
// partials and their tree), so a function of (type, k, K) only.  A lane
// addresses the rows of its slot by a 32-bit offset from the wave's first
// row (up to 4 rows per slot), so the map is kept to rows under 2^29 bytes.
uint32_t lane_map_log2(int t, uint32_t k, uint32_t K) {
    const uint32_t lpr = lanes_per_row_log2(t, k);
    const bool blocks = t == kQ8_0 || t == kQ4K || t == kQ6K || t == kQ5_0;
    const uint32_t tail = pieces_of(t, k) % 64;
    if (REX_HALF_STEP_LANES && blocks && lpr == 6 && K == 1 && tail > 0 && tail <= 32 &&
        row_bytes_of(t, k) < (1u << 29))
        return 5;
    return lpr;
}

MvAttributes mv_attributes(int t) {
    switch (t) {
    case kF16: return attributes_mv_f16;
    case kQ8_0: return attributes_mv_q8_0;
    case kQ4K: return attributes_mv_q4_k;
    case kQ6K: return attributes_mv_q6_k;
    case kF32: return attributes_mv_f32;
    case kBF16: return attributes_mv_bf16;
    default: return attributes_mv_q5_0;
    }
}

// ROW_EXACT_DEBUG (print the schedule inputs; never changes numerics), read
// once per process.
bool debug_enabled() {
    static const bool on = getenv("ROW_EXACT_DEBUG") != nullptr;
    return on;
}

// VGPRs of the plain instance <t, m, nr>, asked of the runtime once per
// instance and process (0 = unknown).
int instance_vgprs(int t, uint32_t m, uint32_t nr) {
    static std::atomic<int> cache[kNumTypes][ROW_EXACT_MAX_ROWS + 1][5];  // -1 after a failed query
    const uint32_t ni = nr == 4 ? 3 : nr;
    std::atomic<int> &slot = cache[t][m][ni];
    int v = slot.load(std::memory_order_relaxed);
    if (v != 0) return v > 0 ? v : 0;
    hipFuncAttributes attr;
    if (mv_attributes(t)(m, nr, &attr) != hipSuccess) {
        (void)hipGetLastError();
        slot.store(-1, std::memory_order_relaxed);
        return 0;
    }
    v = attr.numRegs > 0 ? attr.numRegs : -1;
    slot.store(v, std::memory_order_relaxed);
    return v > 0 ? v : 0;
}

// Workgroups of a kernel instance that fit on one CU at once: VGPRs (512 per
// SIMD lane, 4 SIMDs, waves of a workgroup spread over the SIMDs), at most 8
// waves per SIMD, and LDS.
int workgroups_per_cu(int t, uint32_t m, uint32_t nr, uint32_t waves, size_t lds, size_t lds_per_cu) {
    const int regs = instance_vgprs(t, m, nr);
    if (!regs) return 1;
    const int vg = (regs + 7) / 8 * 8;
    int per_simd = 512 / vg;
    if (per_simd > 8) per_simd = 8;
    const int waves_per_simd_per_wg = (int)((waves + 3) / 4);
    int by_regs = per_simd / waves_per_simd_per_wg;
    int by_lds = lds ? (int)(lds_per_cu / lds) : 8;
    int r = by_regs < by_lds ? by_regs : by_lds;
    if (r > 8) r = 8;
    if (debug_enabled())
        fprintf(stderr, "row_exact_mv: kernel %s m=%u rows/wave=%u: %d VGPRs, %d waves/SIMD, lds %zu -> %d workgroups/CU\n",
                type_name(t), m, nr, regs, per_simd, lds, r < 1 ? 1 : r);
    return r < 1 ? 1 : r;
}

// Waves per workgroup: 8, halved while the row groups would leave waves of
// the device without one, but never fewer than stage the workgroup's m*kc/4
// chunks of x with at most two loads per thread: waves without rows still
// stage x (held-out Q4_K 1024 x 2816, m = 1..4: 8 waves, half of them
// without rows, 3-6% faster than 4 busy waves; F16 256 x 512 at m = 1, 2 KB
// of x: one wave, 7% faster than 8).
uint32_t waves_per_workgroup(uint32_t gpb, uint32_t batch, int cus, uint32_t m, uint32_t kc) {
    uint32_t w = 8;
    while (w > 1 && (uint64_t)gpb * batch < (uint64_t)w * cus) w >>= 1;
    const uint64_t chunks = (uint64_t)m * kc / 4;
    uint32_t wx = 1;
    while (wx < 8 && (uint64_t)wx * 64 * 2 < chunks) wx <<= 1;
    return w > wx ? w : wx;
}

// Most workgroups per batch entry worth launching for gpb row groups: one
// row group per wave, or, when that leaves CUs without a workgroup, one per
// CU while there are row groups (its waves without rows only stage x).
uint32_t max_workgroups(uint32_t gpb, uint32_t waves, uint32_t batch, int cus) {
    const uint32_t by_waves = (gpb + waves - 1) / waves;
    const uint32_t per_cu = (uint32_t)(((uint64_t)cus + batch - 1) / batch);
    const uint32_t by_cus = gpb < per_cu ? gpb : per_cu;
    return by_waves > by_cus ? by_waves : by_cus;
}

// Most rows per wave whose kernel holds all its state in registers at this m.
uint32_t max_rows_per_wave(int t, uint32_t m) {
    if ((t == kQ4K || t == kQ6K) && m >= 5) return 2;
    return 4;
}

// fused_norm: the schedule of row_exact_mv_add_rmsnorm (its instances carry
// the normalisation prologue; rows per wave as before the single-row rule
// below, which measured 3% slower there at m = 4).
int default_schedule(int t, uint32_t n, uint32_t k, uint32_t m, uint32_t batch, row_exact_schedule_t &s,
                     bool fused_norm = false) {
    DevInfo di;
    int rc = device_info(di);
    if (rc) return rc;
    const uint64_t rows = (uint64_t)n * batch;
    s.k_split = derived_k_split(t, k, n);
    s.lanes_per_row = 1u << lane_map_log2(t, k, s.k_split);
    const uint32_t step = wave_step_values(t);
    if (s.k_split > 1) {
        // Skinny outputs, K waves per row group: max(4, K) waves per
        // workgroup (one or two row groups of single rows; 4 waves measured
        // 2-14% faster than 8 at K = 2 and up to 3% at K = 4), one round of
        // row groups; LDS passes of the most whole wave steps that fit when
        // x does not.
        const uint32_t K = s.k_split;
        uint32_t kc = k;
        if (lds_bytes(t, m, k, k, K) > di.lds_max) {
            kc = step;
            while (kc + step < k && lds_bytes(t, m, k, kc + step, K) <= di.lds_max) kc += step;
        }
        s.k_chunk = kc;
        s.rows_per_wave = 1;
        s.waves_per_workgroup = K > 4 ? K : 4;
        const uint32_t groups = s.waves_per_workgroup / K;
        s.workgroups_per_batch = (n + groups - 1) / groups;
        return 0;
    }
    // LDS passes: one if the m staged rows fit, else the largest wave-step multiple that fits
    uint32_t kc = k;
    if (lds_bytes(t, m, k, k) > di.lds_max) {
        kc = step;
        while (kc + step < k && lds_bytes(t, m, k, kc + step) <= di.lds_max) kc += step;
    }
    s.k_chunk = kc;
    if (m <= 2 && kc >= k) {
        // Few input rows: the weight loads dominate.  Measured best on
        // MI355X: about 32 waves per CU over the whole grid (the hardware
        // balances the tail across workgroups), single rows.  Where the
        // rows would give each of those waves between one and two of them,
        // single rows on 24 waves per CU instead, so each wave walks two or
        // more: a row of one wave step is one item, and a wave with one item
        // has nothing to multiply while its loads are in flight (Q4_K
        // 14336 x 4096: 12.3 -> 10.8 us at m = 1); for rows of several
        // steps, against two rows per wave on 32 waves per CU (one row group
        // per wave): 14336 x 8192 Q4_K -11%, 14336 x 4096 Q8_0 -7%, 14336 x
        // 8192 Q6_K -24% at m = 1, 14336 x 4096 Q8_0 -4% at m = 2.
        uint64_t target = (uint64_t)di.cus * 32;
        const uint32_t lpr = lane_map_log2(t, k, 1);
        const uint64_t wave_rows = rows >> (6 - lpr);  // rows / slots per wave
        const uint32_t steps = (pieces_of(t, k) + (1u << lpr) - 1) >> lpr;
        uint32_t nr = 1;
        if (m == 2 && steps >= 2) {
            // two input rows, rows of several wave steps: 16 waves per CU
            // (against 24 or 32: 14336 x 6144 Q4_K -16%, 14336 x 4096 Q8_0
            // -7%, 12288 x 4096 Q8_0 and BF16 -2%, 14336 x 2048 F16 +0.4%)
            target = (uint64_t)di.cus * 16;
        } else if (wave_rows > target && wave_rows <= 2 * target) {
            if (m == 2 && steps < 2) {
                // two input rows: 2 rows per wave on 8 waves per CU, each
                // wave walking several groups (Q4_K 14336 x 4096: -8%)
                nr = 2;
                target = (uint64_t)di.cus * 8;
            } else {
                target = (uint64_t)di.cus * 24;
            }
        }
        // A workgroup's x stage that leaves room for at most one more on a
        // CU (m*k*4 bytes over a third of the LDS): each further round of
        // workgroups stages x again on a CU with little else to run, so one
        // workgroup per CU, each wave walking its share of row groups; at
        // m = 2 two rows per wave when waves then get more than one group
        // (4096 x 8192 Q8_0, one group of two rows per wave: 12% slower than
        // two single rows).
        // Against the rule above, m = 2: 16384 x 11008 Q8_0 -16%, 16384 x
        // 14336 Q6_K -20%, 14336 x 14336 Q4_K -28%, 16 x 1024 x 11008 grouped
        // Q5_0 -18%, 4096 x 8192 Q8_0 -9%, 14336 x 8192 Q4_K -17%; m = 1:
        // 14336 x 14336 Q4_K -9%, 16384 x 14336 Q6_K -3% (within 2% of it
        // on 4096 x 14336 Q8_0, 8192 x 14336 Q6_K, 16384 x 8192 Q6_K at m = 2).
        const bool one_per_cu = di.lds_max / lds_bytes(t, m, k, kc) < 3;
        if (one_per_cu)
            nr = m == 2 && steps >= 2 && wave_rows > 2ull * 8 * di.cus ? 2 : 1;
        s.rows_per_wave = nr;
        const uint32_t rg = nr << (6 - lpr);  // rows per group
        const uint32_t gpb = (n + rg - 1) / rg;
        const uint32_t waves = waves_per_workgroup(gpb, batch, di.cus, m, kc);
        s.waves_per_workgroup = waves;
        const uint32_t max_wgs = max_workgroups(gpb, waves, batch, di.cus);
        if (one_per_cu) {
            const uint32_t w1 = (uint32_t)((di.cus + batch - 1) / batch);
            s.workgroups_per_batch = w1 < max_wgs ? w1 : max_wgs;
            return 0;
        }
        uint64_t w = (target / waves + batch - 1) / batch;
        // as for more input rows below: no more workgroups than keep each
        // one's weight bytes at or above the m*k*4 bytes of x it stages
        // (Q6_K 4096 x 14336 at m = 2: 512 -> 256 workgroups, -16%)
        const uint64_t x_wg = (uint64_t)m * k * sizeof(float);
        const u128 by_x = (u128)rows * row_bytes_of(t, k) / x_wg / di.cus * di.cus;
        const uint64_t cap = by_x > di.cus ? (uint64_t)by_x : (uint64_t)di.cus;
        if (w > (cap + batch - 1) / batch) w = (cap + batch - 1) / batch;
        if (w < 1) w = 1;
        s.workgroups_per_batch = (uint32_t)(w < max_wgs ? w : max_wgs);
        return 0;
    }
    // rows per wave: the most that still leaves 8 waves per CU (counted in
    // row slots: 32-lane rows of several steps take one row per slot, which
    // measured 4-16% faster than two for Q4_K, Q6_K and Q8_0 rows of 224
    // pieces at m = 5..8)
    const uint64_t target_waves = (uint64_t)di.cus * 8;
    const uint32_t lpr = lane_map_log2(t, k, 1);
    const uint64_t wave_rows = rows >> (6 - lpr);
    uint32_t nr = max_rows_per_wave(t, m);
    while (nr > 1 && wave_rows / nr < target_waves) nr >>= 1;
    // Up to 4 input rows and fewer than 16 rows per wave: single rows for
    // rows of several wave steps, so each wave walks more items with loads
    // in flight behind the multiply (3-10% faster than 2 or 4 rows per wave
    // at m = 3..4 on 4096 x 4096 Q8_0, BF16, F32 and 16 x 1024 x 4096 Q5_0);
    // rows of one wave step take 2 (each x value then feeds two rows;
    // 14336 x 4096 Q4_K at m = 4: -7% against single rows).  The
    // 128256-row head keeps 4.  Short rows (a wave already covers 2 or 4
    // rows per item) and the fused-norm instances measured slower with it
    // and keep the rule above.
    const uint32_t steps = (pieces_of(t, k) + (1u << lpr) - 1) >> lpr;
    if (m <= 4 && kc >= k && (lpr == 6 || steps >= 2) && !fused_norm && wave_rows < 16 * target_waves)
        nr = steps >= 2 ? 1u : (nr < 2u ? nr : 2u);  // never more than leaves 8 waves per CU
    s.rows_per_wave = nr;
    const uint32_t rg = nr << (6 - lpr);  // rows per group
    const uint32_t gpb = (n + rg - 1) / rg;
    const uint32_t waves = waves_per_workgroup(gpb, batch, di.cus, m, kc);
    s.waves_per_workgroup = waves;
    // workgroups: single pass -> as many as fit on the device at once (each
    // then walks its share of row groups); several passes -> one row group
    // per wave
    const uint32_t max_wgs = max_workgroups(gpb, waves, batch, di.cus);
    uint32_t wgs;
    if (kc >= k) {
        const int per_cu = workgroups_per_cu(t, m, nr, waves, lds_bytes(t, m, k, kc), di.lds_max);
        uint64_t target = (uint64_t)di.cus * (uint64_t)per_cu;
        // Each workgroup stages m*k*4 bytes of x from L2: fewer workgroups
        // (whole rounds of the device) when more would stream fewer weight
        // bytes each than they stage (Q8_0 4096 x 4096 at m = 4: one
        // workgroup per CU, 8.7 -> 8.2 us).
        const uint64_t x_wg = (uint64_t)m * k * sizeof(float);
        const u128 by_x = (u128)rows * row_bytes_of(t, k) / x_wg / di.cus * di.cus;
        if (by_x < target) target = by_x > di.cus ? (uint64_t)by_x : (uint64_t)di.cus;
        uint64_t w = (target + batch - 1) / batch;
        if (w < 1) w = 1;
        wgs = (uint32_t)(w < max_wgs ? w : max_wgs);
    } else {
        wgs = max_wgs;
    }
    s.workgroups_per_batch = wgs;
    return 0;
}

// Checks that need no device (every field's range).  k_split may differ
// from the derived one (the caller then chooses the numerics, e.g. to keep
// the bits of an unsharded product on a row shard).
int check_schedule_fields(int t, uint32_t k, const row_exact_schedule_t &s) {
    const uint32_t K = s.k_split;
    if (!(K == 1 || K == 2 || K == 4 || K == 8))
        return fail(ROW_EXACT_ESCHEDULE, "schedule k_split (%u) must be 1, 2, 4 or 8", K);
    if (K > 1 && lanes_per_row_log2(t, k) < 6)
        return fail(ROW_EXACT_ESCHEDULE, "schedule k_split (%u): %s rows of k = %u (at most 32 pieces) are not split",
                    K, type_name(t), k);
    if (K > pieces_of(t, k) / 64 && K > 1)
        return fail(ROW_EXACT_ESCHEDULE, "schedule k_split (%u) exceeds the %u whole wave steps of a %s row of k = %u",
                    K, pieces_of(t, k) / 64, type_name(t), k);
    if (!(s.rows_per_wave == 1 || s.rows_per_wave == 2 || s.rows_per_wave == 4))
        return fail(ROW_EXACT_ESCHEDULE, "schedule rows_per_wave (%u) must be 1, 2 or 4", s.rows_per_wave);
    const uint32_t L = s.lanes_per_row;
    if (!(L == 0 || L == 16 || L == 32 || L == 64))
        return fail(ROW_EXACT_ESCHEDULE, "schedule lanes_per_row (%u) must be 0 (derived), 16, 32 or 64", L);
    if (L && L < 64 && K > 1)
        return fail(ROW_EXACT_ESCHEDULE, "schedule lanes_per_row (%u): a k_split (%u) needs 64 lanes per row", L, K);
    if (L && L < 64 && (uint64_t)(64 / L) * s.rows_per_wave * row_bytes_of(t, k) >= (1ull << 32))
        return fail(ROW_EXACT_ESCHEDULE,
                    "schedule lanes_per_row (%u) with rows_per_wave (%u): %s rows of k = %u are too long for the "
                    "32-bit row offsets of a wave's row slots",
                    L, s.rows_per_wave, type_name(t), k);
    if (s.waves_per_workgroup < 1 || s.waves_per_workgroup > 8)
        return fail(ROW_EXACT_ESCHEDULE, "schedule waves_per_workgroup (%u) must be 1 to 8", s.waves_per_workgroup);
    if (s.waves_per_workgroup % K)
        return fail(ROW_EXACT_ESCHEDULE, "schedule waves_per_workgroup (%u) must be a multiple of k_split (%u)",
                    s.waves_per_workgroup, K);
    if (s.workgroups_per_batch < 1)
        return fail(ROW_EXACT_ESCHEDULE, "schedule workgroups_per_batch must be >= 1");
    const uint32_t step = wave_step_values(t);
    if (s.k_chunk < k && (s.k_chunk == 0 || s.k_chunk % step))
        return fail(ROW_EXACT_ESCHEDULE, "schedule k_chunk (%u) must be >= k (%u) or a multiple of %u for %s",
                    s.k_chunk, k, step, type_name(t));
    return 0;
}

// Checks against the current device's limits.
int check_schedule_device(int t, uint32_t k, uint32_t m, const row_exact_schedule_t &s, const DevInfo &di) {
    const size_t l = lds_bytes(t, m, k, s.k_chunk, s.k_split);
    if (l > di.lds_max)
        return fail(ROW_EXACT_ESCHEDULE, "schedule needs %zu bytes of LDS, the device allows %zu", l, di.lds_max);
    return 0;
}

MvLauncher mv_launcher(int t) {
    switch (t) {
    case kF16: return launch_mv_f16;
    case kQ8_0: return launch_mv_q8_0;
    case kQ4K: return launch_mv_q4_k;
    case kQ6K: return launch_mv_q6_k;
    case kF32: return launch_mv_f32;
    case kBF16: return launch_mv_bf16;
    default: return launch_mv_q5_0;
    }
}

DqLauncher dq_launcher(int t) {
    switch (t) {
    case kF16: return launch_dq_f16;
    case kQ8_0: return launch_dq_q8_0;
    case kQ4K: return launch_dq_q4_k;
    case kQ6K: return launch_dq_q6_k;
    case kF32: return launch_dq_f32;
    case kBF16: return launch_dq_bf16;
    default: return launch_dq_q5_0;
    }
}

// Inputs of the fused add + RMS normalisation.
struct Norm {
    const float *r, *g;
    float *h;
    float eps;
};

// r, g, h against each other and the product's operands; r and h have x's
// layout, so x's byte extent.
int validate_norm(const Norm &nm, const void *W, const float *x, const float *y, uint32_t k, uint64_t wb,
                  uint64_t xbytes, uint64_t ybytes) {
    if (!nm.r) return fail(ROW_EXACT_EARG, "r must be a non-NULL device pointer");
    if (!(nm.eps >= 0.0f) || nm.eps > 3.4e38f) return fail(ROW_EXACT_EARG, "eps must be finite and >= 0");
    if ((uintptr_t)nm.r % 16 || (uintptr_t)nm.g % 16 || (uintptr_t)nm.h % 16)
        return fail(ROW_EXACT_EALIGN, "r, g and h must be 16-byte aligned");
    const uint64_t gb = nm.g ? 4ull * k : 0;
    if (overlap((uintptr_t)y, ybytes, (uintptr_t)nm.r, xbytes) || (nm.g && overlap((uintptr_t)y, ybytes, (uintptr_t)nm.g, gb)))
        return fail(ROW_EXACT_EALIAS, "output range overlaps r or g");
    if (nm.h && (overlap((uintptr_t)nm.h, xbytes, (uintptr_t)x, xbytes) ||
                 overlap((uintptr_t)nm.h, xbytes, (uintptr_t)nm.r, xbytes) ||
                 overlap((uintptr_t)nm.h, xbytes, (uintptr_t)W, wb) || overlap((uintptr_t)nm.h, xbytes, (uintptr_t)y, ybytes) ||
                 (nm.g && overlap((uintptr_t)nm.h, xbytes, (uintptr_t)nm.g, gb))))
        return fail(ROW_EXACT_EALIAS, "h overlaps x, r, g, W or y (other workgroups still read the inputs)");
    return 0;
}

int run_norm_two_launch(int t, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m,
                        uint32_t batch, const row_exact_strides_t &s, const Norm &nm, hipStream_t stream,
                        void *work);

// A product launch, scheduled and checked, not yet enqueued.
struct MvLaunch {
    int t;
    MvArgs a;
    uint32_t m, nr;
    dim3 grid, block;
    size_t lds, lds_max;
};

// Schedules the product of operands that have passed validate_mv (strides
// resolved) and fills its launch; enqueues nothing.  row_scale: per (batch
// entry, input row) output scales, [batch][m] (the second launch of the
// two-launch normalisations), or NULL.
int plan_mv(int t, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
            const row_exact_strides_t &s, const row_exact_schedule_t *pin, const int32_t *ids, uint32_t num_experts,
            const Norm *norm, const double *row_scale, MvLaunch &L) {
    int rc = 0;
    if (pin) {
        rc = check_schedule_fields(t, k, *pin);
        if (rc) return rc;
    }
    DevInfo di;
    rc = device_info(di);
    if (rc) return rc;
    row_exact_schedule_t sch;
    if (pin) {
        sch = *pin;
    } else {
        rc = default_schedule(t, n, k, m, batch, sch, norm != nullptr);
        if (rc) return rc;
    }
    rc = check_schedule_fields(t, k, sch);
    if (!rc) rc = check_schedule_device(t, k, m, sch, di);
    if (rc) return rc;

    MvArgs a;
    a.W = (const uint8_t *)W;
    a.x = x;
    a.y = y;
    a.row_bytes = row_bytes_of(t, k);
    a.batch_bytes = a.row_bytes * n;
    a.xbs = s.x_batch_stride;
    a.ybs = s.y_batch_stride;
    a.n = n;
    a.k = k;
    a.xrs = s.x_row_stride;
    a.yrs = s.y_row_stride;
    a.pieces = pieces_of(t, k);
    a.lpr_log2 = sch.lanes_per_row == 16 ? 4u : sch.lanes_per_row == 32 ? 5u : sch.lanes_per_row == 64 ? 6u
                                                                       : lane_map_log2(t, k, sch.k_split);
    const uint32_t nr = sch.rows_per_wave;
    const uint32_t rg = nr << (6 - a.lpr_log2);  // rows per group: NR rows in each of the wave's slots
    a.groups_per_batch = (n + rg - 1) / rg;
    uint32_t wgs = sch.workgroups_per_batch < a.groups_per_batch ? sch.workgroups_per_batch : a.groups_per_batch;
    a.groups_per_wg = (a.groups_per_batch + wgs - 1) / wgs;
    a.batch = batch;
    wgs = (a.groups_per_batch + a.groups_per_wg - 1) / a.groups_per_wg;  // as the kernel recomputes it
    const uint32_t step = wave_step_values(t);
    if (sch.k_chunk >= k) {
        a.nchunks = 1;
        a.kchunk = k;
        a.pieces_per_chunk = a.pieces;
    } else {
        a.kchunk = sch.k_chunk;
        a.pieces_per_chunk = sch.k_chunk / step * 64;
        a.nchunks = (a.pieces + a.pieces_per_chunk - 1) / a.pieces_per_chunk;
    }
    a.xs_stride = xs_stride(t, a.kchunk, m);
    a.ids = ids;
    a.num_experts = num_experts;
    a.r = norm ? norm->r : nullptr;
    a.g = norm ? norm->g : nullptr;
    a.h = norm ? norm->h : nullptr;
    a.eps = norm ? norm->eps : 0.0f;
    a.norm_offset = (uint32_t)lds_x_bytes(t, m, k, sch.k_chunk);
    a.sx_offset = (uint32_t)lds_sx_offset(t, m, k, sch.k_chunk);
    a.sx_stride = sx_stride(t, k, sch.k_chunk);
    // x by loads that write LDS directly where, at m = 1, it is larger than
    // the register staging requests ahead of the weights (2 chunks of 4
    // values per thread; the rest would be requested behind the weights, a
    // second memory round trip before the first multiply: Q6_K 4096 x 14336
    // -7%).  At m = 2 (4 chunks per thread ahead) the same measured 3%
    // slower than the register staging, and elsewhere it is not needed.
    {
        const uint64_t ahead = 4ull * 2 * 64 * sch.waves_per_workgroup;
        const bool dma_type = t == kQ6K;  // the types with a DMA staging path (Tr<T>::LOADS > 0)
        a.x_dma = (a.nchunks == 1 && m == 1 && !norm && dma_type && k > ahead && sch.k_split == 1) ? 1u : 0u;
    }
    a.row_scale = row_scale;
    a.row_scale_stride = m;
    a.k_split = sch.k_split;
    a.kp_offset = (uint32_t)lds_kp_offset(t, m, k, sch.k_chunk);
    {
        // items a wave walks in the single pass: its row groups x wave steps
        const uint32_t waves = sch.waves_per_workgroup;
        const uint64_t steps = (a.pieces + (1u << a.lpr_log2) - 1) >> a.lpr_log2;
        const uint64_t items = (uint64_t)((a.groups_per_wg + waves - 1) / waves) * steps;
        a.walk_unconditional = items >= REX_WALK_UNCONDITIONAL_MIN_ITEMS ? 1u : 0u;
    }
    const uint64_t grid_x = (uint64_t)wgs * batch;
    if (grid_x > 0x7fffffffull)
        return fail(ROW_EXACT_ESCHEDULE, "grid of %llu workgroups exceeds the launch limit", (unsigned long long)grid_x);
    L.t = t;
    L.a = a;
    L.m = m;
    L.nr = nr;
    L.grid = dim3((uint32_t)grid_x);
    L.block = dim3(64 * sch.waves_per_workgroup);
    L.lds = lds_bytes(t, m, k, sch.k_chunk, sch.k_split);
    L.lds_max = di.lds_max;
    return 0;
}

int enqueue_mv(const MvLaunch &L, hipStream_t stream) {
    hipError_t e = mv_launcher(L.t)(L.a, L.m, L.nr, L.grid, L.block, L.lds, L.lds_max, stream);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return 0;
}

// Validates every operand, then plans and enqueues the product (two launches
// for the fused normalisation on a work buffer).
int run(int t, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
        const row_exact_strides_t *strides, const row_exact_schedule_t *pin, hipStream_t stream,
        const int32_t *ids = nullptr, uint32_t num_experts = 0, const Norm *norm = nullptr,
        void *norm_work = nullptr) {
    g_err.clear();
    const row_exact_strides_t s = resolve_strides(strides, m, n, k);
    uint64_t wb, xbytes, ybytes;
    int rc = validate_mv(t, W, x, y, n, k, m, batch, s, wb, xbytes, ybytes, ids, num_experts);
    if (rc) return rc;
    if (norm) {
        rc = validate_norm(*norm, W, x, y, k, wb, xbytes, ybytes);
        if (rc) return rc;
        if (norm_work) return run_norm_two_launch(t, W, x, y, n, k, m, batch, s, *norm, stream, norm_work);
    }
    MvLaunch L;
    rc = plan_mv(t, W, x, y, n, k, m, batch, s, pin, ids, num_experts, norm, nullptr, L);
    if (rc) return rc;
    return enqueue_mv(L, stream);
}

// Bytes of the two-launch fused normalisation's work buffer: u ([batch][m][k]
// floats, rounded up to 256 bytes) then the inverse RMS values ([batch][m]
// doubles); ROW_EXACT_NORM_WORK_BYTES in the header.
uint64_t norm_work_bytes(uint32_t k, uint32_t m, uint32_t batch) {
    const uint64_t u = ((uint64_t)batch * m * k * sizeof(float) + 255) & ~255ull;
    return u + (uint64_t)batch * m * sizeof(double);
}

// The product of the two-launch normalisations on the work buffer: u =
// [batch][m][k] floats, each output scaled by its row's inv ([batch][m]
// doubles), y in the caller's layout s.  Planned before the first of the two
// launches, so that a call that fails enqueues nothing.  Also checks the
// extents the work buffer's layout adds (the u view's batch stride m * k and
// the first launch's grid of batch * m workgroups); the caller has checked
// W, y and the work buffer itself.
int plan_scaled_product(int t, const void *W, const float *u, float *y, uint32_t n, uint32_t k, uint32_t m,
                        uint32_t batch, const row_exact_strides_t &s, const double *inv, MvLaunch &L) {
    if ((uint64_t)batch * m > 0x7fffffffull)
        return fail(ROW_EXACT_EEXTENT, "batch (%u) x m (%u) normalised rows exceed one launch's 2^31 - 1 workgroups",
                    batch, m);
    if (batch > 1 && (uint64_t)m * k > 0xffffffffull)
        return fail(ROW_EXACT_EEXTENT, "m (%u) x k (%u) values per batch entry exceed the 32-bit batch stride", m, k);
    row_exact_strides_t su;
    su.x_row_stride = k;
    su.x_batch_stride = batch > 1 ? m * k : 0;
    su.y_row_stride = s.y_row_stride;
    su.y_batch_stride = s.y_batch_stride;
    return plan_mv(t, W, u, y, n, k, m, batch, su, nullptr, nullptr, 0, nullptr, inv, L);
}

// Work bytes of a call, or 0 (with the error set) when they reach 2^62.
uint64_t checked_norm_work_bytes(uint32_t k, uint32_t m, uint32_t batch) {
    if ((unsigned __int128)batch * m * k * sizeof(float) >= ((unsigned __int128)1 << 62)) {
        fail(ROW_EXACT_EEXTENT, "the work buffer of batch %u x m %u x k %u floats spans 2^62 bytes or more", batch, m, k);
        return 0;
    }
    return norm_work_bytes(k, m, batch);
}

// Scratch of row_exact_mv_add_rmsnorm_noalloc (the work buffer of the
// two-launch fused normalisation, for callers that cannot allocate): one
// array per GPU, held until the process ends.  Host code never
// uses its name as an address (that is a host-side stand-in); it asks the
// runtime for the array's device address once per device.
static __device__ __align__(256) uint8_t scratch[ROW_EXACT_NOALLOC_SCRATCH_BYTES];

// Device address of the current device's scratch array (looked up on the
// first call on that device, with it current).
int noalloc_scratch(void *&out) {
    static std::mutex mu;
    static void *ptrs[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(ROW_EXACT_EHIP, "device %d beyond the library's 64-device table", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ROW_EXACT_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        ptrs[dev] = p;
    }
    out = ptrs[dev];
    return 0;
}

// The fused add + RMS norm as two launches on `stream`: norm_rows_kernel
// writes h (when requested), u = (x + r) * g and each input row's inverse
// RMS into the work buffer (norm_work_bytes, a device address); the plain
// mat-vec multiplies u and scales each output by its row's value.  Outputs
// have the bits of the single-kernel form (same u, same statistic order,
// same scaling).  Arguments are validated by the caller.
int run_norm_two_launch(int t, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m,
                        uint32_t batch, const row_exact_strides_t &s, const Norm &nm, hipStream_t stream,
                        void *work) {
    float *u = (float *)work;
    double *inv = (double *)((uint8_t *)work + (((uint64_t)batch * m * k * sizeof(float) + 255) & ~255ull));
    NormArgs na;
    na.x = x;
    na.r = nm.r;
    na.g = nm.g;
    na.h = nm.h;
    na.u = u;
    na.inv = inv;
    na.xbs = s.x_batch_stride;
    na.xrs = s.x_row_stride;
    na.k = k;
    na.m = m;
    na.eps = nm.eps;
    MvLaunch L;
    int rc = plan_scaled_product(t, W, u, y, n, k, m, batch, s, inv, L);
    if (rc) return rc;
    hipError_t e = launch_norm_rows(na, batch, stream);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return enqueue_mv(L, stream);
}

}  // namespace

extern "C" {

int row_exact_mv(row_exact_weight_t wt, const void *W, const float *x, float *y, uint32_t n, uint32_t k, uint32_t m,
                 uint32_t batch, const row_exact_strides_t *strides, hipStream_t stream) {
    return run((int)wt, W, x, y, n, k, m, batch, strides, nullptr, stream);
}

int row_exact_mv_scheduled(row_exact_weight_t wt, const void *W, const float *x, float *y, uint32_t n, uint32_t k,
                           uint32_t m, uint32_t batch, const row_exact_strides_t *strides,
                           const row_exact_schedule_t *schedule, hipStream_t stream) {
    if (!schedule) {
        g_err.clear();
        return fail(ROW_EXACT_ESCHEDULE, "schedule must be non-NULL");
    }
    return run((int)wt, W, x, y, n, k, m, batch, strides, schedule, stream);
}

int row_exact_mv_gather(row_exact_weight_t wt, const void *W, uint32_t num_experts, const int32_t *expert_ids,
                        const float *x, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                        const row_exact_strides_t *strides, hipStream_t stream) {
    if (!expert_ids) {
        g_err.clear();
        return fail(ROW_EXACT_EARG, "expert_ids must be a non-NULL device pointer");
    }
    return run((int)wt, W, x, y, n, k, m, batch, strides, nullptr, stream, expert_ids, num_experts);
}

int row_exact_mv_add_rmsnorm(row_exact_weight_t wt, const void *W, const float *x, const float *r, const float *g,
                             float eps, float *h, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                             const row_exact_strides_t *strides, hipStream_t stream) {
    const Norm nm{r, g, h, eps};
    return run((int)wt, W, x, y, n, k, m, batch, strides, nullptr, stream, nullptr, 0, &nm);
}

int row_exact_mv_add_rmsnorm_ws(row_exact_weight_t wt, const void *W, const float *x, const float *r, const float *g,
                                float eps, float *h, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                                const row_exact_strides_t *strides, void *work, uint64_t work_bytes,
                                hipStream_t stream) {
    g_err.clear();
    int rc = check_shape((int)wt, n, k, m, batch);
    if (rc) return rc;
    if (!work) return fail(ROW_EXACT_EARG, "work must be a non-NULL device pointer");
    if ((uintptr_t)work % 16) return fail(ROW_EXACT_EALIGN, "work must sit on a 16-byte boundary");
    const uint64_t need = checked_norm_work_bytes(k, m, batch);
    if (!need) return ROW_EXACT_EEXTENT;
    if (work_bytes < need)
        return fail(ROW_EXACT_EARG, "work holds %llu bytes, the call needs %llu", (unsigned long long)work_bytes,
                    (unsigned long long)need);
    // work is written: it must not overlap any operand
    const row_exact_strides_t s = resolve_strides(strides, m, n, k);
    uint64_t wb = 0, xb = 0, yb = 0;
    rc = sizes((int)wt, n, k, m, batch, s, wb, xb, yb);
    if (rc) return rc;
    const uintptr_t wp = (uintptr_t)work;
    if (overlap(wp, need, (uintptr_t)W, wb) || overlap(wp, need, (uintptr_t)x, xb) ||
        overlap(wp, need, (uintptr_t)r, xb) || overlap(wp, need, (uintptr_t)y, yb) ||
        (h && overlap(wp, need, (uintptr_t)h, xb)) || (g && overlap(wp, need, (uintptr_t)g, 4ull * k)))
        return fail(ROW_EXACT_EALIAS, "work overlaps W, x, r, g, h or y");
    const Norm nm{r, g, h, eps};
    return run((int)wt, W, x, y, n, k, m, batch, strides, nullptr, stream, nullptr, 0, &nm, work);
}

int row_exact_mv_add_rmsnorm_noalloc(row_exact_weight_t wt, const void *W, const float *x, const float *r,
                                     const float *g, float eps, float *h, float *y, uint32_t n, uint32_t k, uint32_t m,
                                     uint32_t batch, const row_exact_strides_t *strides, hipStream_t stream) {
    g_err.clear();
    int rc = check_shape((int)wt, n, k, m, batch);
    if (rc) return rc;
    const uint64_t need = checked_norm_work_bytes(k, m, batch);
    if (!need) return ROW_EXACT_EEXTENT;
    if (need > ROW_EXACT_NOALLOC_SCRATCH_BYTES)
        return fail(ROW_EXACT_EEXTENT,
                    "the call needs %llu bytes of scratch (ROW_EXACT_NORM_WORK_BYTES), the allocation-free "
                    "scratch holds %u",
                    (unsigned long long)need, (unsigned)ROW_EXACT_NOALLOC_SCRATCH_BYTES);
    void *ptr = nullptr;
    rc = noalloc_scratch(ptr);
    if (rc) return rc;
    const Norm nm{r, g, h, eps};
    return run((int)wt, W, x, y, n, k, m, batch, strides, nullptr, stream, nullptr, 0, &nm, ptr);
}

int row_exact_mv_residual_rmsnorm_ws(row_exact_weight_t wt, const void *W, const float *h, const float *x,
                                     const float *w, const float *c, const float *w2, float eps, float eps2,
                                     float *hout, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                                     const row_exact_strides_t *strides, void *work, uint64_t work_bytes,
                                     hipStream_t stream) {
    g_err.clear();
    int rc = check_shape((int)wt, n, k, m, batch);
    if (rc) return rc;
    // the product's checks with x as its input (h and hout share x's layout)
    const row_exact_strides_t s = resolve_strides(strides, m, n, k);
    uint64_t wb = 0, xb = 0, yb = 0;
    rc = validate_mv((int)wt, W, x, y, n, k, m, batch, s, wb, xb, yb, nullptr, 0);
    if (rc) return rc;
    if (!h) return fail(ROW_EXACT_EARG, "h must be a non-NULL device pointer");
    if (!(eps >= 0.0f) || eps > 3.4e38f || !(eps2 >= 0.0f) || eps2 > 3.4e38f)
        return fail(ROW_EXACT_EARG, "eps and eps2 must be finite and >= 0");
    if ((uintptr_t)h % 16 || (uintptr_t)w % 16 || (uintptr_t)c % 16 || (uintptr_t)w2 % 16 || (uintptr_t)hout % 16)
        return fail(ROW_EXACT_EALIGN, "h, w, c, w2 and hout must be 16-byte aligned");
    const uint64_t vb = 4ull * k;
    const uintptr_t yp = (uintptr_t)y;
    if (overlap(yp, yb, (uintptr_t)h, xb) || (w && overlap(yp, yb, (uintptr_t)w, vb)) ||
        (c && overlap(yp, yb, (uintptr_t)c, vb)) || (w2 && overlap(yp, yb, (uintptr_t)w2, vb)))
        return fail(ROW_EXACT_EALIAS, "y overlaps h, w, c or w2");
    if (hout) {
        const uintptr_t hp = (uintptr_t)hout;
        if (overlap(hp, xb, (uintptr_t)x, xb) || overlap(hp, xb, (uintptr_t)W, wb) || overlap(hp, xb, yp, yb) ||
            (w && overlap(hp, xb, (uintptr_t)w, vb)) || (c && overlap(hp, xb, (uintptr_t)c, vb)) ||
            (w2 && overlap(hp, xb, (uintptr_t)w2, vb)) || (hout != h && overlap(hp, xb, (uintptr_t)h, xb)))
            return fail(ROW_EXACT_EALIAS, "hout overlaps x, W, y, w, c, w2 or (other than exactly) h");
    }
    if (!work) return fail(ROW_EXACT_EARG, "work must be a non-NULL device pointer");
    if ((uintptr_t)work % 16) return fail(ROW_EXACT_EALIGN, "work must sit on a 16-byte boundary");
    const uint64_t need = checked_norm_work_bytes(k, m, batch);
    if (!need) return ROW_EXACT_EEXTENT;
    if (work_bytes < need)
        return fail(ROW_EXACT_EARG, "work holds %llu bytes, the call needs %llu", (unsigned long long)work_bytes,
                    (unsigned long long)need);
    const uintptr_t wp = (uintptr_t)work;
    if (overlap(wp, need, (uintptr_t)W, wb) || overlap(wp, need, (uintptr_t)x, xb) ||
        overlap(wp, need, (uintptr_t)h, xb) || overlap(wp, need, yp, yb) ||
        (hout && overlap(wp, need, (uintptr_t)hout, xb)) || (w && overlap(wp, need, (uintptr_t)w, vb)) ||
        (c && overlap(wp, need, (uintptr_t)c, vb)) || (w2 && overlap(wp, need, (uintptr_t)w2, vb)))
        return fail(ROW_EXACT_EALIAS, "work overlaps W, x, h, hout, w, c, w2 or y");
    ResidualArgs ra;
    ra.h = h;
    ra.x = x;
    ra.w = w;
    ra.c = c;
    ra.w2 = w2;
    ra.hout = hout;
    ra.u = (float *)work;
    ra.inv = (double *)((uint8_t *)work + (((uint64_t)batch * m * k * sizeof(float) + 255) & ~255ull));
    ra.xbs = s.x_batch_stride;
    ra.xrs = s.x_row_stride;
    ra.k = k;
    ra.m = m;
    ra.eps = eps;
    ra.eps2 = eps2;
    MvLaunch L;
    rc = plan_scaled_product((int)wt, W, ra.u, y, n, k, m, batch, s, ra.inv, L);
    if (rc) return rc;
    hipError_t e = launch_residual_rows(ra, batch, stream);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return enqueue_mv(L, stream);
}

int row_exact_schedule(row_exact_weight_t wt, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                       row_exact_schedule_t *out) {
    g_err.clear();
    int rc = check_shape((int)wt, n, k, m, batch);
    if (rc) return rc;
    if (!out) return fail(ROW_EXACT_EARG, "out must be non-NULL");
    return default_schedule((int)wt, n, k, m, batch, *out);
}

uint64_t row_exact_row_bytes(row_exact_weight_t wt, uint32_t k) {
    return valid_type((int)wt) ? row_bytes_of((int)wt, k) : 0;
}

int row_exact_required_bytes(row_exact_weight_t wt, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                             const row_exact_strides_t *strides, uint64_t *w_bytes, uint64_t *x_bytes,
                             uint64_t *y_bytes) {
    g_err.clear();
    int rc = check_shape((int)wt, n, k, m, batch);
    if (rc) return rc;
    const row_exact_strides_t s = resolve_strides(strides, m, n, k);
    uint64_t wb, xb, yb;
    rc = sizes((int)wt, n, k, m, batch, s, wb, xb, yb);
    if (rc) return rc;
    if (w_bytes) *w_bytes = wb;
    if (x_bytes) *x_bytes = xb;
    if (y_bytes) *y_bytes = yb;
    return 0;
}

int row_exact_dequant(row_exact_weight_t wt, const void *W, float *out, uint32_t rows, uint32_t k,
                      hipStream_t stream) {
    g_err.clear();
    const int t = (int)wt;
    int rc = check_shape(t, rows, k, 1, 1);
    if (rc) return rc;
    if (!W || !out) return fail(ROW_EXACT_EARG, "W and out must be non-NULL device pointers");
    if ((uintptr_t)W % w_align(t) || (uintptr_t)out % 4)
        return fail(ROW_EXACT_EALIGN, "%s weights must sit on a %u-byte boundary and out on a 4-byte one",
                    type_name(t), w_align(t));
    const u128 wb = (u128)row_bytes_of(t, k) * rows;
    const u128 ob = (u128)rows * k * 4;
    if (wb >= ((u128)1 << 62) || ob >= ((u128)1 << 62))
        return fail(ROW_EXACT_EEXTENT, "W or out spans 2^62 bytes or more");
    if (overlap((uintptr_t)out, (uint64_t)ob, (uintptr_t)W, (uint64_t)wb))
        return fail(ROW_EXACT_EALIAS, "out overlaps the bytes of W");
    DqArgs a;
    a.W = (const uint8_t *)W;
    a.out = out;
    a.row_bytes = row_bytes_of(t, k);
    a.rows = rows;
    a.k = k;
    a.pieces = pieces_of(t, k);
    if ((uint64_t)a.rows * a.pieces / 256 >= 0x7fffffffull)
        return fail(ROW_EXACT_EEXTENT, "too many rows for one launch");
    hipError_t e = dq_launcher(t)(a, stream);
    if (e != hipSuccess) return fail(ROW_EXACT_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return 0;
}

const char *row_exact_last_error(void) { return g_err.c_str(); }

uint64_t row_exact_launch_count(void) { return g_launches.load(std::memory_order_relaxed); }

}  // extern "C"
