/*
 * row_exact_mv.h — C ABI of the row-exact few-row mat-vec for MI355X (gfx950).
 *
 *   y[b][j][i] = sum_kk W[b*n + i][kk] * x[b][j][kk]
 *
 * for 1 <= m <= 8 float32 input rows j, n weight rows i per batch, k inner
 * values, batch independent products; F16, Q8_0, Q4_K, Q6_K or Q5_0 weights,
 * float32 output.  Defined by mlx-native 0.18.0, src/ops/row_exact_matvec.rs:
 * module docs (the product, "Row exactness", "Batched / grouped products"),
 * RowExactWeight, RowExactMatvecShape, RowExactMatvecSchedule, validate(),
 * dispatch_row_exact_matvec and dispatch_row_exact_matvec_scheduled.
 * Dense float32 and bfloat16 weights (ROW_EXACT_F32, ROW_EXACT_BF16) carry
 * the same contract: nuvec-core 0.6.0, src/gpu.rs, the matmul routing of
 * "a few rows" to gemv_rows, whose every row has the bits of its one-row
 * product (the row-independence contract).
 *
 * Row exactness: output row j is bitwise identical whether it is computed with
 * m = 1 or as one row of any m <= 8, and identical across repeated calls.  The
 * only things that change the bits of an output are the reduction split and
 * the lanes per row (row_exact_schedule_t.k_split, .lanes_per_row), which the
 * library derives from the weight type, k and the rows n of one batch entry
 * (never from m or the batch); every other schedule field only packs work.
 *
 * Conventions for every entry point:
 *  - Pointers W, x, y, out are device pointers (HBM).  The caller owns them;
 *    the library keeps no reference after the call returns.
 *  - Calls only enqueue work on `stream` (a hipStream_t; 0 = the null stream)
 *    and never synchronize.  Results are defined once the stream reaches the
 *    enqueued kernels.  Inputs must not change until then.
 *  - Return 0 on success or a negative ROW_EXACT_E* code.  Every argument is
 *    checked before anything is enqueued: on error nothing is launched and y
 *    is untouched.  row_exact_last_error() then describes the failure.
 *  - Thread safety: calls may come from several host threads; the error text
 *    is per thread.
 */
#ifndef ROW_EXACT_MV_H
#define ROW_EXACT_MV_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight storage (RowExactWeight; same order as its index()).
 *  F16  : row-major [batch*n, k] IEEE half; k % 4 == 0; W 8-byte aligned.
 *  Q8_0 : row-major [batch*n, k/32] blocks of 34 bytes (f16 d, 32 int8);
 *         k % 32 == 0; W 2-byte aligned.
 *  Q4_K : row-major [batch*n, k/256] super-blocks of 144 bytes (f16 d, f16
 *         dmin, 12 bytes of 6-bit scales/mins, 128 bytes of nibbles);
 *         k % 256 == 0; W 16-byte aligned.
 *  Q6_K : row-major [batch*n, k/256] super-blocks of 210 bytes (128 bytes of
 *         low nibbles, 64 bytes of 2-bit highs, 16 int8 scales, f16 d);
 *         k % 256 == 0; W 2-byte aligned.
 *  Q5_0 : row-major [batch*n, k/32] blocks of 22 bytes (f16 d, 32 high bits,
 *         16 bytes of nibbles); k % 32 == 0; W 2-byte aligned.
 *  F32  : row-major [batch*n, k] IEEE single; k % 4 == 0; W 16-byte aligned.
 *  BF16 : row-major [batch*n, k] bfloat16 (the upper 16 bits of an IEEE
 *         single); k % 4 == 0; W 8-byte aligned.
 * Block layouts are those of the GGML types of the same names (the pages give
 * their byte sizes only).  Alignments are the page's validate() weight
 * alignments for its five types (8 / 2 / 16 / 2 / 2 bytes); no load reads a
 * byte before W or past its last row. */
typedef enum {
    ROW_EXACT_F16 = 0,
    ROW_EXACT_Q8_0 = 1,
    ROW_EXACT_Q4_K = 2,
    ROW_EXACT_Q6_K = 3,
    ROW_EXACT_Q5_0 = 4,
    ROW_EXACT_F32 = 5,
    ROW_EXACT_BF16 = 6
} row_exact_weight_t;

/* Maximum input rows per call (ROW_EXACT_MATVEC_MAX_ROWS). */
#define ROW_EXACT_MAX_ROWS 8

/* Element strides of x and y (RowExactMatvecShape).  x row/batch strides must
 * be multiples of 4; the x pointer 16-byte aligned; the y pointer 4-byte
 * aligned.  Passing NULL selects the contiguous layout x [m, k], y [m, n],
 * batch strides 0 (RowExactMatvecShape::contiguous).  The grouped token-major
 * layout of RowExactMatvecShape::grouped_token_major is
 * {groups*k, k, groups*n, n} with batch = groups. */
typedef struct {
    uint32_t x_row_stride;
    uint32_t x_batch_stride;
    uint32_t y_row_stride;
    uint32_t y_batch_stride;
} row_exact_strides_t;

/* Launch schedule (RowExactMatvecSchedule, re-planned for CDNA4 wave64).
 *  k_split              : numerics.  Waves whose partial sums form one output:
 *                         1, 2, 4 or 8.  With 1 the lanes_per_row lanes of
 *                         one wave split the row and a fixed permlane/DPP
 *                         tree adds them; with K > 1 (64 lanes per row) wave
 *                         s of K takes the row's wave steps s, s + K, s + 2K,
 *                         ..., each wave's lanes are added by the same tree,
 *                         and the K wave sums by the pairwise tree
 *                         ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)) cut to K terms.  row_exact_schedule() derives it
 *                         from (weight type, k, n): the largest power of two
 *                         <= min(1024 / n, 8, whole 64-piece wave steps of
 *                         a row); 1 for rows of at most 32 pieces or fewer
 *                         than 3 whole wave steps.  A pinned
 *                         schedule may carry any valid value (<= the row's
 *                         wave steps, dividing waves_per_workgroup); outputs
 *                         then follow that value, e.g. to keep the bits of
 *                         an unsharded product on a row shard.
 *  rows_per_wave        : packing.  Weight rows a wave streams at once
 *                         (each x value read from LDS serves all of them):
 *                         1, 2 or 4.
 *  waves_per_workgroup  : packing.  1..8 (64..512 threads).
 *  workgroups_per_batch : packing.  Workgroups per batch entry; the grid
 *                         holds workgroups_per_batch x batch of them,
 *                         flattened batch-fastest (workgroup w of entry b
 *                         is w * batch + b).
 *  k_chunk              : packing.  Input values per row staged in LDS per
 *                         pass; >= k means one pass.  Otherwise a multiple of
 *                         the weight type's wave step (512 values for F16 /
 *                         BF16, 256 for F32, 2048 for Q8_0 / Q5_0, 4096 for
 *                         Q4_K / Q6_K); with k_split > 1 a pass of fewer than
 *                         k_split wave steps leaves some waves idle.
 *  lanes_per_row        : numerics.  Lanes of a wave that split one row
 *                         (piece p of the row goes to lane p mod L; a wave
 *                         covers 64 / L rows side by side): 16, 32 or 64, or
 *                         0 for the value derived from (weight type, k,
 *                         k_split).  row_exact_schedule() gives the derived
 *                         value: 16 / 32 for rows of at most 16 / 32 pieces;
 *                         32 for rows of Q8_0, Q4_K, Q6_K and Q5_0 of 64 s + r
 *                         pieces, 0 < r <= 32, with k_split 1 and under 2^29
 *                         bytes (their last 64-lane step would be at most
 *                         half full); 64 otherwise.  A pinned value gives
 *                         that lane map's sums; below 64 it needs k_split 1
 *                         and (64 / L) * rows_per_wave * row bytes < 2^32.
 * Packing fields never change the bits of y. */
typedef struct {
    uint32_t k_split;
    uint32_t rows_per_wave;
    uint32_t waves_per_workgroup;
    uint32_t workgroups_per_batch;
    uint32_t k_chunk;
    uint32_t lanes_per_row;
} row_exact_schedule_t;

/* Error codes. */
#define ROW_EXACT_OK 0
#define ROW_EXACT_EARG (-1)      /* weight type, m, n, k, batch, k multiple, NULL pointer */
#define ROW_EXACT_EALIGN (-2)    /* W / x / y pointer alignment */
#define ROW_EXACT_ESTRIDE (-3)   /* x strides not multiples of 4 */
#define ROW_EXACT_EALIAS (-4)    /* output views overlap each other, W or x */
#define ROW_EXACT_EEXTENT (-5)   /* n >= 2^31, a row over 2^31 - 1 bytes, or sizes past 2^62 bytes */
#define ROW_EXACT_ESCHEDULE (-6) /* pinned schedule invalid, or over the device's limits */
#define ROW_EXACT_EHIP (-7)      /* HIP runtime error (device query or launch) */

/* Enqueue y[b, j, :] = W[b] . x[b, j, :] for b < batch, j < m with the
 * default schedule (dispatch_row_exact_matvec).
 *  wt      : weight storage, see row_exact_weight_t.
 *  W       : device pointer to batch*n rows of row_exact_row_bytes(wt, k)
 *            bytes; batch b starts at b * n * row_bytes.
 *  x       : device float32, element (b, j, kk) at b*x_batch_stride +
 *            j*x_row_stride + kk.
 *  y       : device float32, element (b, j, i) at b*y_batch_stride +
 *            j*y_row_stride + i.  Only these m*n*batch elements are written.
 *  n, k, m, batch : n, k, batch >= 1 (n < 2^31); 1 <= m <= 8.
 *  strides : NULL for contiguous; see row_exact_strides_t.
 *  stream  : HIP stream to enqueue on.
 * Errors: ROW_EXACT_EARG, EALIGN, ESTRIDE, EALIAS (the y layout must nest:
 * of the row and batch axes with more than one entry, the one with the larger
 * stride steps past the whole extent of the other, which steps past n values
 * -- the output-aliasing contract of validate(); y's bytes must not overlap
 * W's or x's), EEXTENT, EHIP. */
int row_exact_mv(row_exact_weight_t wt, const void *W, const float *x, float *y, uint32_t n, uint32_t k,
                 uint32_t m, uint32_t batch, const row_exact_strides_t *strides, hipStream_t stream);

/* As row_exact_mv with an explicit schedule
 * (dispatch_row_exact_matvec_scheduled).  Outputs are bitwise identical to
 * row_exact_mv's for every valid schedule with the derived k_split and
 * lanes_per_row: packing is inert; another k_split or lane count gives that
 * reduction's sums.  Extra error:
 * ROW_EXACT_ESCHEDULE (a field out of range, k_split not dividing the waves
 * or above the row's wave steps, k_chunk not a wave-step multiple,
 * lanes_per_row below 64 with k_split > 1 or rows too long for it, LDS need
 * above the device limit). */
int row_exact_mv_scheduled(row_exact_weight_t wt, const void *W, const float *x, float *y, uint32_t n,
                           uint32_t k, uint32_t m, uint32_t batch, const row_exact_strides_t *strides,
                           const row_exact_schedule_t *schedule, hipStream_t stream);

/* Gathered product for mixture-of-experts layers: batch entry b multiplies
 * by weight set expert_ids[b] of num_experts sets instead of set b,
 *   y[b, j, :] = W[expert_ids[b]] . x[b, j, :],
 * the per-expert weight selection of nuvec-core 0.6.0, src/gpu.rs (the
 * GatherQmm / GatherMm fast ops; tokens grouped by expert as its
 * SortedOffsets primitive groups them), here over the row-exact block types
 * and with the row-exact contract: every output has the bits row_exact_mv
 * gives for that batch entry with W advanced to its weight set.
 *  W          : device pointer to num_experts * n rows of
 *               row_exact_row_bytes(wt, k) bytes; set e starts at
 *               e * n * row_bytes.
 *  expert_ids : device int32[batch], 4-byte aligned, caller-owned, only read
 *               (by the kernel, so it may be written by earlier work on the
 *               same stream).  An id outside [0, num_experts) reads no
 *               weights and sets that batch entry's m*n outputs to NaN.
 *  x, y, n, k, m, batch, strides, stream : as row_exact_mv (a token routed
 *               to several experts can use x_batch_stride = 0).
 * Errors: as row_exact_mv, plus ROW_EXACT_EARG for NULL expert_ids or
 * num_experts == 0, ROW_EXACT_EALIGN for misaligned expert_ids, and
 * ROW_EXACT_EALIAS if y overlaps expert_ids[0 .. batch). */
int row_exact_mv_gather(row_exact_weight_t wt, const void *W, uint32_t num_experts, const int32_t *expert_ids,
                        const float *x, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                        const row_exact_strides_t *strides, hipStream_t stream);

/* The product with its input produced by a fused add + RMS normalisation:
 *   h[b, j, :] = x[b, j, :] + r[b, j, :]                       (float32 adds)
 *   x'[b, j, v] = h[b, j, v] / sqrt(mean_v h[b, j, v]^2 + eps) * g[v]
 *   y[b, j, :] = W[b] . x'[b, j, :]
 * (nuvec-core 0.6.0, src/gpu.rs, add_rms_norm / FastOp::AddRmsNorm: the sum
 * x + r and its RMS normalisation with weight g, the step that produces the
 * input of the next projection).  The mean is over the k values of each
 * input row; its sum of squares is taken in float64 in a fixed order.  The
 * normalisation is linear per row, so the product runs on u = h * g (float32)
 * and each output is scaled once by the row's inverse RMS (float64, one
 * rounding); y keeps the row-exact contract (bitwise the same for m = 1 and
 * every row of m <= 8, for every packing).  One kernel: every workgroup
 * forms the statistic of the rows it needs.
 *  x, r  : device float32, both in x's layout (strides as row_exact_mv).
 *  g     : device float32[k], or NULL for no weight (g = 1).
 *  eps   : finite, >= 0 (eps = 0 and an all-zero row give NaN outputs).
 *  h     : device float32 in x's layout receiving x + r, or NULL.  Written
 *          once (by one workgroup per batch entry); must not overlap x, r,
 *          g, W or y.
 *  r, g, h 16-byte aligned.  Other arguments as row_exact_mv.
 * Errors: as row_exact_mv, plus ROW_EXACT_EARG (NULL r, bad eps),
 * ROW_EXACT_EALIGN and ROW_EXACT_EALIAS for r, g and h. */
int row_exact_mv_add_rmsnorm(row_exact_weight_t wt, const void *W, const float *x, const float *r, const float *g,
                             float eps, float *h, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                             const row_exact_strides_t *strides, hipStream_t stream);

/* Bytes of the work buffer row_exact_mv_add_rmsnorm_ws needs: u (batch*m*k
 * floats, rounded up to 256 bytes), then batch*m doubles. */
#define ROW_EXACT_NORM_WORK_BYTES(k, m, batch)                                                                 \
    ((((uint64_t)(batch) * (m) * (k) * 4u + 255u) & ~(uint64_t)255u) + (uint64_t)(batch) * (m) * 8u)

/* row_exact_mv_add_rmsnorm as two launches on `stream`, with the same
 * results bit for bit: the add and the statistic in a kernel of their own
 * (writing h, u = h * g and each input row's inverse RMS into `work`), then
 * the plain mat-vec on u, every output scaled by its row's value.  Faster
 * from m = 4 on (the product keeps its staging of the input ahead of the
 * weights, and the statistic is formed once instead of in every
 * workgroup); one launch more.
 *  work       : device buffer of at least ROW_EXACT_NORM_WORK_BYTES(k, m,
 *               batch) bytes, 16-byte aligned, caller-owned, overwritten
 *               (its contents are undefined afterwards); must not overlap W,
 *               x, r, g, h or y, nor be in use by other work until the
 *               stream has passed this call.
 *  work_bytes : its size.
 * Other arguments as row_exact_mv_add_rmsnorm.  Errors: as
 * row_exact_mv_add_rmsnorm, plus ROW_EXACT_EARG (NULL work, work_bytes too
 * small), ROW_EXACT_EALIGN and ROW_EXACT_EALIAS for work, and
 * ROW_EXACT_EEXTENT when batch * m exceeds 2^31 - 1, when batch > 1 and
 * m * k exceeds 2^32 - 1 (the work buffer's batch stride), or when the work
 * buffer would span 2^62 bytes or more.  Both launches are planned before
 * the first is enqueued: a call that fails its checks enqueues nothing.  A
 * launch error of the second kernel leaves h written and y untouched. */
int row_exact_mv_add_rmsnorm_ws(row_exact_weight_t wt, const void *W, const float *x, const float *r, const float *g,
                                float eps, float *h, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                                const row_exact_strides_t *strides, void *work, uint64_t work_bytes,
                                hipStream_t stream);

/* The product whose input is a residual RMS normalisation (nuvec-core
 * 0.6.0, src/gpu.rs, residual_rms_norm: the residual stream plus the RMS
 * normalisation of a layer output, optionally scaled, and that sum's own
 * RMS normalisation for the next projection), as two launches on `stream`
 * with a caller's work buffer.  For every batch entry b and input row j,
 * over its k values:
 *   hs = (h + x / sqrt(mean(x^2) + eps) * w) * c
 *   y[b, j, :] = W[b] . (hs / sqrt(mean(hs^2) + eps2) * w2)
 * Reading of the page (its kernel is not shown): w, c, w2 are k-vectors
 * (NULL: 1, no scaling, 1); the first normalisation's value is rounded to
 * float32 once, the addition and the scaling are float32 operations; both
 * statistics are float64 sums in one fixed order.  The first kernel writes
 * hs to hout (NULL: not written), u = hs * w2 and each row's inverse RMS of
 * hs into `work`; the plain mat-vec then runs on u, every output scaled by
 * its row's value, so outputs are row-exact as row_exact_mv's.
 *  h, x       : device, the layout of x in row_exact_mv (strides), 16-byte
 *               aligned; h is the residual stream, x the layer output.
 *  w, c, w2   : device, k floats each, 16-byte aligned, or NULL.
 *  eps, eps2  : finite, >= 0.
 *  hout       : device, x's layout, 16-byte aligned, or NULL; may be h
 *               itself (updated in place) but must not overlap anything else.
 *  work       : as row_exact_mv_add_rmsnorm_ws (ROW_EXACT_NORM_WORK_BYTES).
 * Other arguments as row_exact_mv.  Errors: as row_exact_mv, plus
 * ROW_EXACT_EARG (NULL h or work, eps or eps2 out of range, work_bytes too
 * small), ROW_EXACT_EALIGN, ROW_EXACT_EALIAS (y against h, w, c, w2; hout
 * against everything but h; work against every operand) and
 * ROW_EXACT_EEXTENT as row_exact_mv_add_rmsnorm_ws.  A call that fails its
 * checks enqueues nothing (hout untouched). */
int row_exact_mv_residual_rmsnorm_ws(row_exact_weight_t wt, const void *W, const float *h, const float *x,
                                     const float *w, const float *c, const float *w2, float eps, float eps2,
                                     float *hout, float *y, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                                     const row_exact_strides_t *strides, void *work, uint64_t work_bytes,
                                     hipStream_t stream);

/* Bytes of the scratch array behind row_exact_mv_add_rmsnorm_noalloc, per
 * GPU: it serves calls whose ROW_EXACT_NORM_WORK_BYTES(k, m, batch) is at
 * most this. */
#define ROW_EXACT_NOALLOC_SCRATCH_BYTES (4u << 20)

/* row_exact_mv_add_rmsnorm_ws for callers that cannot allocate device
 * memory, not even a work buffer (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same two kernels and
 * the same results bit for bit, the work buffer being an array of
 * ROW_EXACT_NOALLOC_SCRATCH_BYTES per GPU that the library holds from its
 * first call on that GPU until the process ends.  Allocates nothing.  Every
 * call on a GPU uses that GPU's one array: calls that overlap on one GPU
 * (other streams, other host threads) race and give undefined results;
 * calls in order on one stream are safe.  The array keeps the last call's
 * contents; nothing in it needs clearing (each call writes all it reads).
 * Arguments as row_exact_mv_add_rmsnorm.  Errors: as
 * row_exact_mv_add_rmsnorm, plus ROW_EXACT_EEXTENT when
 * ROW_EXACT_NORM_WORK_BYTES(k, m, batch) exceeds the array, ROW_EXACT_EHIP
 * when the array's device address cannot be had. */
int row_exact_mv_add_rmsnorm_noalloc(row_exact_weight_t wt, const void *W, const float *x, const float *r,
                                     const float *g, float eps, float *h, float *y, uint32_t n, uint32_t k,
                                     uint32_t m, uint32_t batch, const row_exact_strides_t *strides,
                                     hipStream_t stream);

/* Default schedule for a shape (RowExactMatvecSchedule::for_device).  k_split
 * depends on (wt, k, n) only, lanes_per_row on (wt, k, k_split); the packing
 * fields may depend on every argument and on the current device.  Unlike the page's query (weight, rows, k), this
 * one takes m: the packing is chosen per m because the m-row kernel's
 * register and LDS needs decide how many rows a wave and how many workgroups
 * a CU can hold.  m never reaches k_split or lanes_per_row, so outputs stay
 * row-exact.
 * Writes *out; errors: EARG, EHIP. */
int row_exact_schedule(row_exact_weight_t wt, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                       row_exact_schedule_t *out);

/* Bytes per weight row of k values (RowExactWeight::row_bytes):
 * F16 2k; Q8_0 34*(k/32); Q4_K 144*(k/256); Q6_K 210*(k/256); Q5_0 22*(k/32);
 * F32 4k; BF16 2k.
 * Returns 0 for an unknown type. */
uint64_t row_exact_row_bytes(row_exact_weight_t wt, uint32_t k);

/* Bytes the product reads or writes (validate()'s size checks; strided_extent
 * = last element + 1): *w_bytes = row_bytes * n * batch;
 * *x_bytes = 4 * ((batch-1)*x_batch_stride + (m-1)*x_row_stride + k);
 * *y_bytes = 4 * ((batch-1)*y_batch_stride + (m-1)*y_row_stride + n).
 * strides NULL = contiguous.  Any output pointer may be NULL.
 * Errors: EARG, EEXTENT. */
int row_exact_required_bytes(row_exact_weight_t wt, uint32_t n, uint32_t k, uint32_t m, uint32_t batch,
                             const row_exact_strides_t *strides, uint64_t *w_bytes, uint64_t *x_bytes,
                             uint64_t *y_bytes);

/* Enqueue out[r*k + v] = float32 value of weight v of row r, for rows
 * consecutive weight rows at W: the weights the product multiplies
 * (RowExactWeight's storage formats with the block sizes of the page's block
 * constants, decoded exactly; Q4_K's d*sc*q - dmin*mn rounded once).  Uses
 * the same device block loads and decoders as the mat-vec, so the values can
 * be compared bit for bit with an independent decode.  W aligned as for
 * row_exact_mv; out 4-byte aligned and not overlapping W.
 * Errors: EARG, EALIGN, EALIAS, EEXTENT, EHIP. */
int row_exact_dequant(row_exact_weight_t wt, const void *W, float *out, uint32_t rows, uint32_t k,
                      hipStream_t stream);

/* Text of the calling thread's last error ("" if none), the counterpart of
 * the page's invalid() error (an InvalidArgument message with the op's name
 * as prefix): prefixed "row_exact_mv: ".  Cleared by each call and set when
 * the call fails; the pointer stays valid until the thread's next call. */
const char *row_exact_last_error(void);

/* Number of kernels this process has enqueued through the library. */
uint64_t row_exact_launch_count(void);

#ifdef __cplusplus
}
#endif

#endif /* ROW_EXACT_MV_H */
