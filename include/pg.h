/*
 * pg.h — packed-weight products for MI355X (gfx950): the C ABI of libpg.
 *
 * The library evaluates the data-parallel hot path of a portable LLM
 * inference runtime (cortiq-engine's GPU frames, as described on its docs.rs
 * source pages): products of packed weights with f32 activations, the decode
 * matrix-vector product at one position, the batched prefill product over up
 * to 64 positions with every weight read once per pass, the fused residual
 * add + RMSNorm and relu^2 stages around them, and the routed-MoE step that
 * groups (position, slot) pairs per expert so each selected expert is
 * streamed once per pass.
 *
 * Conventions shared by every call
 *  - Pointers named as tensors are DEVICE pointers owned by the caller.  The
 *    library never allocates or frees, and synchronizes only in
 *    decode_frame_q8_status (a status query); every other call enqueues
 *    kernels on `stream` (a hipStream_t; NULL is the null stream) and returns.
 *  - Return value: PG_OK, or a negative PG_E* code.  On any error other than
 *    PG_ELAUNCH nothing has been enqueued.  PG_ELAUNCH reports a failed kernel
 *    launch (hipGetLastError after the launch); faults during execution show
 *    up at the caller's next synchronization of `stream`.
 *  - q8 weight format ("q8 block"): q is int8 [rows][cols] row-major; every
 *    32 consecutive columns of a row form a block with one f32 scale and one
 *    f32 bias, stored [rows][cols/32] row-major; the weight is
 *        w[r][c] = scale[r][c/32] * q[r][c] + bias[r][c/32].
 *    cols % 32 == 0.  The pages' own int8 format (q8_2f: int8 body, f16 row
 *    scales, f16 column field; nemotron_prefill.rs `pb_q8_bank`,
 *    gemma_batch.rs `q8_2f_mm_r2`) folds its factors the same way: the column
 *    factor into the staged activations, the row factor onto the finished sum.
 *  - act: 0 = none, 1 = relu^2, y = max(y, 0)^2 on the finished product
 *    (nemotron_prefill.rs, `pb_relu2` and `PqP.act`).
 *  - Alignment: q, scale, bias, activation and output pointers must be
 *    16-byte aligned (the kernels move 16 bytes per lane); PG_EINVAL if not.
 *  - Calls are stateless and thread-safe; calls that share a workspace or
 *    output buffer and overlap on different streams race.
 */
#ifndef PG_H
#define PG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *pg_stream_t; /* a hipStream_t */

enum {
    PG_OK = 0,
    PG_EINVAL = -1,        /* null pointer, non-positive size, misalignment, aliasing */
    PG_EUNSUPPORTED = -2,  /* shape outside what the kernels handle (listed per call) */
    PG_ELAUNCH = -3,       /* a kernel launch failed */
    PG_EWORKSPACE = -4,    /* workspace pointer NULL or smaller than the query returns */
    PG_ETIMEOUT = -5       /* a device-wide barrier wait gave up (decode_frame_q8_status) */
};

/* A q8-block matrix on the device (the format above): q [rows][cols] int8,
 * scale and bias [rows][cols/32] f32. */
typedef struct pg_q8 {
    const int8_t *q;
    const float *scale;
    const float *bias;
    int32_t rows;
    int32_t cols;
} pg_q8;

/* Human-readable text of a PG_* code (static storage). */
const char *pg_strerror(int code);

/* Library version string, e.g. "0.1.0 gfx950". */
const char *pg_version(void);

/*
 * gemv_q8 — decode matrix-vector product at one position:
 *     y[r] = act( sum_c w[r][c] * x[c] ),  r < rows,
 * with w the q8-block weight.  The weight stays packed in HBM and is decoded
 * in registers as it streams (embryo_wide.wgsl, header comment: matrices stay
 * in the file's form on the device, read in 16-byte loads).
 *   q [rows][cols] int8, scale/bias [rows][cols/32] f32, x [cols] f32,
 *   y [rows] f32 (written; must not overlap x).
 * PG_EUNSUPPORTED: cols % 32 != 0, cols > 32768.
 */
int gemv_q8(const int8_t *q, const float *scale, const float *bias, int32_t rows,
            int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream);

/*
 * gemv_q8_addnorm — the residual add + RMSNorm that precedes a projection,
 * fused into the decode product (nemotron_prefill.rs `pb_add_rms` with
 * add = 1 feeding the next matrix stage; embryo_wide.wgsl header comment:
 * stages are fused because every dispatch boundary costs microseconds):
 *     h'[c]  = h[c] + delta[c]                       (delta NULL: h' = h)
 *     x[c]   = w[c] * h'[c] / sqrt( (1/cols) sum_c h'[c]^2 + eps )
 *     y[r]   = act( sum_c wq[r][c] * x[c] ),  r < rows, wq the q8-block weight
 * Each workgroup stages w * h' together with sum h'^2 (the same order in
 * every workgroup) and multiplies its finished dot products by the scalar
 * 1/rms, so no separate pass over the activations is made.
 *   q/scale/bias as gemv_q8 (cols = the hidden size); h, delta, w [cols] f32;
 *   h_out [cols] f32 receives h' (NULL: not written); x_out [cols] f32
 *   receives x (NULL: not written); y [rows] f32.  h_out, x_out and y must not
 *   overlap each other or h, delta, w (PG_EINVAL): workgroups read the whole
 *   of h, delta and w while others write.
 * PG_EINVAL also for eps < 0 or NaN.  PG_EUNSUPPORTED: cols % 32 != 0, cols > 32768.
 */
int gemv_q8_addnorm(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                    int32_t cols, const float *h, const float *delta, const float *w, float eps,
                    float *h_out, float *x_out, float *y, int32_t act, pg_stream_t stream);

/*
 * gemv_q8_residual / gemv_q8_normed — the residual add + RMSNorm between two
 * decode products, split so that neither call makes an extra pass over the
 * activations (nemotron_prefill.rs `pb_add_rms`, add = 1, between the matrix
 * stages; embryo_wide.wgsl header comment on fusing stages to save dispatch
 * boundaries):
 *   gemv_q8_residual: y[r] = act( sum_c wq[r][c] * x[c] ), r < rows, and for
 *     r < hidden:  h_out[r] = h[r] + y[r],   xw[r] = w[r] * h_out[r],
 *     and parts[0 .. gemv_q8_norm_parts(hidden)) = sums of h_out[r]^2 over a
 *     fixed partition of [0, hidden) into consecutive row ranges (f32).
 *   gemv_q8_normed: y[r] = act( (sum_c wq[r][c] * xw[c]) / sqrt( sum_j parts[j] / cols + eps ) ),
 *     j < gemv_q8_norm_parts(cols), the parts summed in the same fixed order
 *     by every workgroup.  With xw and parts from gemv_q8_residual (cols =
 *     hidden) this is the product of W with rmsnorm(h + y[:hidden]) * w.
 *   x [cols] f32; y [rows] f32; h, w [hidden] f32 (hidden <= rows); h_out
 *   [hidden] f32 (NULL: not written; h_out == h updates the residual in
 *   place); xw [hidden] f32; parts [gemv_q8_norm_parts(hidden)] f32.  Outputs
 *   may not overlap each other or the inputs (other than h_out == h): PG_EINVAL.
 * PG_EINVAL also for eps < 0 or NaN.  PG_EUNSUPPORTED: cols % 32 != 0, cols > 32768.
 */
int32_t gemv_q8_norm_parts(int32_t hidden);
int gemv_q8_residual(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                     int32_t cols, const float *x, float *y, int32_t act, const float *h,
                     const float *w, int32_t hidden, float *h_out, float *xw, float *parts,
                     pg_stream_t stream);
int gemv_q8_normed(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                   int32_t cols, const float *xw, const float *parts, float eps, float *y,
                   int32_t act, pg_stream_t stream);

/*
 * gemv_f16 — the same product with binary16 weights, f32 accumulation:
 *     y[r] = act( sum_c f16(w[r][c]) * x[c] )
 * (embryo_wide.wgsl, header comment: f16 matrices are read in place.)
 *   w [rows][cols] binary16 bits, x [cols] f32, y [rows] f32.
 * PG_EUNSUPPORTED: cols % 8 != 0, cols > 32768.
 */
int gemv_f16(const uint16_t *w, int32_t rows, int32_t cols, const float *x, float *y,
             int32_t act, pg_stream_t stream);

/*
 * gemv_q82 — the decode product on the pages' own int8 format, q8_2f
 * (gemma_batch.rs, `q8_2f_mm_r2` doc comment and epilogue; nemotron_prefill.rs,
 * the q8_2f expert-bank payload): an int8 body, one binary16 scale per row and
 * one binary16 factor per column (the column field),
 *     y[r] = act( f16(row_scale[r]) * sum_c q[r][c] * (f16(col_field[c]) * x[c]) ).
 * The column field multiplies the activation once (f32) before the product, the
 * row scale the finished f32 sum.
 *   q [rows][cols] int8 row-major (16-byte aligned), row_scale [rows] and
 *   col_field [cols] binary16 bits (col_field 8-byte aligned), x [cols] f32
 *   (16-byte aligned), y [rows] f32 (must not overlap x).  The pages keep the
 *   three parts in one buffer in this order; here they are separate pointers.
 * PG_EUNSUPPORTED: cols % 16 != 0, cols > 32768.
 */
int gemv_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field, int32_t rows,
             int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream);

/*
 * gemv_q4tp — the decode product on the pages' 4-bit format, q4tp
 * (nemotron_prefill.rs, the q4tp expert bank `pb_q4_bank` and its nibble and
 * code readers).  Per row r: 4-bit codes, two a byte (column c in the low half
 * of byte c/2 when c is even, the high half when odd), the weight integer being
 * the code minus 8; a 32-bit parameter word holding binary16 base (low half)
 * and step (high half); a 5-bit log-scale code per 32-column group g, least
 * significant bit first at bit 5g of the row's code bytes:
 *     y[r] = act( sum_g 2^(base_r + code_{r,g} * step_r) * sum_{c in g} (nib_r(c) - 8) * x[c] ).
 *   nib [rows][cols/2] bytes (16-byte aligned), params [rows] uint32 (4-byte
 *   aligned), codes [rows][(5 * cols/32 + 7) / 8] bytes, x [cols] f32 (16-byte
 *   aligned), y [rows] f32 (must not overlap x).  The pages keep the three
 *   parts of an expert in one buffer in this order; here they are separate.
 * Arithmetic: the group scale is exp2 in f32 of base + code * step (exact in
 * f32); each group's sum is formed in f32 as sum nib * x - 8 * sum x.
 * PG_EUNSUPPORTED: cols % 32 != 0, cols > 32768.
 */
int gemv_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t rows,
              int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream);

/*
 * prefill_gemm_q4tp — the batched prefill product on the q4tp format
 * (nemotron_prefill.rs, `pb_q4_bank` and its nibble and code readers, applied
 * to one pass of n <= 64 positions with every weight read once):
 *     Y[b][r] = act( sum_c 2^(base_r + code_{r,c/32} step_r) (nib_r(c) - 8) X[b][c] )
 * with the layout of gemv_q4tp (nibbles, parameter words, 5-bit group codes).
 * On the bf16 matrix cores: the nibble n enters as itself (exact), X as bf16
 * hi + lo, each 32-column group's sum scaled by its group scale (hardware
 * exp2 of fma(code, step, base) in f32, as gemv_q4tp), and the - 8 through a
 * contraction of -8 * scale with the groups' sums of X.
 *   nib [rows][cols/2] (16-byte aligned), params [rows] u32 and codes
 *   [rows][ceil(5 cols/32 / 8)] (4-byte aligned), X [n][cols] f32, Y [n][rows]
 *   f32 (16-byte aligned, not overlapping X or the workspace), act 0 or 1;
 *   workspace: prefill_gemm_q8_workspace_bytes(rows, cols, n) bytes.
 * PG_EUNSUPPORTED: cols % 32 != 0, n > 64.  PG_EINVAL: null or misaligned
 *   pointers, rows, cols or n < 1, act not 0/1, overlaps.  PG_EWORKSPACE.
 */
int prefill_gemm_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t rows,
                      int32_t cols, const float *X, int32_t n, float *Y, int32_t act, void *workspace,
                      size_t workspace_bytes, pg_stream_t stream);

/*
 * argmax_rows — the token chosen at each position (nemotron_prefill.rs,
 * `pb_argmax`, the verify passes):
 *     ids[b] = the smallest i with logits[b][i] the largest of row b,
 * counting only logits above -3.0e38 (NaN never counts; a row with no such
 * logit gives 0).  Comparisons in f32.
 *   logits [n][vocab] f32 (4-byte aligned; 16-byte alignment and vocab % 4 == 0
 *   take the vector path), ids [n] uint32 (must not overlap logits).
 * PG_EINVAL: n < 1, vocab < 1, misaligned or overlapping pointers.
 */
int argmax_rows(const float *logits, int32_t n, int32_t vocab, uint32_t *ids, pg_stream_t stream);

/*
 * prefill_gemm_q8 — batched prefill product over one pass of n positions,
 * every weight read from HBM once per pass (nemotron_prefill.rs, module doc:
 * up to PB_MAX = 64 positions a pass; gemma_batch.rs, `encode_q82_mm`:
 * y[nb][rows] = x[nb][cols] . W^T):
 *     Y[b][r] = act( sum_c w[r][c] * X[b][c] ),  b < n, r < rows.
 *   X [n][cols] f32, Y [n][rows] f32 (must not overlap X or the workspace).
 *   workspace: device scratch of at least
 *   prefill_gemm_q8_workspace_bytes(rows, cols, n) bytes (contents on entry
 *   do not matter; the call overwrites them).
 * Arithmetic: the weights enter the matrix cores as exact bf16 integers, the
 * activations as an exact-to-2^-17 bf16 hi+lo pair, products accumulate in
 * f32 per 32-column block, the block scale multiplies each block sum in f32
 * and the bias term sum_blk bias[r][blk] * (sum_{c in blk} X[b][c]) is added.
 * Where the K range is split over workgroups, the partial sums are added in
 * split order (the result does not depend on timing).
 * PG_EUNSUPPORTED: cols % 32 != 0, n < 1 or n > 64.
 */
int prefill_gemm_q8(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                    int32_t cols, const float *X, int32_t n, float *Y, int32_t act,
                    void *workspace, size_t workspace_bytes, pg_stream_t stream);
size_t prefill_gemm_q8_workspace_bytes(int32_t rows, int32_t cols, int32_t n);

/*
 * prefill_gemm_q8_noalloc — prefill_gemm_q8 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same product, the same kernels and bits, with
 * no workspace argument.  Its scratch is a fixed device array of
 * PG_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library, one per device, held
 * until the process ends; the call allocates and frees nothing.  Every call on
 * one device shares that device's array, so calls that overlap in time on one
 * device (two streams, two host threads) race: serialize them.
 *   Arguments, layouts and codes as prefill_gemm_q8.
 *   PG_EUNSUPPORTED also when prefill_gemm_q8_workspace_bytes(rows, cols, n)
 *   exceeds PG_NOALLOC_SCRATCH_BYTES (nothing enqueued); every product of the
 *   hidden-4096 layer frame (up to 32000 x 4096 and 4096 x 14336) fits at n = 64.
 *   PG_ELAUNCH if the array's device address cannot be obtained.
 */
#define PG_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int prefill_gemm_q8_noalloc(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                            int32_t cols, const float *X, int32_t n, float *Y, int32_t act,
                            pg_stream_t stream);

/*
 * prefill_gemm_q82 — the batched prefill product on the q8_2f format
 * (gemma_batch.rs, `encode_q82_mm` and the `q8_2f_mm_r2` epilogue: the column
 * field scales the activation, the row scale the finished dot product):
 *     Y[b][r] = act( f16(row_scale[r]) * sum_c q[r][c] * (f16(col_field[c]) * X[b][c]) ),
 *     b < n, r < rows.
 *   q [rows][cols] int8 row-major (16-byte aligned); row_scale [rows] and
 *   col_field [cols] binary16 bits; X [n][cols] f32; Y [n][rows] f32 (must not
 *   overlap X or the workspace); workspace as prefill_gemm_q8
 *   (prefill_gemm_q8_workspace_bytes(rows, cols, n), contents on entry do not
 *   matter).
 * Arithmetic: f16(col_field[c]) * X[b][c] is formed in f32 and enters the
 * matrix cores as an exact-to-2^-17 bf16 hi+lo pair, the int8 body as exact
 * bf16 integers; the products accumulate in f32 (split partials added in split
 * order) and the row scale multiplies the f32 total.
 * PG_EUNSUPPORTED: cols % 32 != 0, n < 1 or n > 64.
 */
int prefill_gemm_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field,
                     int32_t rows, int32_t cols, const float *X, int32_t n, float *Y, int32_t act,
                     void *workspace, size_t workspace_bytes, pg_stream_t stream);

/*
 * prefill_gemm_q8_addnorm — prefill_gemm_q8 on rmsnorm(H + delta) * w, the
 * add + norm done per position while the activations are staged for the
 * matrix cores (nemotron_prefill.rs `pb_add_rms`, add = 1, then the product):
 *     H'[b][c] = H[b][c] + delta[b * delta_stride + c]   (delta NULL: H' = H)
 *     X[b][c]  = w[c] * H'[b][c] / sqrt( (1/cols) sum_c H'[b][c]^2 + eps )
 *     Y[b][r]  = act( sum_c wq[r][c] * X[b][c] ),  b < n, r < rows
 *   H [n][cols] f32; delta rows delta_stride floats apart (delta_stride >=
 *   cols, a multiple of 4); w [cols] f32; H_out [n][cols] receives H' (NULL:
 *   not written; H_out == H updates the residual in place); X_out [n][cols]
 *   receives X (NULL: not written); Y [n][rows]; workspace as prefill_gemm_q8
 *   (prefill_gemm_q8_workspace_bytes(rows, cols, n)).  Other overlaps among
 *   H_out, X_out, H, delta, w, Y and the workspace: PG_EINVAL.
 * Arithmetic of the product as prefill_gemm_q8.
 * PG_EUNSUPPORTED: cols % 32 != 0, cols > 16384, n < 1 or n > 64.
 */
int prefill_gemm_q8_addnorm(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                            int32_t cols, const float *H, const float *delta, int32_t delta_stride,
                            const float *w, float eps, int32_t n, float *H_out, float *X_out,
                            float *Y, int32_t act, void *workspace, size_t workspace_bytes,
                            pg_stream_t stream);

/*
 * decode_frame_q8 — the whole q8 decode layer frame at one position in ONE
 * launch (embryo_wide.wgsl, header comment: the token frame fuses its stages
 * because each dispatch boundary costs microseconds; nemotron_prefill.rs
 * `pb_add_rms`, add = 1, between the matrix stages; `pb_relu2` on the up
 * product):
 *     qkv    = Wqkv x0                       [rows_qkv], rows_qkv >= H
 *     h1     = h + qkv[:H];   x1 = w1 * h1 / sqrt(mean(h1^2) + eps)
 *     u      = relu^2(Wup x1)                [I]
 *     d      = Wdown u                       [H]
 *     h2     = h1 + d;        x2 = w2 * h2 / sqrt(mean(h2^2) + eps)
 *     logits = Whead x2                      [V]
 *     h     <- h2  (in place)
 * with H = qkv_w->cols = up_w->cols = head_w->cols = down_w->rows and
 * I = up_w->rows = down_w->cols.  One workgroup per compute unit runs the
 * four products on its share of each matrix's rows, with a device-wide
 * barrier between products; each weight byte is read once.  The barrier
 * needs every workgroup resident at once: the launch takes the whole device
 * (one workgroup per compute unit), so work on other streams that holds
 * compute units for the length of the launch delays it.  Barrier waits are
 * bounded (about a second) instead of hanging, and count themselves
 * (below).  The call may be captured into a graph.  The mean of squares is
 * summed in one fixed order, the same for every launch and every row.
 *   x0 [H], h [H] in/out, w1, w2 [H], qkv [rows_qkv], u [I], d [H],
 *   logits [V]: f32 device vectors, 16-byte aligned, not overlapping.
 *   workspace: at least decode_frame_q8_workspace_bytes(H, I) bytes, set up
 *   once by decode_frame_q8_workspace_init before its first use (it holds
 *   the barrier counters, a launch counter, w * h and the norm sums).  The
 *   32-bit word at byte offset 8 counts barrier waits that gave up; non-zero
 *   means a launch's outputs are not to be trusted: decode_frame_q8_status
 *   reports it.  Launches that share a workspace must not overlap (same
 *   stream, or ordered streams).
 * PG_EUNSUPPORTED: a cols % 1024 != 0 or > 16384, a matrix of 2^31 or more
 *   bytes, or one with more than about 2047 rows per compute unit.
 *   PG_EINVAL: shapes that do not chain as above, null or misaligned
 *   pointers, eps < 0 or NaN.  PG_EWORKSPACE: workspace missing or small.
 */
size_t decode_frame_q8_workspace_bytes(int32_t hidden, int32_t inter);
int decode_frame_q8_workspace_init(void *workspace, size_t workspace_bytes, pg_stream_t stream);
/* decode_frame_q8_status — waits for `stream`, then returns PG_ETIMEOUT if any
 * barrier wait of the launches on this workspace since its init gave up (their
 * outputs are not trustworthy), else PG_OK.  The one call here that blocks the
 * host.  PG_EWORKSPACE: workspace NULL, small or misaligned; PG_ELAUNCH: the
 * copy or the wait failed. */
int decode_frame_q8_status(const void *workspace, size_t workspace_bytes, pg_stream_t stream);
int decode_frame_q8(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                    const float *w1, const float *w2, float eps, const float *x0, float *h, float *qkv,
                    float *u, float *d, float *logits, void *workspace, size_t workspace_bytes,
                    pg_stream_t stream);

/*
 * prefill_frame_q8 — the q8 layer frame over one prefill pass of n <= 64
 * positions, every weight read once (nemotron_prefill.rs, module doc: a pass
 * of up to PB_MAX = 64 positions; `pb_add_rms`, add = 1, between the matrix
 * stages; `pb_relu2` on the up product), per position b:
 *     qkv[b]    = Wqkv X0[b]
 *     h1        = H[b] + qkv[b][:H];   x1 = w1 * h1 / sqrt(mean(h1^2) + eps)
 *     u[b]      = relu^2(Wup x1)
 *     d[b]      = Wdown u[b]
 *     h2        = h1 + d[b];           x2 = w2 * h2 / sqrt(mean(h2^2) + eps)
 *     logits[b] = Whead x2
 *     H[b]     <- h2  (in place)
 * with H = qkv_w->cols = up_w->cols = head_w->cols = down_w->rows and
 * I = up_w->rows = down_w->cols.  Five launches: the staging of X0, then the
 * four matrix-core passes; each pass finishes the add + RMSNorm work around
 * it in its epilogue (the residual add, the staging of w * h' for the next
 * product, per-position sums of squares) and the next pass multiplies its
 * finished sums by the position's 1 / rms, so the norm needs no pass of its
 * own.  Split-K partial sums are added in split order inside the passes.
 * Arithmetic of each product as prefill_gemm_q8 (the product of a normed
 * input runs on w * h' and is scaled afterwards); sums of squares and split
 * partials are added in fixed orders, so results repeat bit for bit.
 *   X0, H [n][H]; w1, w2 [H]; qkv [n][rows_qkv]; u [n][I]; d [n][H];
 *   logits [n][V]: f32 device arrays, 16-byte aligned, not overlapping each
 *   other or the workspace.  workspace: prefill_frame_q8_workspace_bytes(H,
 *   rows_qkv, I, V, n) bytes (contents on entry do not matter).
 * PG_EUNSUPPORTED: a cols % 32 != 0 (so H and I are multiples of 32), n > 64.
 *   PG_EINVAL: shapes that do not chain as above, null or misaligned pointers, n < 1, eps < 0 or
 *   NaN.  PG_EWORKSPACE: workspace missing or small.
 */
size_t prefill_frame_q8_workspace_bytes(int32_t hidden, int32_t qkv_rows, int32_t inter, int32_t vocab,
                                        int32_t n);
int prefill_frame_q8(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                     const float *w1, const float *w2, float eps, const float *X0, float *H, int32_t n,
                     float *qkv, float *u, float *d, float *logits, void *workspace, size_t workspace_bytes,
                     pg_stream_t stream);

/*
 * prefill_frame_q8_meta — prefill_frame_q8 with the pass size on the device,
 * so that one recorded launch sequence (a HIP graph) serves every pass of a
 * prompt (nemotron_prefill.rs, module doc: the bind groups are built once and
 * the pass's n and pos0 sit in the `Meta` uniform buffer):
 *     meta[0] = n (1..64), meta[1] = pos0 (>= 0), read by the kernels at launch;
 * the pass works on rows pos0 .. pos0 + n - 1 of X0 and H and writes the same
 * rows of qkv, u, d and logits, each buffer holding rows_total rows:
 *   X0, H [rows_total][H]; qkv [rows_total][rows_qkv]; u [rows_total][I];
 *   d [rows_total][H]; logits [rows_total][V]; meta: 2 int32 in device memory
 *   (8-byte aligned, not overlapping the rest).  The caller may change meta
 *   between launches (for instance between replays of a graph that holds
 *   this call); a pass with n outside 1..64, pos0 < 0 or pos0 + n > rows_total
 *   does nothing (no output is written).  Arithmetic, order and results are
 *   those of prefill_frame_q8 on the same n positions, bit for bit.
 *   workspace: prefill_frame_q8_workspace_bytes(H, rows_qkv, I, V, 64) bytes.
 * Codes as prefill_frame_q8 (rows_total < 1: PG_EINVAL; meta NULL: PG_EINVAL).
 */
int prefill_frame_q8_meta(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                          const float *w1, const float *w2, float eps, const float *X0, float *H,
                          int32_t rows_total, const int32_t *meta, float *qkv, float *u, float *d, float *logits,
                          void *workspace, size_t workspace_bytes, pg_stream_t stream);

/*
 * add_rmsnorm — fused residual add + RMSNorm, per position b < n
 * (nemotron_prefill.rs `pb_add_rms` with add = 1; gemma_batch.rs
 * `g4_add_norm_b` without the layer scalar):
 *     h[b][i] += delta[b * delta_stride + i]        (skipped if delta is NULL)
 *     out[b][i] = w[i] * h[b][i] / sqrt( (1/hidden) sum_i h[b][i]^2 + eps )
 *   h [n][hidden] f32, updated in place; delta rows delta_stride floats apart
 *   (delta_stride >= hidden; it lets a wider product output, e.g. the first
 *   `hidden` columns of a [n][6144] QKV result, be added in place);
 *   w [hidden] f32; out [n][hidden] f32 (must not overlap h or delta).
 * PG_EUNSUPPORTED: hidden % 4 != 0, hidden > 16384, delta_stride % 4 != 0.
 */
int add_rmsnorm(float *h, const float *delta, int32_t delta_stride, const float *w, float eps,
                int32_t hidden, int32_t n, float *out, pg_stream_t stream);

/*
 * moe_grouped — one routed-MoE pass over n positions (nemotron_prefill.rs:
 * `pb_f32_mm` router, `pb_route` top-k, `pb_lists` per-expert lists,
 * `pb_q8_bank` expert banks with act = relu^2 on the up product, `pb_add_rms`
 * with add = 2 for the slot-ordered weighted sum into the residual):
 *     logits[b][e] = sum_c X[b][c] * Wr[e][c]                     (f32, order below)
 *     p[b][.]      = softmax(logits[b][.]) over all E experts
 *     sel[b][t]    = t-th largest logit (t < top_k), lower index wins a tie
 *     route_w[b][t]= p[b][sel[b][t]]  (divided by sum_t p[b][sel[b][t]] if renorm)
 *     counts[e], lists[e][0..counts[e]) = the entries j = b*top_k + t with
 *                    sel[b][t] == e, in ascending j
 *     u_j = relu^2( Up_e . X[b] ),  d_j = Down_e . u_j            (e = sel of j)
 *     h[b] += sum_t route_w[b][t] * d_{b*top_k+t}                  (t ascending)
 *     out[b] = w_norm * h[b] / sqrt(mean(h[b]^2) + eps)
 * Each selected expert's weights are streamed from HBM once for all of its
 * entries.  The logit is an f32 value in a fixed order: 64 partial sums, the
 * l-th chaining fused multiply-adds over the 4-column groups l, l+64, ... (the
 * 4 columns of a group in order), then folded pairwise for s = 32, 16, ..., 1
 * (partial l += partial l+s).  Expert choice is taken on those bits.
 *   X [n][H] f32 (the normed input), Wr [E][H] f32,
 *   up_q [E][I][H] int8, up_scale/up_bias [E][I][H/32] f32,
 *   down_q [E][H][I] int8, down_scale/down_bias [E][H][I/32] f32,
 *   h [n][H] f32 in/out, w_norm [H] f32, out [n][H] f32,
 *   logits [n][E] f32, sel [n][top_k] int32, route_w [n][top_k] f32,
 *   counts [E] int32, lists [E][n] int32 (entries past counts[e] unspecified),
 *   workspace of at least moe_grouped_workspace_bytes(n, H, I, E, top_k) bytes
 *   (16-byte aligned).  On return the workspace starts with the per-entry
 *   expert outputs: u [n*top_k][I] f32 at byte 0, then d [n*top_k][H] f32 at
 *   byte round_up(n*top_k*I*4, 256); row j is entry j = b*top_k + t.
 * PG_EUNSUPPORTED: n < 1 or n > 64, H % 32 or I % 32 != 0, H > 16384,
 *   E < 1 or E > 1024, top_k < 1 or top_k > min(E, 16).
 */
int moe_grouped(const float *X, int32_t n, int32_t H, const float *Wr, int32_t E,
                int32_t top_k, int32_t renorm, const int8_t *up_q, const float *up_scale,
                const float *up_bias, int32_t I, const int8_t *down_q, const float *down_scale,
                const float *down_bias, float *h, const float *w_norm, float eps, float *out,
                float *logits, int32_t *sel, float *route_w, int32_t *counts, int32_t *lists,
                void *workspace, size_t workspace_bytes, pg_stream_t stream);
size_t moe_grouped_workspace_bytes(int32_t n, int32_t H, int32_t I, int32_t E, int32_t top_k);

/*
 * moe_route_sigmoid — the sigmoid router with a selection bias
 * (nemotron_prefill.rs, `pb_route`), per position b of n:
 *     c[e]          = sigmoid32(logits[b][e]) + router_bias[e]     (one f32 add)
 *     sel[b][t]     = the t-th largest c (t < top_k), lower index wins a tie
 *     route_w[b][t] = sigmoid32(logits[b][sel]) / den * scale,
 *     den           = sum_t sigmoid32(logits[b][sel[b][t]]) + 1e-20 if renorm, else 1.
 * The bias steers the choice only.  sigmoid32 is one fixed sequence of
 * correctly rounded binary32 operations, so the choice it decides is
 * reproducible on any IEEE machine: x = clamp(-l, -80, 80);
 * k = rint(x * f32(log2 e)); r = fma(-k, ln2_tail, fma(-k, ln2_head, x)) with
 * ln2_head = 0.693145751953125 and ln2_tail = f32(ln 2 - ln2_head) (the
 * Cody-Waite reduction); p = the Taylor polynomial sum_{i<=7} r^i / i! by
 * Horner's rule from the r^7 term, one fma a term, coefficients f32(1/i!);
 * sigmoid32 = 1 / (1 + ldexp(p, k)).  The weights use the same values.
 *   logits [n][E] f32, router_bias [E] f32, sel [n][top_k] int32, route_w [n][top_k] f32.
 * PG_EUNSUPPORTED: E > 1024, top_k > min(E, 16).
 */
int moe_route_sigmoid(const float *logits, const float *router_bias, int32_t n, int32_t E,
                      int32_t top_k, int32_t renorm, float scale, int32_t *sel, float *route_w,
                      pg_stream_t stream);

/*
 * moe_grouped_sigmoid — moe_grouped with the sigmoid + bias router of
 * moe_route_sigmoid in place of softmax, and an optional dense term added with
 * the slots (nemotron_prefill.rs `pb_add_rms`, add = 2: the shared expert's
 * output starts the sum):
 *     h[b] += shared[b] + sum_t route_w[b][t] * d_{b*top_k+t}   (shared first, then t ascending)
 *     out[b] = w_norm * h[b] / sqrt(mean(h[b]^2) + eps)
 *   shared [n][H] f32 (16-byte aligned; NULL: no dense term; must not overlap h or
 *   out); every other argument, the workspace and the codes as moe_grouped.
 */
int moe_grouped_sigmoid(const float *X, int32_t n, int32_t H, const float *Wr, int32_t E,
                        int32_t top_k, const float *router_bias, int32_t renorm, float scale,
                        const int8_t *up_q, const float *up_scale, const float *up_bias, int32_t I,
                        const int8_t *down_q, const float *down_scale, const float *down_bias,
                        const float *shared, float *h, const float *w_norm, float eps, float *out,
                        float *logits, int32_t *sel, float *route_w, int32_t *counts, int32_t *lists,
                        void *workspace, size_t workspace_bytes, pg_stream_t stream);

/*
 * expert_bank_q82 — the grouped expert product on the q8_2f format
 * (nemotron_prefill.rs, the q8_2f bank payload of `pb_q8_bank`'s pass: int8
 * body, binary16 row scales, binary16 column field per expert).  For every
 * expert e and every entry j in lists[e][0 .. counts[e]):
 *     out[j][r] = act( rs[e][r] * sum_c q[e][r][c] * (cf[e][c] * x[j / src_div][c]) ),  r < rows.
 * Each expert's weights are read once for all of its entries.
 *   q [E][rows][cols] int8 (16-byte aligned), row_scale [E][rows] and
 *   col_field [E][cols] binary16 bits (col_field 16-byte aligned), x rows ldx
 *   floats apart (ldx % 4 == 0, 16-byte aligned), counts [E], lists [E][cap]
 *   int32 (entries ascending, as moe_grouped's lists), out rows ldo floats apart
 *   (rows of entries no expert lists are not written).
 * Arithmetic as prefill_gemm_q82: cf * x in f32 entering the matrix cores as an
 * exact-to-2^-17 bf16 hi + lo pair, int8 as exact bf16, f32 sums, the row scale
 * on the total.
 * PG_EUNSUPPORTED: cols % 32 != 0, cap > 64, E > 1024, rows * cols >= 2^31.
 */
int expert_bank_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field, int32_t E,
                    int32_t rows, int32_t cols, const float *x, int64_t ldx, int32_t src_div,
                    const int32_t *counts, const int32_t *lists, int32_t cap, float *out, int64_t ldo,
                    int32_t act, pg_stream_t stream);

/*
 * expert_bank_q4tp — the grouped expert product on the q4tp format
 * (nemotron_prefill.rs, `pb_q4_bank` over the experts of a pass): for expert
 * e < E and each of its listed entries j = lists[e][m], m < counts[e]:
 *     out[j][r] = act( sum_c 2^(base_er + code_{e,r,c/32} step_er) (nib_er(c) - 8) x[j / src_div][c] )
 * each expert's weights read once for all of its entries.  Layout per expert
 * as gemv_q4tp: nib [E][rows][cols/2] (16-byte aligned), params [E][rows] u32
 * (4-byte aligned), codes [E][rows][ceil(5 cols/32 / 8)]; x rows ldx floats
 * apart (16-byte aligned, ldx % 4 == 0), out rows ldo floats apart; counts,
 * lists and cap (<= 64) as expert_bank_q82.  The nibble n enters the matrix
 * cores as 128 + n (bf16, exact) and the - (128 + 8) as a per-block term
 * -136 * scale times the block's sum of the activations as the products see
 * them (bf16 hi + lo).
 * PG_EUNSUPPORTED: cols % 32 != 0, cap > 64, E > 1024, a code buffer under 8
 * bytes.  PG_EINVAL: null or misaligned pointers, sizes < 1, act not 0/1.
 */
int expert_bank_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t E, int32_t rows,
                     int32_t cols, const float *x, int64_t ldx, int32_t src_div, const int32_t *counts,
                     const int32_t *lists, int32_t cap, float *out, int64_t ldo, int32_t act, pg_stream_t stream);

/*
 * attn_kv_append — the pass's K and V rows into the caches (nemotron_prefill.rs,
 * `pb_kv_append`): kc[pos0 * width + i] = k[i], vc[...] = v[i] for i < n * width.
 *   k, v [n][width] f32, kc, vc [cap][width] f32 (width = nkv * hd, a multiple of 4;
 *   all 16-byte aligned).  PG_EINVAL: pos0 + n > cap.
 */
int attn_kv_append(const float *k, const float *v, int32_t n, int32_t width, int32_t pos0, float *kc,
                   float *vc, int32_t cap, pg_stream_t stream);

/*
 * attn_prefill — causal grouped-query attention over one pass of n positions at
 * absolute positions pos0 .. pos0 + n - 1 (nemotron_prefill.rs, `pb_attn` and
 * `pb_attn_merge`; the rows of the pass must already be in the caches):
 *     s_j        = (scale * q[b][h]) . kc[j][g],   g = h / (nh / nkv),  j <= pos0 + b
 *     o[b][h][d] = sum_j exp(s_j - max s) vc[j][g][d] / sum_j exp(s_j - max s)
 *   q [n][nh][hd] f32, kc, vc [>= pos0 + n][nkv][hd] f32 (16-byte aligned),
 *   o [n][nh][hd] f32; workspace of attn_prefill_workspace_bytes(...) bytes
 *   (split partials; contents on entry do not matter; must not overlap o).
 * Arithmetic: f32 throughout; the keys are cut into splits, each with its own
 * running maximum and sum, merged in split order.
 * PG_EUNSUPPORTED: hd not 64 or 128, 64 % (nh / nkv) != 0, n > 64.
 */
int attn_prefill(const float *q, const float *kc, const float *vc, int32_t n, int32_t pos0, int32_t nh,
                 int32_t nkv, int32_t hd, float scale, float *o, void *workspace, size_t workspace_bytes,
                 pg_stream_t stream);
size_t attn_prefill_workspace_bytes(int32_t n, int32_t pos0, int32_t nh, int32_t nkv, int32_t hd);

/*
 * pg_stream_read — a measurement call, not a product: reads `bytes` bytes at
 * `src` once, with 16-byte non-temporal loads, workgroup g of `workgroups`
 * reading the g-th contiguous share, and xors each workgroup's words into
 * sink[g] (its value means nothing; it keeps the loads alive).  Its rate is the
 * achievable HBM read ceiling the bandwidth-bound products are compared with
 * (the published peak is 8 TB/s).
 *   src 16-byte aligned, bytes a multiple of 16; sink [workgroups] 32-bit words.
 *   PG_EINVAL: null pointers, bytes 0 or not a multiple of 16, workgroups < 1.
 */
int pg_stream_read(const void *src, size_t bytes, int32_t workgroups, float *sink, pg_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PG_H */
