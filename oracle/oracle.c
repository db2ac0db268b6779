/*
 * Plain CPU oracle for the packed-weight product path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  The HIP product path
 * never includes, links or calls it, and it shares no source with that path.
 *
 * Every result is the plain definition written out in double precision from
 * the f32 / int8 / binary16 inputs: no blocking, no fusion, no reordering
 * beyond what the definition states.  The exceptions are the two binary32
 * values that decide an integer (the chosen experts): the f32 router logit
 * (oracle_router_logits_f32), summed in a fixed order, and the sigmoid
 * router's choice value (oracle_sigmoid_f32), one fixed sequence of binary32
 * operations; both are defined so that the device and this oracle take the
 * decision on identical bits.
 *
 * Sources (cortiq-engine docs.rs source pages):
 *  - weights stay packed on the device and are decoded inside the product:
 *    embryo_wide.wgsl (0.8.53), header comment;
 *  - residual add + RMSNorm per position: nemotron_prefill.rs (0.8.50),
 *    `pb_add_rms`; gemma_batch.rs (0.8.82), `g4_add_norm_b`;
 *  - relu^2 activation on the finished product: nemotron_prefill.rs,
 *    `pb_relu2` and the `act == 1` branch of `pb_q8_bank`;
 *  - router, top-k selection (lower expert id wins an exact tie), per-expert
 *    lists in ascending entry order: nemotron_prefill.rs, `pb_f32_mm`,
 *    `pb_route`, `pb_lists`;
 *  - routed expert FFN and the slot-ordered weighted sum into the residual:
 *    nemotron_prefill.rs, `pb_q8_bank` and `pb_add_rms` (add == 2).
 *
 * Two int8 formats: the block format (32 consecutive columns of a row share
 * one f32 scale and one f32 bias, w = scale*q + bias), and the pages' own
 * q8_2f format (int8 body, f16 row scales, f16 column field, w = rs*cf*q).
 *
 * Parity status: every function here is pinned by the CPU test suite (closed
 * forms, invariants, brute force, textbook routines); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BLOCK 32

/* ------------------------------------------------------------ binary16 */

/* IEEE 754 binary16 decode: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double oracle_f16_to_f64(uint16_t bits) {
    int sign = bits >> 15;
    int e = (bits >> 10) & 31;
    int m = bits & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: (m/1024) * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)m, e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------ dequant */

static inline double q8_weight(const int8_t *q, const float *scale, const float *bias,
                               int64_t cols, int64_t r, int64_t c) {
    int64_t b = r * (cols / BLOCK) + c / BLOCK;
    return (double)scale[b] * (double)q[r * cols + c] + (double)bias[b];
}

/* w[r][c] = scale[r][c/32] * q[r][c] + bias[r][c/32] */
void oracle_dequant_q8(const int8_t *q, const float *scale, const float *bias,
                       int64_t rows, int64_t cols, double *w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            w[r * cols + c] = q8_weight(q, scale, bias, cols, r, c);
}

static inline double act_apply(int act, double v) {
    if (act == 1) {              /* relu^2: max(v, 0)^2 */
        double t = v > 0.0 ? v : 0.0;
        return t * t;
    }
    return v;
}

/* ------------------------------------------------------------ products */

/* Y[b][r] = act( sum_c w[r][c] * X[b][c] ),  X [n][cols] f32, Y [n][rows] f64. */
void oracle_gemm_q8(const int8_t *q, const float *scale, const float *bias,
                    int64_t rows, int64_t cols, const float *X, int64_t n, int act,
                    double *Y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * rows; ++i) {
        int64_t b = i / rows, r = i % rows;
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c)
            acc += q8_weight(q, scale, bias, cols, r, c) * (double)X[b * cols + c];
        Y[b * rows + r] = act_apply(act, acc);
    }
}

/* Same product over a subset of output rows (for sampled checks of large
 * matrices): Y[b][j] = act( sum_c w[row_idx[j]][c] * X[b][c] ). */
void oracle_gemm_q8_rows(const int8_t *q, const float *scale, const float *bias,
                         int64_t rows, int64_t cols, const int64_t *row_idx, int64_t nrows,
                         const float *X, int64_t n, int act, double *Y) {
    (void)rows;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * nrows; ++i) {
        int64_t b = i / nrows, j = i % nrows, r = row_idx[j];
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c)
            acc += q8_weight(q, scale, bias, cols, r, c) * (double)X[b * cols + c];
        Y[b * nrows + j] = act_apply(act, acc);
    }
}

/* Y[b][r] = act( sum_c f16(W[r][c]) * X[b][c] ),  W as binary16 bits. */
void oracle_gemm_f16(const uint16_t *W, int64_t rows, int64_t cols, const float *X,
                     int64_t n, int act, double *Y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * rows; ++i) {
        int64_t b = i / rows, r = i % rows;
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c)
            acc += oracle_f16_to_f64(W[r * cols + c]) * (double)X[b * cols + c];
        Y[b * rows + r] = act_apply(act, acc);
    }
}

/* ------------------------------------------------------------ q8_2f */

/* The pages' own int8 format (gemma_batch.rs, `q8_2f_mm_r2` doc comment and
 * epilogue; nemotron_prefill.rs, the q8_2f expert-bank payload): an int8 body
 * q[rows][cols], one binary16 scale per row rs[rows] and one binary16 factor per
 * column cf[cols] (the "column field").  The column field multiplies the
 * activation before the product and the row scale the finished sum, so the
 * weight the product applies is
 *     w[r][c] = rs[r] * cf[c] * q[r][c]. */
static inline double q82_weight(const int8_t *q, const uint16_t *rs, const uint16_t *cf,
                                int64_t cols, int64_t r, int64_t c) {
    return oracle_f16_to_f64(rs[r]) * oracle_f16_to_f64(cf[c]) * (double)q[r * cols + c];
}

void oracle_dequant_q82(const int8_t *q, const uint16_t *rs, const uint16_t *cf, int64_t rows,
                        int64_t cols, double *w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            w[r * cols + c] = q82_weight(q, rs, cf, cols, r, c);
}

/* Y[b][r] = act( sum_c w[r][c] * X[b][c] ) with the q8_2f weight above. */
void oracle_gemm_q82(const int8_t *q, const uint16_t *rs, const uint16_t *cf, int64_t rows,
                     int64_t cols, const float *X, int64_t n, int act, double *Y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * rows; ++i) {
        int64_t b = i / rows, r = i % rows;
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c)
            acc += q82_weight(q, rs, cf, cols, r, c) * (double)X[b * cols + c];
        Y[b * rows + r] = act_apply(act, acc);
    }
}

/* The pages' 4-bit format, q4tp (nemotron_prefill.rs, the q4tp expert bank
 * `pb_q4_bank` and its nibble and code readers).  Per row r:
 *  - a 4-bit code per column: byte c/2 of the row's nibble bytes holds column
 *    c in its low half when c is even and in its high half when c is odd; the
 *    weight integer is that code minus 8 (range -8 .. 7);
 *  - two binary16 parameters in one 32-bit word: base in the low half, step in
 *    the high half;
 *  - a 5-bit log-scale code per 32-column group g, packed least significant
 *    bit first: the code of g occupies bits 5g .. 5g+4 of the row's code
 *    bytes (cstride = ceil(5 * cols/32 / 8) bytes a row);
 *  - the group's scale is 2 ** (base + code * step).
 * So   w[r][c] = 2 ** (base_r + code_{r, c/32} * step_r) * (nib_r(c) - 8). */
static double q4tp_weight(const uint8_t *nib, const uint32_t *params, const uint8_t *codes,
                          int64_t cols, int64_t r, int64_t c) {
    const int64_t gpr = cols / 32, cstride = (5 * gpr + 7) / 8;
    const uint8_t *cr = codes + r * cstride;
    const int64_t bit = 5 * (c / 32);
    unsigned field = 0;
    for (int i = 0; i < 5; ++i) {
        const int64_t k = bit + i;
        field |= (unsigned)((cr[k / 8] >> (k % 8)) & 1u) << i;
    }
    const double base = oracle_f16_to_f64((uint16_t)(params[r] & 0xFFFFu));
    const double step = oracle_f16_to_f64((uint16_t)(params[r] >> 16));
    const uint8_t byte = nib[r * (cols / 2) + c / 2];
    const int v = (int)((c % 2 == 0) ? (byte & 0xFu) : (byte >> 4)) - 8;
    return exp2(base + (double)field * step) * (double)v;
}

void oracle_dequant_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes,
                         int64_t rows, int64_t cols, double *w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) w[r * cols + c] = q4tp_weight(nib, params, codes, cols, r, c);
}

/* Y[b][r] = act( sum_c w[r][c] * X[b][c] ) with the q4tp weight above. */
void oracle_gemm_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int64_t rows,
                      int64_t cols, const float *X, int64_t n, int act, double *Y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * rows; ++i) {
        int64_t b = i / rows, r = i % rows;
        double acc = 0.0;
        for (int64_t c = 0; c < cols; ++c)
            acc += q4tp_weight(nib, params, codes, cols, r, c) * (double)X[b * cols + c];
        Y[b * rows + r] = act_apply(act, acc);
    }
}

/* ------------------------------------------------------------ prefill attention */

/* Causal grouped-query attention over one pass (nemotron_prefill.rs,
 * `pb_kv_append` then `pb_attn` / `pb_attn_merge`).  The pass holds n positions
 * at absolute positions pos0 .. pos0 + n - 1; their K and V rows are already in
 * the caches kc, vc [pos][nkv][hd].  Query head h of position b reads KV head
 * g = h / (nh / nkv) and every key position j <= pos0 + b:
 *     s_j  = scale * sum_d q[b][h][d] * kc[j][g][d]
 *     o[b][h][d] = sum_j exp(s_j - max_j s) vc[j][g][d] / sum_j exp(s_j - max_j s)
 * in f64 from the f32 inputs. */
void oracle_attn_prefill(const float *q, const float *kc, const float *vc, int64_t n, int64_t pos0,
                         int64_t nh, int64_t nkv, int64_t hd, double scale, double *o) {
    const int64_t rep = nh / nkv;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * nh; ++i) {
        const int64_t b = i / nh, h = i % nh, g = h / rep, J = pos0 + b + 1;
        double *s = (double *)malloc((size_t)J * sizeof(double));
        double mx = -INFINITY;
        for (int64_t j = 0; j < J; ++j) {
            double acc = 0.0;
            for (int64_t d = 0; d < hd; ++d)
                acc += (double)q[(b * nh + h) * hd + d] * (double)kc[(j * nkv + g) * hd + d];
            s[j] = scale * acc;
            if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < J; ++j) {
            s[j] = exp(s[j] - mx);
            den += s[j];
        }
        for (int64_t d = 0; d < hd; ++d) {
            double num = 0.0;
            for (int64_t j = 0; j < J; ++j) num += s[j] * (double)vc[(j * nkv + g) * hd + d];
            o[(b * nh + h) * hd + d] = num / den;
        }
        free(s);
    }
}

/* ------------------------------------------------------------ argmax */

/* Token choice of every position (nemotron_prefill.rs, `pb_argmax`, the verify
 * passes): ids[b] is the smallest index i whose logit L[b][i] is the largest
 * of the row, where only logits above -3.0e38 take part (the search starts
 * from that value at index 0, so a row with no such logit, or all NaN, gives
 * 0).  Comparisons are in f32, the logits' own precision. */
void oracle_argmax_rows(const float *L, int64_t n, int64_t vocab, uint32_t *ids) {
    for (int64_t b = 0; b < n; ++b) {
        float best = -3.0e38f;
        uint32_t at = 0;
        for (int64_t i = 0; i < vocab; ++i) {
            const float v = L[b * vocab + i];
            if (v > best) {
                best = v;
                at = (uint32_t)i;
            }
        }
        ids[b] = at;
    }
}

/* ------------------------------------------------------------ add + RMSNorm */

/* Per position b:  h'[i] = h[b][i] + delta[b*delta_stride + i]   (no add if delta is NULL)
 *                  out[b][i] = w[i] * h'[i] / sqrt( (1/H) sum_i h'[i]^2 + eps ).
 * h_out receives h'; both outputs in f64. */
void oracle_add_rmsnorm(const float *h, const float *delta, int64_t delta_stride,
                        const float *w, double eps, int64_t hidden, int64_t n,
                        double *h_out, double *out) {
    for (int64_t b = 0; b < n; ++b) {
        double ss = 0.0;
        for (int64_t i = 0; i < hidden; ++i) {
            double v = (double)h[b * hidden + i];
            if (delta) v += (double)delta[b * delta_stride + i];
            h_out[b * hidden + i] = v;
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)hidden + eps);
        for (int64_t i = 0; i < hidden; ++i)
            out[b * hidden + i] = (double)w[i] * h_out[b * hidden + i] * inv;
    }
}

/* ------------------------------------------------------------ router */

/* logits[b][e] = sum_c X[b][c] * Wr[e][c], in f64. */
void oracle_router_logits_f64(const float *X, const float *Wr, int64_t n, int64_t H,
                              int64_t E, double *logits) {
    for (int64_t b = 0; b < n; ++b)
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t c = 0; c < H; ++c)
                acc += (double)X[b * H + c] * (double)Wr[e * H + c];
            logits[b * E + e] = acc;
        }
}

/* The same logit as an f32 value, summed in the order the device uses, so that
 * the expert choice (an integer decided by f32 compares) is taken on the same
 * bits on both sides.  Order: the row is cut into 4-column groups g; 64 partial
 * sums p[l] each chain a single-rounding fused multiply-add over the groups
 * g = l, l+64, l+128, ... and, inside a group, over its 4 columns in order;
 * the 64 partials then fold pairwise, for s = 32, 16, 8, 4, 2, 1:
 * p[l] = p[l] + p[l+s] for l < s.  The logit is p[0].  Requires H % 4 == 0. */
void oracle_router_logits_f32(const float *X, const float *Wr, int64_t n, int64_t H,
                              int64_t E, float *logits) {
    int64_t groups = H / 4;
    for (int64_t b = 0; b < n; ++b)
        for (int64_t e = 0; e < E; ++e) {
            float p[64];
            for (int l = 0; l < 64; ++l) {
                float acc = 0.0f;
                for (int64_t g = l; g < groups; g += 64)
                    for (int t = 0; t < 4; ++t)
                        acc = fmaf(Wr[e * H + 4 * g + t], X[b * H + 4 * g + t], acc);
                p[l] = acc;
            }
            for (int s = 32; s >= 1; s >>= 1)
                for (int l = 0; l < s; ++l)
                    p[l] = p[l] + p[l + s];
            logits[b * E + e] = p[0];
        }
}

/* Softmax over all E experts and top-k selection for each position.
 * Selection follows the page's router: k rounds; each round takes the largest
 * remaining score, the lower expert index winning an exact tie, then removes it.
 * The score ranked is the f32 logit (softmax is strictly increasing in it, and
 * ranking the logit avoids ties that rounding of probabilities would create).
 * probs[b][e] = exp(l_e - max) / sum_e' exp(l_e' - max) in f64;
 * rw[b][t] = probs[b][sel[b][t]], divided by sum_t probs[b][sel[b][t]] if renorm. */
void oracle_route(const float *logits, int64_t n, int64_t E, int64_t k, int renorm,
                  int32_t *sel, double *rw, double *probs) {
    char *taken = (char *)malloc((size_t)E);
    for (int64_t b = 0; b < n; ++b) {
        const float *l = logits + b * E;
        double mx = -INFINITY;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > mx) mx = (double)l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) z += exp((double)l[e] - mx);
        for (int64_t e = 0; e < E; ++e) probs[b * E + e] = exp((double)l[e] - mx) / z;

        memset(taken, 0, (size_t)E);
        double sum = 0.0;
        for (int64_t t = 0; t < k; ++t) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: lower index keeps a tie */
            }
            taken[best] = 1;
            sel[b * k + t] = (int32_t)best;
            rw[b * k + t] = probs[b * E + best];
            sum += probs[b * E + best];
        }
        if (renorm)
            for (int64_t t = 0; t < k; ++t) rw[b * k + t] /= sum;
    }
    free(taken);
}

/* The sigmoid as one fixed sequence of IEEE binary32 operations, so that the
 * expert choice it decides is taken on the same bits wherever the sequence is
 * carried out (nemotron_prefill.rs, `pb_route`, takes its choice value in f32).
 *
 * exp(x) by the argument reduction of W. J. Cody and W. Waite, "Software
 * Manual for the Elementary Functions" (1980): x = k ln2 + r with
 * k = rint(x log2 e) and r = x - k ln2 taken in two steps with ln2 split into
 * a head of 16 significant bits and the binary32 rounding of the remainder;
 * e^r by its Taylor series through r^7 (|r| <= ln2 / 2, truncation below
 * 1e-8 relative), evaluated by Horner's rule with one fused multiply-add a
 * term; then e^x = 2^k e^r.  x is first clamped to [-80, 80], so that no
 * value in the sequence below is subnormal or infinite (sigma(l) for
 * |l| > 80 then differs from the true value by less than 2e-35).
 * sigma(l) = 1 / (1 + exp(-l)): one binary32 add and one correctly rounded
 * binary32 divide. */
static const float kLog2e = 1.44269502162933349609375f;     /* binary32(log2 e) */
static const float kLn2Hi = 0.693145751953125f;             /* ln 2, 16 significant bits */
static const float kLn2Lo = 1.428606765330187045037746429443359375e-06f; /* binary32(ln 2 - head) */

float oracle_exp_f32(float x) {
    x = fminf(fmaxf(x, -80.0f), 80.0f);
    const float k = rintf(x * kLog2e);
    float r = fmaf(-k, kLn2Hi, x);
    r = fmaf(-k, kLn2Lo, r);
    /* 1/n!, n = 7 .. 0, each rounded to binary32 */
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)k);
}

float oracle_sigmoid_f32(float l) {
    const float e = oracle_exp_f32(-l);
    const float d = 1.0f + e;
    return 1.0f / d;
}

void oracle_sigmoid_f32_array(const float *l, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid_f32(l[i]);
}

/* The sigmoid router with a selection bias (nemotron_prefill.rs, `pb_route`):
 * per position b the choice value of expert e is the binary32 value
 *     c_e = sigma32(l_e) + bias[e]   (one binary32 add),
 * with sigma32 the fixed-sequence sigmoid above, and k rounds each take the
 * largest remaining c (the lower index on a tie) and remove it.  The bias
 * steers the choice only; the weight of slot t is the definition in f64,
 *     rw[b][t] = sigma(l_sel) / den * scale,  sigma(x) = 1 / (1 + exp(-x)),
 *     den = sum_t sigma(l_sel[t]) + 1e-20 when norm, else 1.
 * choice[b][e] receives c_e. */
void oracle_route_sigmoid(const float *logits, const float *bias, int64_t n, int64_t E, int64_t k,
                          int norm, double scale, int32_t *sel, double *rw, float *choice) {
    char *taken = (char *)malloc((size_t)E);
    for (int64_t b = 0; b < n; ++b) {
        const float *l = logits + b * E;
        float *c = choice + b * E;
        for (int64_t e = 0; e < E; ++e) {
            const float sg = oracle_sigmoid_f32(l[e]);
            c[e] = sg + bias[e];
        }
        memset(taken, 0, (size_t)E);
        double sum = 0.0;
        for (int64_t t = 0; t < k; ++t) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || c[e] > c[best]) best = e;   /* strict: lower index keeps a tie */
            }
            taken[best] = 1;
            sel[b * k + t] = (int32_t)best;
            sum += 1.0 / (1.0 + exp(-(double)l[best]));
        }
        const double den = norm ? sum + 1e-20 : 1.0;
        for (int64_t t = 0; t < k; ++t)
            rw[b * k + t] = (1.0 / (1.0 + exp(-(double)l[sel[b * k + t]]))) / den * scale;
    }
    free(taken);
}

/* Per expert e, the entries j = b*k + t (ascending) whose selection is e.
 * lists is [E][cap]; counts[e] = number of entries; entries past counts[e] are
 * left untouched. */
void oracle_group(const int32_t *sel, int64_t n, int64_t k, int64_t E, int64_t cap,
                  int32_t *counts, int32_t *lists) {
    for (int64_t e = 0; e < E; ++e) {
        int32_t c = 0;
        for (int64_t j = 0; j < n * k; ++j)
            if (sel[j] == e) lists[e * cap + c++] = (int32_t)j;
        counts[e] = c;
    }
}

/* ------------------------------------------------------------ routed experts */

/* One (position, slot) pair j = b*k + t with expert e = sel[j]:
 *   u_j = relu^2( Up_e . X[b] )      [I]
 *   d_j = Down_e . u_j               [H]
 * Banks: up q [E][I][H], scale/bias [E][I][H/32]; down q [E][H][I], scale/bias [E][H][I/32]. */
static void expert_pair(const float *X, int64_t H, int64_t I, int64_t b, int64_t e,
                        const int8_t *up_q, const float *up_s, const float *up_b,
                        const int8_t *dn_q, const float *dn_s, const float *dn_b,
                        double *u, double *d) {
    const int8_t *uq = up_q + e * I * H;
    const float *us = up_s + e * I * (H / BLOCK), *ub = up_b + e * I * (H / BLOCK);
    for (int64_t r = 0; r < I; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < H; ++c)
            acc += q8_weight(uq, us, ub, H, r, c) * (double)X[b * H + c];
        u[r] = act_apply(1, acc);
    }
    const int8_t *dq = dn_q + e * H * I;
    const float *ds = dn_s + e * H * (I / BLOCK), *db = dn_b + e * H * (I / BLOCK);
    for (int64_t r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < I; ++c)
            acc += q8_weight(dq, ds, db, I, r, c) * u[c];
        d[r] = acc;
    }
}

/* Ungrouped: loop over the pairs in entry order.  U [n*k][I], D [n*k][H]. */
void oracle_moe_experts_ungrouped(const float *X, int64_t n, int64_t H, int64_t I,
                                  const int32_t *sel, int64_t k,
                                  const int8_t *up_q, const float *up_s, const float *up_b,
                                  const int8_t *dn_q, const float *dn_s, const float *dn_b,
                                  double *U, double *D) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t j = 0; j < n * k; ++j)
        expert_pair(X, H, I, j / k, sel[j], up_q, up_s, up_b, dn_q, dn_s, dn_b,
                    U + j * I, D + j * H);
}

/* Grouped: loop over experts, and for each over its list of entries (the
 * expert-major walk of the device).  Per pair the arithmetic is the ungrouped
 * one, so both walks give the same bits. */
void oracle_moe_experts_grouped(const float *X, int64_t n, int64_t H, int64_t I,
                                int64_t E, int64_t k, const int32_t *counts,
                                const int32_t *lists, int64_t cap,
                                const int8_t *up_q, const float *up_s, const float *up_b,
                                const int8_t *dn_q, const float *dn_s, const float *dn_b,
                                double *U, double *D) {
    (void)n;
#pragma omp parallel for schedule(dynamic)
    for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < counts[e]; ++i) {
            int64_t j = lists[e * cap + i];
            expert_pair(X, H, I, j / k, e, up_q, up_s, up_b, dn_q, dn_s, dn_b,
                        U + j * I, D + j * H);
        }
}

/* Combine into the residual and norm, per position b (nemotron_prefill.rs,
 * `pb_add_rms` with add = 2; `shared` is its optional dense term, the output of
 * a shared expert, which starts the sum before the slots; NULL: none):
 *   m[i] = shared[b][i] + sum_{t=0..k-1} rw[b][t] * D[b*k+t][i]   (slot order)
 *   h'   = h[b] + m;   out[b] = w * h' / sqrt(mean(h'^2) + eps). */
void oracle_moe_combine(const float *h, const float *shared, const double *D, const double *rw,
                        int64_t n, int64_t k, int64_t H, const float *w, double eps,
                        double *h_out, double *out) {
    for (int64_t b = 0; b < n; ++b) {
        double ss = 0.0;
        for (int64_t i = 0; i < H; ++i) {
            double m = shared ? (double)shared[b * H + i] : 0.0;
            for (int64_t t = 0; t < k; ++t) m += rw[b * k + t] * D[(b * k + t) * H + i];
            double v = (double)h[b * H + i] + m;
            h_out[b * H + i] = v;
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t i = 0; i < H; ++i) out[b * H + i] = (double)w[i] * h_out[b * H + i] * inv;
    }
}

/* Thread count the OpenMP loops above run with (1 when built without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP thread count of the parallel loops above (timing only). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
