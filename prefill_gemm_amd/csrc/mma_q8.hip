// Batched prefill product (prefill_gemm_q8) and the activation staging it
// shares with the grouped expert banks.
//
// nemotron_prefill.rs (module doc): a pass holds up to 64 positions and every
// weight is read once per pass.  gemma_batch.rs (`encode_q82_mm`): the prompt
// GEMM computes y[nb][rows] = x[nb][cols] . W^T and refuses (encodes nothing
// for) shapes its tile does not cover.
#include <algorithm>
#include <mutex>

#include "dense_q8.h"
#include "pg_host.h"

namespace pg {

// Fragment layout for the dense pass (see dense_q8.h): one thread per (row m,
// 16-column half block) over mts * 32 rows (rows >= n are zero) and 16 * ng blocks.
// The staging launch also clears zero[0 .. nzero) (split tickets and block
// sums of the launches that follow), grid-stride.
__device__ __forceinline__ void clear_words(unsigned *zero, int nzero) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nzero; i += gridDim.x * blockDim.x) zero[i] = 0u;
}

// meta (device {n, pos0}, or NULL): the pass size read at launch; X then
// addresses row pos0 of a buffer of rows_total rows.  A pass outside it stages
// nothing (the products that follow return at once too).
__global__ __launch_bounds__(256) void stage_x_frag_kernel(const float *__restrict__ X, int n,
                                                           int cols, int mts, u32x4 *__restrict__ xp,
                                                           __bf16 *__restrict__ xs, unsigned *zero, int nzero,
                                                           const uint16_t *__restrict__ cf,
                                                           const int *__restrict__ meta, int rows_total) {
    clear_words(zero, nzero);
    if (meta) {
        n = __builtin_amdgcn_readfirstlane(meta[0]);
        const int pos0 = __builtin_amdgcn_readfirstlane(meta[1]);
        if (n < 1 || n > mts * 32 || pos0 < 0 || pos0 > rows_total - n) return;
        X += (long long)pos0 * cols;
    }
    const int nb = cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int per_row = ng * 32;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int m = (int)(t / per_row);
    const int hb = (int)(t % per_row);
    const int blk = hb >> 1, h = hb & 1;
    if (m >= mts * 32) return;
    const bool live = m < n && blk < nb;
    float v[16];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(X + (long long)m * cols + 32 * blk + 16 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = src[j];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
        if (cf) {
            // q8_2f: the column field folds into the staged activation.
            const uint16_t *c = cf + 32 * blk + 16 * h;
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] *= (float)__builtin_bit_cast(_Float16, c[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    put_frag_half(v, m, blk, h, nb, mts, xp, xs);
}

// Residual add + RMSNorm fused into the fragment staging (nemotron_prefill.rs,
// `pb_add_rms` with add = 1, ahead of the next product): workgroup m holds A
// row m, kStageNormIter half blocks per thread in registers:
//     h' = H[m] + delta[m];  X[m] = w * h' / sqrt(mean(h'^2) + eps)
// H_out[m] = h' and X_out[m] = X[m] are written if given.  Rows m >= n stage zeros.
constexpr int kStageNormIter = 4;  // cols <= 4 * 256 * 16 = 16384

__global__ __launch_bounds__(256) void stage_norm_frag_kernel(
    const float *__restrict__ H, const float *__restrict__ delta, int dstride, const float *__restrict__ w,
    float eps, int n, int cols, int mts, float *__restrict__ H_out, float *__restrict__ X_out,
    u32x4 *__restrict__ xp, __bf16 *__restrict__ xs, unsigned *zero, int nzero) {
    __shared__ float red[4];
    clear_words(zero, nzero);
    const int nb = cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int per_row = ng * 32;
    const int m = blockIdx.x;
    const bool row_live = m < n;
    float v[kStageNormIter][16];
    float ss = 0.0f;
#pragma unroll
    for (int it = 0; it < kStageNormIter; ++it) {
        const int hb = threadIdx.x + 256 * it;
        const int c0 = 16 * hb;
        const bool live = row_live && c0 < cols;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 a = make_float4(0, 0, 0, 0);
            if (live) {
                a = reinterpret_cast<const float4 *>(H + (long long)m * cols + c0)[j];
                if (delta) {
                    const float4 d = reinterpret_cast<const float4 *>(delta + (long long)m * dstride + c0)[j];
                    a.x += d.x; a.y += d.y; a.z += d.z; a.w += d.w;
                }
                if (H_out) reinterpret_cast<float4 *>(H_out + (long long)m * cols + c0)[j] = a;
                ss += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
            }
            v[it][4 * j] = a.x; v[it][4 * j + 1] = a.y; v[it][4 * j + 2] = a.z; v[it][4 * j + 3] = a.w;
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = rsqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)cols + eps);
#pragma unroll
    for (int it = 0; it < kStageNormIter; ++it) {
        const int hb = threadIdx.x + 256 * it;
        if (hb >= per_row) break;  // uniform across each pair of lanes (per_row is even)
        const int c0 = 16 * hb;
        if (row_live && c0 < cols) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 g = reinterpret_cast<const float4 *>(w + c0)[j];
                v[it][4 * j] = g.x * (v[it][4 * j] * inv);
                v[it][4 * j + 1] = g.y * (v[it][4 * j + 1] * inv);
                v[it][4 * j + 2] = g.z * (v[it][4 * j + 2] * inv);
                v[it][4 * j + 3] = g.w * (v[it][4 * j + 3] * inv);
                if (X_out)
                    reinterpret_cast<float4 *>(X_out + (long long)m * cols + c0)[j] =
                        make_float4(v[it][4 * j], v[it][4 * j + 1], v[it][4 * j + 2], v[it][4 * j + 3]);
            }
        }
        put_frag_half(v[it], m, hb >> 1, hb & 1, nb, mts, xp, xs);
    }
}

// Dense pass: workgroup id -> (panel of 128 rows, K split).  Splits of one
// panel take consecutive ids.  The activation ring is dynamic LDS (more than
// the 64 KB a static array may take).
constexpr int kDNK = 4, kDNX = 2, kDNW = 4;
template <int MT>
using DCfg = DenseCfg<MT, kDNK, kDNX, kDNW>;

template <int MT, int FMT>
__global__ __launch_bounds__(DCfg<MT>::kThreads) void dense_kernel(DenseArgs P, int bps) {
    extern __shared__ u32x4 dlds[];
    // Workgroups go to the 8 chiplets in turn (id % 8), and each chiplet has
    // its own L2: chiplet x takes a contiguous run of items in split-major
    // order, so that its workgroups share the staged activations of one or
    // two K ranges.
    const int G = gridDim.x, x = blockIdx.x % 8;
    const int id = (x * (G / 8) + min(x, G % 8)) + blockIdx.x / 8;
    const int panels = (P.rows + DCfg<MT>::kRows - 1) / DCfg<MT>::kRows;
    const int split = id / panels, panel = id % panels;
    const int nb = P.cols >> 5;
    const int kb0 = split * bps;
    const int kb1 = min(nb, kb0 + bps);
    P.split = split;
    if (!dense_resolve_meta(P)) return;
    dense_panel<MT, kDNK, kDNX, kDNW, FMT>(P, panel * DCfg<MT>::kRows, kb0, kb1, dlds);
}

template <int MT, int FMT>
static int launch_dense(const DenseArgs &P, int grid, int bps, hipStream_t s) {
    constexpr size_t lds = (size_t)DCfg<MT>::kLdsU4 * sizeof(u32x4);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(dense_kernel<MT, FMT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return PG_ELAUNCH;
    hipLaunchKernelGGL((dense_kernel<MT, FMT>), dim3(grid), dim3(DCfg<MT>::kThreads), lds, s, P, bps);
    return launch_status();
}

// Blocks per K split of a dense pass: a multiple of 16 (one bias group per
// loop iteration), with as many splits as keep panels x splits within one
// workgroup per compute unit (256).
int dense_blocks_per_split(int rows, int cols) {
    const int panels = ceil_div(rows, DCfg<2>::kRows);
    const int groups = ceil_div(cols / 32, 16);
    const int s = std::min(std::max(1, 256 / panels), groups);
    return 16 * ceil_div(groups, s);
}

int dense_splits(int rows, int cols) { return ceil_div(cols / 32, dense_blocks_per_split(rows, cols)); }

}  // namespace pg

using namespace pg;

// Fragment-layout staging sizes of n rows (mts tiles of 32 rows).
static size_t frag_x_bytes(int n, int cols) { return (size_t)ceil_div(n, 32) * cols * 128; }
static size_t frag_s_bytes(int n, int cols) {
    return (size_t)ceil_div(n, 32) * ceil_div(cols / 32, 16) * 2048;
}
static int dense_panels(int rows) { return ceil_div(rows, DCfg<2>::kRows); }
static size_t parts_bytes(int rows, int cols, int n) {
    const int s = dense_splits(rows, cols);
    return s > 1 ? (size_t)s * n * ceil_div(rows, DCfg<2>::kRows) * DCfg<2>::kRows * sizeof(float) : 0;
}

// Workspace of one product: staged fragments, block sums, split tickets,
// split partials.
struct OneLayout {
    size_t xs, tickets, parts, total;
};
static OneLayout one_layout(int rows, int cols, int n) {
    OneLayout L;
    L.xs = round_up(frag_x_bytes(n, cols), 256);
    L.tickets = L.xs + round_up(frag_s_bytes(n, cols), 256);
    L.parts = L.tickets + round_up((size_t)dense_panels(rows) * 4, 256);
    L.total = L.parts + parts_bytes(rows, cols, n);
    return L;
}

extern "C" size_t prefill_gemm_q8_workspace_bytes(int32_t rows, int32_t cols, int32_t n) {
    if (rows <= 0 || cols <= 0 || n <= 0 || cols % 32) return 0;
    return one_layout(rows, cols, n).total;
}

// Residual add + RMSNorm ahead of a prefill product (stage_norm_frag_kernel).
struct StageNorm {
    const float *H;
    const float *delta;
    int dstride;
    const float *w;
    float eps;
    float *H_out;
    float *X_out;
};

static int launch_stage_frag(const float *X, int n, int cols, void *xp, void *xs, unsigned *zero, int nzero,
                             hipStream_t s, const uint16_t *cf = nullptr, const int *meta = nullptr,
                             int rows_total = 0) {
    const int mts = ceil_div(n, 32);
    const int nb = cols / 32, ng = (nb + 15) / 16;
    const long long threads = (long long)mts * 32 * ng * 32;
    hipLaunchKernelGGL(stage_x_frag_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, X, n, cols,
                       mts, reinterpret_cast<u32x4 *>(xp), reinterpret_cast<__bf16 *>(xs), zero, nzero, cf, meta,
                       rows_total);
    return launch_status();
}

// The dense pass over one product whose activations are staged at (xp, xs);
// the epilogue fields of P are the caller's.  Split partials and tickets at
// (parts, tickets); the tickets must be zero.  fmt: the weight format (kFmtQ82:
// format (P.rs row scales; the column field is already in the staged activations).
static int run_dense(DenseArgs P, const void *xp, const void *xs, float *parts, unsigned *tickets, hipStream_t s,
                     int fmt = kFmtQ8) {
    P.xp = reinterpret_cast<const u32x4 *>(xp);
    P.xs = reinterpret_cast<const u32x4 *>(xs);
    P.mts = ceil_div(P.n, 32);
    if (!P.meta) P.nl = P.n;
    const int nb = P.cols / 32;
    const int bps = dense_blocks_per_split(P.rows, P.cols);
    P.splits = ceil_div(nb, bps);  // splits that hold at least one block
    P.parts = parts;
    P.tickets = tickets;
    const int grid = dense_panels(P.rows) * P.splits;
    if (fmt == kFmtQ82)
        return P.mts == 2 ? launch_dense<2, kFmtQ82>(P, grid, bps, s) : launch_dense<1, kFmtQ82>(P, grid, bps, s);
    if (fmt == kFmtQ4)
        return P.mts == 2 ? launch_dense<2, kFmtQ4>(P, grid, bps, s) : launch_dense<1, kFmtQ4>(P, grid, bps, s);
    return P.mts == 2 ? launch_dense<2, kFmtQ8>(P, grid, bps, s) : launch_dense<1, kFmtQ8>(P, grid, bps, s);
}

// Staging (plain or normed) into the workspace, then the dense matrix-core pass
// (split partials added in order inside it).  Arguments are checked by the callers.
static int prefill_run(const int8_t *q, const float *scale, const float *bias, int rows, int cols,
                       const float *X, const StageNorm *nm, int n, float *Y, int act, void *workspace,
                       hipStream_t s) {
    char *ws = static_cast<char *>(workspace);
    const OneLayout L = one_layout(rows, cols, n);
    void *xp = ws, *xs = ws + L.xs;
    unsigned *tickets = reinterpret_cast<unsigned *>(ws + L.tickets);
    const int mts = ceil_div(n, 32);
    int rc;
    if (nm) {
        hipLaunchKernelGGL(stage_norm_frag_kernel, dim3(mts * 32), dim3(256), 0, s, nm->H, nm->delta,
                           nm->dstride, nm->w, nm->eps, n, cols, mts, nm->H_out, nm->X_out,
                           reinterpret_cast<u32x4 *>(xp), reinterpret_cast<__bf16 *>(xs), tickets, dense_panels(rows));
        rc = launch_status();
    } else {
        rc = launch_stage_frag(X, n, cols, xp, xs, tickets, dense_panels(rows), s);
    }
    if (rc) return rc;
    DenseArgs P{};
    P.q = q;
    P.scale = scale;
    P.bias = bias;
    P.rows = rows;
    P.cols = cols;
    P.n = n;
    P.out = Y;
    P.ldo = rows;
    P.act = act;
    P.mode = kDensePlain;
    return run_dense(P, xp, xs, reinterpret_cast<float *>(ws + L.parts), tickets, s);
}
extern "C" int prefill_gemm_q8(const int8_t *q, const float *scale, const float *bias,
                               int32_t rows, int32_t cols, const float *X, int32_t n, float *Y,
                               int32_t act, void *workspace, size_t workspace_bytes,
                               pg_stream_t stream) {
    if (!q || !scale || !bias || !X || !Y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || n <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(X) || !aligned16(Y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || n > 64) return PG_EUNSUPPORTED;
    const size_t need = prefill_gemm_q8_workspace_bytes(rows, cols, n);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PG_EWORKSPACE;
    return prefill_run(q, scale, bias, rows, cols, X, nullptr, n, Y, act, workspace, as_stream(stream));
}

// prefill_gemm_q8_noalloc: prefill_gemm_q8 with its workspace in a file-scope
// device array instead of a caller's buffer, for callers that cannot allocate.
// Each device holds its own copy of the array (allocated when the library's
// code object is loaded on it, kept until the process ends).  Host code never
// passes the array's name to a kernel: its device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and kept.
// The staging launch clears the split tickets itself, so the array needs no
// clearing between calls; calls that overlap on one device share the array
// and race.
static __device__ __align__(256) unsigned char scratch[PG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The current device's address of `scratch` (nullptr on failure).
static void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

extern "C" int prefill_gemm_q8_noalloc(const int8_t *q, const float *scale, const float *bias,
                                       int32_t rows, int32_t cols, const float *X, int32_t n, float *Y,
                                       int32_t act, pg_stream_t stream) {
    if (!q || !scale || !bias || !X || !Y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || n <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(X) || !aligned16(Y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || n > 64) return PG_EUNSUPPORTED;
    if (prefill_gemm_q8_workspace_bytes(rows, cols, n) > PG_NOALLOC_SCRATCH_BYTES) return PG_EUNSUPPORTED;
    void *ws = scratch_address();
    if (!ws) return PG_ELAUNCH;
    return prefill_run(q, scale, bias, rows, cols, X, nullptr, n, Y, act, ws, as_stream(stream));
}

extern "C" int prefill_gemm_q8_addnorm(const int8_t *q, const float *scale, const float *bias,
                                       int32_t rows, int32_t cols, const float *H, const float *delta,
                                       int32_t delta_stride, const float *w, float eps, int32_t n,
                                       float *H_out, float *X_out, float *Y, int32_t act,
                                       void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    if (!q || !scale || !bias || !H || !w || !Y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || n <= 0 || !(eps >= 0.0f)) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(H) || !aligned16(w) || !aligned16(Y)) return PG_EINVAL;
    if ((delta && !aligned16(delta)) || (H_out && !aligned16(H_out)) || (X_out && !aligned16(X_out)))
        return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (delta && (delta_stride < cols || delta_stride % 4)) return PG_EINVAL;
    if (cols % 32 || cols > 16384 || n > 64) return PG_EUNSUPPORTED;
    const size_t need = prefill_gemm_q8_workspace_bytes(rows, cols, n);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PG_EWORKSPACE;
    // H_out and X_out are written while other rows of H and delta are still read
    // (H_out == H is allowed: each element is read and then written by one thread);
    // Y is written after the staging has finished.
    const size_t mb = (size_t)n * cols * sizeof(float);
    const size_t db = delta ? ((size_t)(n - 1) * delta_stride + cols) * sizeof(float) : 0;
    const void *outs[2] = {H_out, X_out};
    for (const void *o : outs)
        if ((o != H && overlaps(o, mb, H, mb)) || overlaps(o, mb, delta, db) ||
            overlaps(o, mb, w, cols * sizeof(float)))
            return PG_EINVAL;
    if (X_out && X_out == H) return PG_EINVAL;
    if (overlaps(H_out, mb, X_out, mb)) return PG_EINVAL;
    const size_t yb = (size_t)n * rows * sizeof(float);
    if (overlaps(Y, yb, workspace, need) || overlaps(H_out, mb, workspace, need) ||
        overlaps(X_out, mb, workspace, need))
        return PG_EINVAL;
    const StageNorm nm{H, delta, delta_stride, w, eps, H_out, X_out};
    return prefill_run(q, scale, bias, rows, cols, nullptr, &nm, n, Y, act, workspace, as_stream(stream));
}

// q8_2f prefill product (gemma_batch.rs, `encode_q82_mm`): the column field
// multiplies the activations as they are staged, the int8 body goes through the
// same matrix-core pass as the block format, and the f16 row scale multiplies
// each finished dot product.  The workspace is the block format's.
extern "C" int prefill_gemm_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field,
                                int32_t rows, int32_t cols, const float *X, int32_t n, float *Y, int32_t act,
                                void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    if (!q || !row_scale || !col_field || !X || !Y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || n <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(X) || !aligned16(Y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || n > 64) return PG_EUNSUPPORTED;
    const size_t need = prefill_gemm_q8_workspace_bytes(rows, cols, n);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PG_EWORKSPACE;
    const size_t yb = (size_t)n * rows * sizeof(float);
    if (overlaps(Y, yb, workspace, need)) return PG_EINVAL;
    hipStream_t s = as_stream(stream);
    char *ws = static_cast<char *>(workspace);
    const OneLayout L = one_layout(rows, cols, n);
    void *xp = ws, *xs = ws + L.xs;
    unsigned *tickets = reinterpret_cast<unsigned *>(ws + L.tickets);
    int rc = launch_stage_frag(X, n, cols, xp, xs, tickets, dense_panels(rows), s, col_field);
    if (rc) return rc;
    DenseArgs P{};
    P.q = q;
    P.rs = row_scale;
    P.rows = rows;
    P.cols = cols;
    P.n = n;
    P.out = Y;
    P.ldo = rows;
    P.act = act;
    P.mode = kDensePlain;
    return run_dense(P, xp, xs, reinterpret_cast<float *>(ws + L.parts), tickets, s, kFmtQ82);
}

// q4tp prefill product (nemotron_prefill.rs, `pb_q4_bank` and its nibble and
// code readers): the block format's matrix-core pass with the nibbles as
// weights, the group scale 2^(base + code step) in place of the block scale
// and -8 * scale as the group's bias (the nibble n enters as itself).
extern "C" int prefill_gemm_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t rows,
                                 int32_t cols, const float *X, int32_t n, float *Y, int32_t act, void *workspace,
                                 size_t workspace_bytes, pg_stream_t stream) {
    if (!nib || !params || !codes || !X || !Y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || n <= 0) return PG_EINVAL;
    if (!aligned16(nib) || !aligned16(X) || !aligned16(Y) || ((uintptr_t)params & 3) || ((uintptr_t)codes & 3))
        return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || n > 64) return PG_EUNSUPPORTED;
    const size_t need = prefill_gemm_q8_workspace_bytes(rows, cols, n);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PG_EWORKSPACE;
    const size_t yb = (size_t)n * rows * sizeof(float);
    if (overlaps(Y, yb, workspace, need) || overlaps(Y, yb, X, (size_t)n * cols * sizeof(float))) return PG_EINVAL;
    hipStream_t s = as_stream(stream);
    char *ws = static_cast<char *>(workspace);
    const OneLayout L = one_layout(rows, cols, n);
    void *xp = ws, *xs = ws + L.xs;
    unsigned *tickets = reinterpret_cast<unsigned *>(ws + L.tickets);
    int rc = launch_stage_frag(X, n, cols, xp, xs, tickets, dense_panels(rows), s);
    if (rc) return rc;
    DenseArgs P{};
    P.nib = nib;
    P.params = params;
    P.codes = codes;
    P.code_stride = (5 * (cols / 32) + 7) / 8;
    P.code_bytes = (uint32_t)rows * (uint32_t)P.code_stride;
    P.rows = rows;
    P.cols = cols;
    P.n = n;
    P.out = Y;
    P.ldo = rows;
    P.act = act;
    P.mode = kDensePlain;
    return run_dense(P, xp, xs, reinterpret_cast<float *>(ws + L.parts), tickets, s, kFmtQ4);
}

// ---------------------------------------------------------------- prefill frame
// The four products of the layer frame over one pass of n positions, five
// launches: the x0 staging, then QKV, up, down and head, each dense pass
// finishing the add + RMSNorm work around it in its epilogue (DenseMode) and
// staging the next product's activations there.
namespace {

struct FrameLayout {
    size_t xp[4], xs[4];    // staged activations of the four products
    size_t tickets[4];      // split tickets; tickets[0] .. the end of xs[3] are cleared by the first launch
    size_t sumsq1, sumsq2;  // [ceil(H / 128)][n]
    size_t parts, total;
};

FrameLayout frame_layout(int H, int qkv_rows, int I, int V, int n) {
    FrameLayout L;
    const int cols[4] = {H, H, I, H}, rows[4] = {qkv_rows, I, H, V};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes, 256);
        return at;
    };
    for (int i = 0; i < 4; ++i) L.xp[i] = take(frag_x_bytes(n, cols[i]));
    L.xs[0] = take(frag_s_bytes(n, cols[0]));
    for (int i = 0; i < 4; ++i) L.tickets[i] = take((size_t)dense_panels(rows[i]) * 4);
    for (int i = 1; i < 4; ++i) L.xs[i] = take(frag_s_bytes(n, cols[i]));
    const int hp = ceil_div(H, 128);
    L.sumsq1 = take((size_t)hp * n * 4);
    L.sumsq2 = take((size_t)hp * n * 4);
    size_t pb = 0;
    for (int i = 0; i < 4; ++i) pb = std::max(pb, parts_bytes(rows[i], cols[i], n));
    L.parts = take(pb);
    L.total = o;
    return L;
}

}  // namespace

extern "C" size_t prefill_frame_q8_workspace_bytes(int32_t hidden, int32_t qkv_rows, int32_t inter, int32_t vocab,
                                                   int32_t n) {
    if (hidden <= 0 || qkv_rows <= 0 || inter <= 0 || vocab <= 0 || n <= 0 || n > 64) return 0;
    if (hidden % 32 || inter % 32) return 0;
    return frame_layout(hidden, qkv_rows, inter, vocab, n).total;
}

// The frame behind prefill_frame_q8 (meta NULL: n positions at X0, H and the
// outputs) and prefill_frame_q8_meta (meta: device {n, pos0}; n here is the
// largest pass, 64, and the buffers hold rows_total rows).
static int frame_run(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                     const float *w1, const float *w2, float eps, const float *X0, float *H, int n,
                     const int32_t *meta, int rows_total, float *qkv, float *u, float *d, float *logits,
                     void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    if (!qkv_w || !up_w || !down_w || !head_w || !w1 || !w2 || !X0 || !H || !qkv || !u || !d || !logits)
        return PG_EINVAL;
    if (!(eps >= 0.0f) || n <= 0 || rows_total <= 0) return PG_EINVAL;
    const pg_q8 *Ws[4] = {qkv_w, up_w, down_w, head_w};
    for (const pg_q8 *W : Ws) {
        if (!W->q || !W->scale || !W->bias || W->rows <= 0 || W->cols <= 0) return PG_EINVAL;
        if (!aligned16(W->q) || !aligned16(W->scale) || !aligned16(W->bias)) return PG_EINVAL;
        if (W->cols % 32) return PG_EUNSUPPORTED;
    }
    const int Hd = qkv_w->cols, I = up_w->rows;
    if (qkv_w->rows < Hd || up_w->cols != Hd || down_w->cols != I || down_w->rows != Hd || head_w->cols != Hd)
        return PG_EINVAL;
    if (n > 64) return PG_EUNSUPPORTED;
    const float *ptrs[] = {w1, w2, X0, H, qkv, u, d, logits};
    for (const float *p : ptrs)
        if (!aligned16(p)) return PG_EINVAL;
    if (meta && ((uintptr_t)meta & 7)) return PG_EINVAL;
    const FrameLayout L = frame_layout(Hd, qkv_w->rows, I, head_w->rows, n);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return PG_EWORKSPACE;
    {   // workgroups write the outputs while others still read the inputs
        const size_t R = (size_t)rows_total;
        const size_t hb = R * Hd * sizeof(float), vb = (size_t)Hd * sizeof(float);
        const Span sp[] = {{X0, hb}, {H, hb}, {w1, vb}, {w2, vb}, {qkv, R * qkv_w->rows * sizeof(float)},
                           {u, R * I * sizeof(float)}, {d, hb}, {logits, R * head_w->rows * sizeof(float)},
                           {workspace, L.total}, {meta, meta ? 8u : 0u}};
        if (any_overlap(sp)) return PG_EINVAL;
    }
    char *ws = static_cast<char *>(workspace);
    hipStream_t s = as_stream(stream);
    auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
    auto tick = [&](int i) { return reinterpret_cast<unsigned *>(ws + L.tickets[i]); };
    const int nzero = (int)((L.xs[3] + round_up(frag_s_bytes(n, Hd), 256) - L.tickets[0]) / 4);
    int rc = launch_stage_frag(X0, n, Hd, at(L.xp[0]), at(L.xs[0]), tick(0), nzero, s, nullptr, meta, rows_total);
    if (rc) return rc;
    float *parts = reinterpret_cast<float *>(ws + L.parts);
    float *ss1 = reinterpret_cast<float *>(ws + L.sumsq1), *ss2 = reinterpret_cast<float *>(ws + L.sumsq2);
    auto base = [&](const pg_q8 *W, float *out) {
        DenseArgs P{};
        P.q = W->q;
        P.scale = W->scale;
        P.bias = W->bias;
        P.rows = W->rows;
        P.cols = W->cols;
        P.n = n;
        P.out = out;
        P.ldo = W->rows;
        P.hidden = Hd;
        P.eps = eps;
        P.meta = meta;
        P.rows_total = rows_total;
        P.nl = n;
        return P;
    };
    auto next = [&](DenseArgs &P, int i, int cols) {
        P.nxp = reinterpret_cast<u32x4 *>(at(L.xp[i]));
        P.nxs = reinterpret_cast<__bf16 *>(at(L.xs[i]));
        P.nnb = cols / 32;
    };
    // QKV: h1 = h + qkv[:, :H] into H, w1 * h1 staged for up, sums of h1^2.
    DenseArgs P = base(qkv_w, qkv);
    P.mode = kDenseResid;
    P.H = H;
    P.w = w1;
    P.sumsq = ss1;
    next(P, 1, Hd);
    if ((rc = run_dense(P, at(L.xp[0]), at(L.xs[0]), parts, tick(0), s))) return rc;
    // up: u = relu^2(W (w1 * h1) / rms(h1)), staged for down.
    P = base(up_w, u);
    P.mode = kDenseScaled;
    P.act = 1;
    P.sumsq_in = ss1;
    next(P, 2, I);
    if ((rc = run_dense(P, at(L.xp[1]), at(L.xs[1]), parts, tick(1), s))) return rc;
    // down: h2 = h1 + d into H, w2 * h2 staged for the head, sums of h2^2.
    P = base(down_w, d);
    P.mode = kDenseResid;
    P.H = H;
    P.w = w2;
    P.sumsq = ss2;
    next(P, 3, Hd);
    if ((rc = run_dense(P, at(L.xp[2]), at(L.xs[2]), parts, tick(2), s))) return rc;
    // head: logits = W (w2 * h2) / rms(h2).
    P = base(head_w, logits);
    P.mode = kDenseScaled;
    P.sumsq_in = ss2;
    return run_dense(P, at(L.xp[3]), at(L.xs[3]), parts, tick(3), s);
}

extern "C" int prefill_frame_q8(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                                const float *w1, const float *w2, float eps, const float *X0, float *H, int32_t n,
                                float *qkv, float *u, float *d, float *logits, void *workspace,
                                size_t workspace_bytes, pg_stream_t stream) {
    if (n <= 0) return PG_EINVAL;
    return frame_run(qkv_w, up_w, down_w, head_w, w1, w2, eps, X0, H, n, nullptr, n, qkv, u, d, logits, workspace,
                     workspace_bytes, stream);
}

extern "C" int prefill_frame_q8_meta(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w,
                                     const pg_q8 *head_w, const float *w1, const float *w2, float eps,
                                     const float *X0, float *H, int32_t rows_total, const int32_t *meta, float *qkv,
                                     float *u, float *d, float *logits, void *workspace, size_t workspace_bytes,
                                     pg_stream_t stream) {
    if (!meta) return PG_EINVAL;
    return frame_run(qkv_w, up_w, down_w, head_w, w1, w2, eps, X0, H, 64, meta, rows_total, qkv, u, d, logits,
                     workspace, workspace_bytes, stream);
}
