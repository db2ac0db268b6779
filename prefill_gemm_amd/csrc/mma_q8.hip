// Batched prefill product (prefill_gemm_q8) and the activation staging it
// shares with the grouped expert banks.
//
// nemotron_prefill.rs (module doc): a pass holds up to 64 positions and every
// weight is read once per pass.  gemma_batch.rs (`encode_q82_mm`): the prompt
// GEMM computes y[nb][rows] = x[nb][cols] . W^T and refuses (encodes nothing
// for) shapes its tile does not cover.
#include <algorithm>

#include "mma_q8.h"
#include "mma_launch.h"
#include "pg_host.h"

namespace pg {

constexpr int kWch = 2;  // weight chunks in flight per wave

// One thread per (row, 16-column half block), over rows + 1 rows (the last is
// the zero row) and 16 * ng blocks per row (blocks past the last give zeros in xs).
__global__ __launch_bounds__(256) void stage_x_kernel(const float *__restrict__ X, int rows,
                                                      int cols, uint4 *__restrict__ xp,
                                                      __bf16 *__restrict__ xs) {
    const int nb = cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int per_row = ng * 32;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int row = (int)(t / per_row);
    const int hb = (int)(t % per_row);
    const int blk = hb >> 1, h = hb & 1;
    if (row > rows) return;
    const bool live = row < rows && blk < nb;
    float v[16];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(X + (long long)row * cols + 32 * blk + 16 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = src[j];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    __bf16 hi[16], lo[16];
    float half_sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        hi[i] = to_bf16(v[i]);
        lo[i] = to_bf16(v[i] - (float)hi[i]);
        half_sum += v[i];
    }
    if (blk < nb) {
        uint4 rec[4];
        __builtin_memcpy(&rec[0], &hi[0], 16);
        __builtin_memcpy(&rec[1], &hi[8], 16);
        __builtin_memcpy(&rec[2], &lo[0], 16);
        __builtin_memcpy(&rec[3], &lo[8], 16);
        uint4 *dst = xp + (((long long)row * nb + blk) * 2 + h) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = rec[j];
    }
    const float block_sum = half_sum + __shfl_xor(half_sum, 1, kWave);
    if (h == 0) {
        const __bf16 s_hi = to_bf16(block_sum);
        const __bf16 s_lo = to_bf16(block_sum - (float)s_hi);
        const int g = blk >> 4, hh = (blk >> 3) & 1, i = blk & 7;
        __bf16 *rec = xs + (((long long)row * ng + g) * 2 + hh) * 16;
        rec[i] = s_hi;
        rec[8 + i] = s_lo;
    }
}

// Fragment layout for the dense pass (see mma_q8.h): one thread per (row m,
// 16-column half block) over mts * 32 rows (rows >= n are zero) and 16 * ng blocks.
__global__ __launch_bounds__(256) void stage_x_frag_kernel(const float *__restrict__ X, int n,
                                                           int cols, int mts, u32x4 *__restrict__ xp,
                                                           __bf16 *__restrict__ xs) {
    const int nb = cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int per_row = ng * 32;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int m = (int)(t / per_row);
    const int hb = (int)(t % per_row);
    const int blk = hb >> 1, h = hb & 1;
    if (m >= mts * 32) return;
    const int mt = m >> 5, lane = (m & 31) + 32 * h;
    const bool live = m < n && blk < nb;
    float v[16];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(X + (long long)m * cols + 32 * blk + 16 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = src[j];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    __bf16 hi[16], lo[16];
    float half_sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        hi[i] = to_bf16(v[i]);
        lo[i] = to_bf16(v[i] - (float)hi[i]);
        half_sum += v[i];
    }
    if (blk < nb) {
        u32x4 rec[4];
        __builtin_memcpy(&rec[0], &hi[0], 16);
        __builtin_memcpy(&rec[1], &hi[8], 16);
        __builtin_memcpy(&rec[2], &lo[0], 16);
        __builtin_memcpy(&rec[3], &lo[8], 16);
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) xp[(((long long)blk * mts + mt) * 4 + fi) * 64 + lane] = rec[fi];
    }
    const float block_sum = half_sum + __shfl_xor(half_sum, 1, kWave);
    if (h == 0) {
        const __bf16 s_hi = to_bf16(block_sum);
        const __bf16 s_lo = to_bf16(block_sum - (float)s_hi);
        const int g = blk >> 4, hh = (blk >> 3) & 1, i = blk & 7;
        const int sl = (m & 31) + 32 * hh;
        xs[((((long long)g * mts + mt) * 2 + 0) * 64 + sl) * 8 + i] = s_hi;
        xs[((((long long)g * mts + mt) * 2 + 1) * 64 + sl) * 8 + i] = s_lo;
    }
}

int launch_stage_x(const float *X, int rows, int cols, void *xp, void *xs, hipStream_t s) {
    const int nb = cols / 32, ng = (nb + 15) / 16;
    const long long threads = (long long)(rows + 1) * ng * 32;
    const int grid = (int)((threads + 255) / 256);
    hipLaunchKernelGGL(stage_x_kernel, dim3(grid), dim3(256), 0, s, X, rows, cols,
                       reinterpret_cast<uint4 *>(xp), reinterpret_cast<__bf16 *>(xs));
    return launch_status();
}

// Dense pass: workgroup id -> (panel of 128 rows, K split).  Splits of one
// panel take consecutive ids, so with 8 or fewer splits the workgroups that
// read the same activation blocks land on the same XCD (ids are dealt to the
// 8 XCDs round robin).
template <int MT>
__global__ __launch_bounds__(kMmaThreads) void mma_dense_kernel(MmaPanel P, int splits, int bps,
                                                        float *partials, long long plane) {
    __shared__ u32x4 lds[2 * kChunk * MT * 4 * 64];
    const int id = blockIdx.x;
    const int split = id % splits, panel = id / splits;
    const int nb = P.cols >> 5;
    const int kb0 = split * bps;
    const int kb1 = min(nb, kb0 + bps);
    if (splits > 1) {
        P.out = partials + (long long)split * plane;
        P.act = 0;
    }
    mma_panel<MT, kWch>(P, panel * kPanelRows, kb0, kb1, lds);
}

// Y[i] = act( sum_{s < splits} parts[s][i] ), the splits added in order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ parts,
                                                            int splits, long long plane,
                                                            float *__restrict__ Y, int act) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= plane) return;
    float acc = parts[i];
    for (int s = 1; s < splits; ++s) acc += parts[(long long)s * plane + i];
    Y[i] = apply_act(act, acc);
}

// Grouped expert bank: workgroup (panel of 128 rows, expert e).  An expert no
// position chose returns at once (nemotron_prefill.rs, `pb_q8_bank`: cnt == 0).
__global__ __launch_bounds__(kMmaThreads) void mma_expert_kernel(MmaPanel P, const int32_t *counts,
                                                         const int32_t *lists, int cap,
                                                         long long q_stride, long long s_stride) {
    __shared__ u32x4 lds[2 * kChunk * 2 * 4 * 64];
    const int e = blockIdx.y;
    const int cnt = min(counts[e], min(cap, 64));
    if (cnt <= 0) return;
    P.q += e * q_stride;
    P.scale += e * s_stride;
    P.bias += e * s_stride;
    P.src_list = lists + (long long)e * cap;
    P.out_list = lists + (long long)e * cap;
    P.m_valid = cnt;
    const int nb = P.cols >> 5;
    if (cnt > 32)
        mma_panel<2, kWch>(P, blockIdx.x * kPanelRows, 0, nb, lds);
    else
        mma_panel<1, kWch>(P, blockIdx.x * kPanelRows, 0, nb, lds);
}

int launch_expert_bank(const MmaPanel &P, int experts, const int32_t *counts,
                       const int32_t *lists, int cap, hipStream_t s) {
    const long long q_stride = (long long)P.rows * P.cols;
    const long long s_stride = (long long)P.rows * (P.cols / 32);
    dim3 grid(ceil_div(P.rows, kPanelRows), experts);
    hipLaunchKernelGGL(mma_expert_kernel, grid, dim3(kMmaThreads), 0, s, P, counts, lists, cap, q_stride,
                       s_stride);
    return launch_status();
}

// K splits of a dense pass: enough workgroups to cover the 256 compute units
// without cutting a split below 8 blocks; large matrices run unsplit.
int dense_splits(int rows, int cols) {
    const int panels = ceil_div(rows, kPanelRows);
    const int nb = cols / 32;
    if (panels >= 200) return 1;
    int s = ceil_div(256, panels);
    s = std::min(s, std::max(1, nb / 8));
    return std::max(1, s);
}

}  // namespace pg

using namespace pg;

// Fragment-layout staging sizes of n rows (mts tiles of 32 rows).
static size_t frag_x_bytes(int n, int cols) { return (size_t)ceil_div(n, 32) * cols * 128; }
static size_t frag_s_bytes(int n, int cols) {
    return (size_t)ceil_div(n, 32) * ceil_div(cols / 32, 16) * 2048;
}

extern "C" size_t prefill_gemm_q8_workspace_bytes(int32_t rows, int32_t cols, int32_t n) {
    if (rows <= 0 || cols <= 0 || n <= 0 || cols % 32) return 0;
    size_t bytes = round_up(frag_x_bytes(n, cols), 256) + round_up(frag_s_bytes(n, cols), 256);
    const int s = dense_splits(rows, cols);
    if (s > 1) bytes += (size_t)s * n * rows * sizeof(float);
    return bytes;
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
    hipStream_t s = as_stream(stream);

    char *ws = static_cast<char *>(workspace);
    void *xp = ws;
    void *xs = ws + round_up(frag_x_bytes(n, cols), 256);
    float *parts = reinterpret_cast<float *>(ws + round_up(frag_x_bytes(n, cols), 256) +
                                             round_up(frag_s_bytes(n, cols), 256));
    const int mts = ceil_div(n, 32);
    {
        const int nb = cols / 32, ng = (nb + 15) / 16;
        const long long threads = (long long)mts * 32 * ng * 32;
        hipLaunchKernelGGL(stage_x_frag_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           X, n, cols, mts, reinterpret_cast<u32x4 *>(xp), reinterpret_cast<__bf16 *>(xs));
        int rc = launch_status();
        if (rc) return rc;
    }
    int rc = PG_OK;

    MmaPanel P{};
    P.q = q;
    P.scale = scale;
    P.bias = bias;
    P.rows = rows;
    P.cols = cols;
    P.xp = reinterpret_cast<const u32x4 *>(xp);
    P.xs = reinterpret_cast<const u32x4 *>(xs);
    P.zero_row = n;
    P.frag = 1;
    P.src_list = nullptr;
    P.src_div = 1;
    P.m_valid = n;
    P.out = Y;
    P.ldo = rows;
    P.out_list = nullptr;
    P.act = act;

    const int splits = dense_splits(rows, cols);
    const int nb = cols / 32;
    const int bps = ceil_div(nb, splits);
    const int used = ceil_div(nb, bps);  // splits that hold at least one block
    const int grid = ceil_div(rows, kPanelRows) * used;
    const long long plane = (long long)n * rows;
    if (n > 32)
        hipLaunchKernelGGL(mma_dense_kernel<2>, dim3(grid), dim3(kMmaThreads), 0, s, P, used, bps, parts, plane);
    else
        hipLaunchKernelGGL(mma_dense_kernel<1>, dim3(grid), dim3(kMmaThreads), 0, s, P, used, bps, parts, plane);
    rc = launch_status();
    if (rc || used == 1) return rc;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((plane + 255) / 256)), dim3(256), 0, s,
                       parts, used, plane, Y, act);
    return launch_status();
}
