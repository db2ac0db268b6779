// Decode matrix-vector products at one position (gemv_q8, gemv_f16).
//
// embryo_wide.wgsl (header comment): the matrices stay in their packed form
// on the device and are read in 16-byte loads; the activation rides in the
// matrix stage.  Here each lane streams 16 bytes of a weight row per step and
// decodes them in registers; the activation vector sits in LDS in a
// lane-interleaved layout so the 64 lanes of a wave read it without bank
// conflicts; a row's partial sums are folded across the wave with shuffles.
//
// q8 block arithmetic per 16-column segment s of row r (half of a block):
//     acc += scale[r][s/2] * (sum_{c in s} q[r][c] * x[c]) + bias[r][s/2] * (sum_{c in s} x[c])
// which is sum_c (scale*q + bias)[r][c] * x[c] regrouped; the segment sums of
// x are computed once per workgroup.
#include <algorithm>

#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// x staging: segment s (16 columns for q8, 8 for f16) of `per` float4 goes to
// slot ((s / 64) * per + j) * 64 + (s % 64): lane l of step i reads slots
// (i * per + j) * 64 + l, consecutive across the wave.
template <int PER>
__device__ __forceinline__ int xslot(int s, int j) {
    return ((s >> 6) * PER + j) * 64 + (s & 63);
}

// One workgroup per group of 4 * RW rows; wave w owns rows r0 .. r0 + RW - 1.
// Lane l of step i covers segment s = l + 64 i.  Weights are requested in
// batches of U steps, one batch ahead of the arithmetic (the first batch
// before the activation is staged), from clamped in-bounds addresses; a
// segment past the end of the row meets zeros in the staged activation, so
// it adds nothing.
template <int RW, int U>
__global__ __launch_bounds__(kGemvThreads) void gemv_q8_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
    int rows, int cols, const float *__restrict__ x, float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 4;
    const int steps = (nseg + 63) >> 6;
    const int nb = cols >> 5;
    float *seg_sum = reinterpret_cast<float *>(sx + steps * 4 * 64);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * kGemvWaves + wave) * RW;

    const int8_t *qr[RW];
    const float *sr[RW], *br[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const long long r = min(r0 + rr, rows - 1);
        qr[rr] = q + r * cols;
        sr[rr] = scale + r * nb;
        br[rr] = bias + r * nb;
    }
    u32x4 wa[U][RW], wb[U][RW];
    float sa[U][RW], sb[U][RW], ba[U][RW], bb[U][RW];
    auto load = [&](int i0, u32x4 (&w)[U][RW], float (&sc)[U][RW], float (&bi)[U][RW])
        __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u < steps) {
                const int s = min(lane + 64 * (i0 + u), nseg - 1);
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    w[u][rr] = *reinterpret_cast<const u32x4 *>(qr[rr] + 16 * s);
                    sc[u][rr] = sr[rr][s >> 1];
                    bi[u][rr] = br[rr][s >> 1];
                }
            }
        }
    };
    load(0, wa, sa, ba);

    for (int s = threadIdx.x; s < steps * 64; s += kGemvThreads) {
        float4 a[4];
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = s < nseg ? reinterpret_cast<const float4 *>(x)[4 * s + j] : make_float4(0, 0, 0, 0);
            sum += (a[j].x + a[j].y) + (a[j].z + a[j].w);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sx[xslot<4>(s, j)] = a[j];
        seg_sum[s] = sum;
    }
    __syncthreads();

    float acc[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) acc[rr] = 0.0f;
    auto compute = [&](int i0, const u32x4 (&w)[U][RW], const float (&sc)[U][RW],
                       const float (&bi)[U][RW]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u;
            if (i < steps) {
                float xv[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a = sx[(i * 4 + j) * 64 + lane];
                    xv[4 * j] = a.x; xv[4 * j + 1] = a.y; xv[4 * j + 2] = a.z; xv[4 * j + 3] = a.w;
                }
                const float xs = seg_sum[i * 64 + lane];
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    float f[16];
                    q16_to_f32(w[u][rr], f);
                    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
                    for (int k = 0; k < 16; k += 2) {
                        d0 = fmaf(f[k], xv[k], d0);
                        d1 = fmaf(f[k + 1], xv[k + 1], d1);
                    }
                    acc[rr] = fmaf(sc[u][rr], d0 + d1, acc[rr]);
                    acc[rr] = fmaf(bi[u][rr], xs, acc[rr]);
                }
            }
        }
    };
    for (int i0 = 0; i0 < steps; i0 += 2 * U) {
        load(i0 + U, wb, sb, bb);
        compute(i0, wa, sa, ba);
        load(i0 + 2 * U, wa, sa, ba);
        compute(i0 + U, wb, sb, bb);
    }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const float v = wave_sum(acc[rr]);
        if (lane == rr && r0 + rr < rows) y[r0 + rr] = apply_act(act, v);
    }
}

// f16 weights: segment = 8 columns (16 bytes); same batching as gemv_q8_kernel.
template <int RW, int U>
__global__ __launch_bounds__(kGemvThreads) void gemv_f16_kernel(
    const uint16_t *__restrict__ w16, int rows, int cols, const float *__restrict__ x,
    float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 3;
    const int steps = (nseg + 63) >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * kGemvWaves + wave) * RW;
    const uint16_t *wr[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) wr[rr] = w16 + (long long)min(r0 + rr, rows - 1) * cols;
    u32x4 wa[U][RW], wb[U][RW];
    auto load = [&](int i0, u32x4 (&w)[U][RW]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u < steps) {
                const int s = min(lane + 64 * (i0 + u), nseg - 1);
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) w[u][rr] = *reinterpret_cast<const u32x4 *>(wr[rr] + 8 * s);
            }
        }
    };
    load(0, wa);
    for (int s = threadIdx.x; s < steps * 64; s += kGemvThreads) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sx[xslot<2>(s, j)] =
                s < nseg ? reinterpret_cast<const float4 *>(x)[2 * s + j] : make_float4(0, 0, 0, 0);
    }
    __syncthreads();

    float acc[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) acc[rr] = 0.0f;
    auto compute = [&](int i0, const u32x4 (&w)[U][RW]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u;
            if (i < steps) {
                const float4 a = sx[(i * 2) * 64 + lane];
                const float4 b = sx[(i * 2 + 1) * 64 + lane];
                const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    _Float16 hv[8];
                    __builtin_memcpy(hv, &w[u][rr], 16);
                    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; k += 2) {
                        d0 = fmaf((float)hv[k], xv[k], d0);
                        d1 = fmaf((float)hv[k + 1], xv[k + 1], d1);
                    }
                    acc[rr] += d0 + d1;
                }
            }
        }
    };
    for (int i0 = 0; i0 < steps; i0 += 2 * U) {
        load(i0 + U, wb);
        compute(i0, wa);
        load(i0 + 2 * U, wa);
        compute(i0 + U, wb);
    }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const float v = wave_sum(acc[rr]);
        if (lane == rr && r0 + rr < rows) y[r0 + rr] = apply_act(act, v);
    }
}

constexpr int kQ8Rw = 2, kQ8U = 2;
constexpr int kF16Rw = 2, kF16U = 4;
constexpr int kMaxLds = 160 * 1024;

static int gemv_grid(int rows, int rw) { return ceil_div(rows, kGemvWaves * rw); }

}  // namespace pg

using namespace pg;

extern "C" int gemv_q8(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                       int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream) {
    if (!q || !scale || !bias || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(x) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    const int steps = ceil_div(cols / 16, 64);
    const size_t lds = (size_t)steps * 4 * 64 * sizeof(float4) + (size_t)steps * 64 * sizeof(float);
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_q8_kernel<kQ8Rw, kQ8U>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        attr = true;
    }
    hipLaunchKernelGGL((gemv_q8_kernel<kQ8Rw, kQ8U>), dim3(gemv_grid(rows, kQ8Rw)),
                       dim3(kGemvThreads), lds, as_stream(stream), q, scale, bias, rows, cols, x,
                       y, act);
    return launch_status();
}

extern "C" int gemv_f16(const uint16_t *w, int32_t rows, int32_t cols, const float *x, float *y,
                        int32_t act, pg_stream_t stream) {
    if (!w || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 8 || cols > 32768) return PG_EUNSUPPORTED;
    const int steps = ceil_div(cols / 8, 64);
    const size_t lds = (size_t)steps * 2 * 64 * sizeof(float4);
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_f16_kernel<kF16Rw, kF16U>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        attr = true;
    }
    hipLaunchKernelGGL((gemv_f16_kernel<kF16Rw, kF16U>), dim3(gemv_grid(rows, kF16Rw)),
                       dim3(kGemvThreads), lds, as_stream(stream), w, rows, cols, x, y, act);
    return launch_status();
}
