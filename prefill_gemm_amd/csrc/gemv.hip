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

template <int RW, int U>
__global__ __launch_bounds__(kGemvThreads) void gemv_q8_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
    int rows, int cols, const float *__restrict__ x, float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 4;
    const int steps = (nseg + 63) >> 6;
    const int nb = cols >> 5;
    float *seg_sum = reinterpret_cast<float *>(sx + steps * 4 * 64);

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

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ngroups = (rows + kGemvWaves * RW - 1) / (kGemvWaves * RW);
    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int r0 = (g * kGemvWaves + wave) * RW;
        float acc[RW];
        const int8_t *qr[RW];
        const float *sr[RW], *br[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            acc[rr] = 0.0f;
            const long long r = min(r0 + rr, rows - 1);
            qr[rr] = q + r * cols;
            sr[rr] = scale + r * nb;
            br[rr] = bias + r * nb;
        }
        for (int i0 = 0; i0 < steps; i0 += U) {
            uint4 w[U][RW];
            float sc[U][RW], bi[U][RW];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = lane + 64 * (i0 + u);
                const bool ok = s < nseg;
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    w[u][rr] = ok ? *reinterpret_cast<const uint4 *>(qr[rr] + 16 * s) : make_uint4(0, 0, 0, 0);
                    sc[u][rr] = ok ? sr[rr][s >> 1] : 0.0f;
                    bi[u][rr] = ok ? br[rr][s >> 1] : 0.0f;
                }
            }
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
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const float v = wave_sum(acc[rr]);
            if (lane == rr && r0 + rr < rows) y[r0 + rr] = apply_act(act, v);
        }
    }
}

template <int RW, int U>
__global__ __launch_bounds__(kGemvThreads) void gemv_f16_kernel(
    const uint16_t *__restrict__ w16, int rows, int cols, const float *__restrict__ x,
    float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 3;
    const int steps = (nseg + 63) >> 6;
    for (int s = threadIdx.x; s < steps * 64; s += kGemvThreads) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sx[xslot<2>(s, j)] =
                s < nseg ? reinterpret_cast<const float4 *>(x)[2 * s + j] : make_float4(0, 0, 0, 0);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ngroups = (rows + kGemvWaves * RW - 1) / (kGemvWaves * RW);
    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int r0 = (g * kGemvWaves + wave) * RW;
        float acc[RW];
        const uint16_t *wr[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            acc[rr] = 0.0f;
            wr[rr] = w16 + (long long)min(r0 + rr, rows - 1) * cols;
        }
        for (int i0 = 0; i0 < steps; i0 += U) {
            uint4 wv[U][RW];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = lane + 64 * (i0 + u);
#pragma unroll
                for (int rr = 0; rr < RW; ++rr)
                    wv[u][rr] = s < nseg ? *reinterpret_cast<const uint4 *>(wr[rr] + 8 * s) : make_uint4(0, 0, 0, 0);
            }
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
                        __builtin_memcpy(hv, &wv[u][rr], 16);
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
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const float v = wave_sum(acc[rr]);
            if (lane == rr && r0 + rr < rows) y[r0 + rr] = apply_act(act, v);
        }
    }
}

constexpr int kQ8Rw = 2, kQ8U = 4;
constexpr int kF16Rw = 2, kF16U = 8;
constexpr int kMaxLds = 160 * 1024;

static int gemv_grid(int rows, int rw, size_t lds_bytes) {
    const int groups = ceil_div(rows, kGemvWaves * rw);
    const int per_cu = std::max(1, std::min(8, (int)(kMaxLds / std::max<size_t>(lds_bytes, 1))));
    return std::max(1, std::min(groups, 256 * per_cu));
}

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
    hipLaunchKernelGGL((gemv_q8_kernel<kQ8Rw, kQ8U>), dim3(gemv_grid(rows, kQ8Rw, lds)),
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
    hipLaunchKernelGGL((gemv_f16_kernel<kF16Rw, kF16U>), dim3(gemv_grid(rows, kF16Rw, lds)),
                       dim3(kGemvThreads), lds, as_stream(stream), w, rows, cols, x, y, act);
    return launch_status();
}
