// Fused residual add + RMSNorm per position, and the MoE variant that adds
// the routing-weighted expert sum (nemotron_prefill.rs, `pb_add_rms`, add = 1
// and add = 2; gemma_batch.rs, `g4_add_norm_b`).  One workgroup per position:
// the stage reads only activations, so the fusion costs no pass over weights.
#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kNormThreads = 256;
constexpr int kNormMaxV = 16;  // float4 per thread: hidden <= 16384

// Sum over the workgroup; every thread receives the total.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kNormThreads / kWave; ++i) t += red[i];
    return t;
}

// h' = h + delta (optional, rows delta_stride floats apart); out = w * (h' * rsqrt(mean(h'^2) + eps)).
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    float *__restrict__ h, const float *__restrict__ delta, int delta_stride,
    const float *__restrict__ w, float eps, int hidden, float *__restrict__ out) {
    __shared__ float red[kNormThreads / kWave];
    const int b = blockIdx.x;
    const int h4 = hidden >> 2;
    float4 *hr = reinterpret_cast<float4 *>(h + (long long)b * hidden);
    const float4 *dr = delta ? reinterpret_cast<const float4 *>(delta + (long long)b * delta_stride) : nullptr;
    float4 v[kNormMaxV];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kNormMaxV; ++k) {
        const int i = threadIdx.x + k * kNormThreads;
        if (i < h4) {
            float4 a = hr[i];
            if (dr) {
                const float4 d = dr[i];
                a.x += d.x; a.y += d.y; a.z += d.z; a.w += d.w;
                hr[i] = a;
            }
            v[k] = a;
            ss += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
        }
    }
    const float inv = rsqrtf(block_sum(ss, red) / (float)hidden + eps);
    const float4 *wr = reinterpret_cast<const float4 *>(w);
    float4 *orow = reinterpret_cast<float4 *>(out + (long long)b * hidden);
#pragma unroll
    for (int k = 0; k < kNormMaxV; ++k) {
        const int i = threadIdx.x + k * kNormThreads;
        if (i < h4) {
            const float4 g = wr[i];
            orow[i] = make_float4(g.x * (v[k].x * inv), g.y * (v[k].y * inv), g.z * (v[k].z * inv),
                                  g.w * (v[k].w * inv));
        }
    }
}

// MoE combine: h' = h + sum_t rw[b][t] * D[b*k + t] (slot order t ascending);
// out = w * (h' * rsqrt(mean(h'^2) + eps)).
__global__ __launch_bounds__(kNormThreads) void moe_combine_kernel(
    float *__restrict__ h, const float *__restrict__ D, const float *__restrict__ rw, int k,
    const float *__restrict__ w, float eps, int hidden, float *__restrict__ out) {
    __shared__ float red[kNormThreads / kWave];
    const int b = blockIdx.x;
    const int h4 = hidden >> 2;
    float4 *hr = reinterpret_cast<float4 *>(h + (long long)b * hidden);
    float4 v[kNormMaxV];
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kNormMaxV; ++kk) {
        const int i = threadIdx.x + kk * kNormThreads;
        if (i < h4) {
            float4 m = make_float4(0, 0, 0, 0);
            for (int t = 0; t < k; ++t) {
                const float c = rw[b * k + t];
                const float4 d = reinterpret_cast<const float4 *>(D + (long long)(b * k + t) * hidden)[i];
                m.x = fmaf(c, d.x, m.x); m.y = fmaf(c, d.y, m.y);
                m.z = fmaf(c, d.z, m.z); m.w = fmaf(c, d.w, m.w);
            }
            float4 a = hr[i];
            a.x += m.x; a.y += m.y; a.z += m.z; a.w += m.w;
            hr[i] = a;
            v[kk] = a;
            ss += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
        }
    }
    const float inv = rsqrtf(block_sum(ss, red) / (float)hidden + eps);
    const float4 *wr = reinterpret_cast<const float4 *>(w);
    float4 *orow = reinterpret_cast<float4 *>(out + (long long)b * hidden);
#pragma unroll
    for (int kk = 0; kk < kNormMaxV; ++kk) {
        const int i = threadIdx.x + kk * kNormThreads;
        if (i < h4) {
            const float4 g = wr[i];
            orow[i] = make_float4(g.x * (v[kk].x * inv), g.y * (v[kk].y * inv),
                                  g.z * (v[kk].z * inv), g.w * (v[kk].w * inv));
        }
    }
}

int launch_moe_combine(float *h, const float *D, const float *rw, int n, int k, const float *w,
                       float eps, int hidden, float *out, hipStream_t s) {
    hipLaunchKernelGGL(moe_combine_kernel, dim3(n), dim3(kNormThreads), 0, s, h, D, rw, k, w, eps,
                       hidden, out);
    return launch_status();
}

}  // namespace pg

using namespace pg;

static bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x < y + bn && y < x + an;
}

extern "C" int add_rmsnorm(float *h, const float *delta, int32_t delta_stride, const float *w,
                           float eps, int32_t hidden, int32_t n, float *out, pg_stream_t stream) {
    if (!h || !w || !out) return PG_EINVAL;
    if (hidden <= 0 || n <= 0) return PG_EINVAL;
    if (delta && delta_stride < hidden) return PG_EINVAL;
    if (!aligned16(h) || !aligned16(w) || !aligned16(out) || (delta && !aligned16(delta)))
        return PG_EINVAL;
    if (hidden % 4 || hidden > kNormThreads * 4 * kNormMaxV) return PG_EUNSUPPORTED;
    if (delta && delta_stride % 4) return PG_EUNSUPPORTED;
    const size_t hb = (size_t)n * hidden * sizeof(float);
    if (overlaps(out, hb, h, hb)) return PG_EINVAL;
    if (delta && overlaps(out, hb, delta, (size_t)((n - 1) * (size_t)delta_stride + hidden) * sizeof(float)))
        return PG_EINVAL;
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(n), dim3(kNormThreads), 0, as_stream(stream), h,
                       delta, delta ? delta_stride : hidden, w, eps, hidden, out);
    return launch_status();
}
