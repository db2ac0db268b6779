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
template <int THREADS = kNormThreads>
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < THREADS / kWave; ++i) t += red[i];
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

// MoE combine: h' = h + (shared[b] + sum_t rw[b][t] * D[b*k + t]) (the sum
// starting from the dense shared term when given, then slot order t ascending;
// nemotron_prefill.rs `pb_add_rms`, add = 2); out = w * (h' * rsqrt(mean(h'^2) + eps)).
// One workgroup of 1024 threads per position (a position's rows are few and
// short, so every load of the position should be in flight at once): the
// slots' rows come kCombT at a time, and each element adds them in slot order.
constexpr int kCombThreads = 1024;
constexpr int kCombV = 4;  // float4 per thread: hidden <= 16384
constexpr int kCombT = 4;  // slots requested together

__global__ __launch_bounds__(kCombThreads) void moe_combine_kernel(
    float *__restrict__ h, const float *__restrict__ shared, const float *__restrict__ D,
    const float *__restrict__ rw, int k, const float *__restrict__ w, float eps, int hidden,
    float *__restrict__ out) {
    __shared__ float red[kCombThreads / kWave];
    const int b = blockIdx.x;
    const int h4 = hidden >> 2;
    float4 *hr = reinterpret_cast<float4 *>(h + (long long)b * hidden);
    const float4 *sr = shared ? reinterpret_cast<const float4 *>(shared + (long long)b * hidden) : nullptr;
    float4 v[kCombV], m[kCombV];
#pragma unroll
    for (int kk = 0; kk < kCombV; ++kk) {
        const int i = threadIdx.x + kk * kCombThreads;
        v[kk] = i < h4 ? hr[i] : make_float4(0, 0, 0, 0);
        m[kk] = sr && i < h4 ? sr[i] : make_float4(0, 0, 0, 0);
    }
    for (int t0 = 0; t0 < k; t0 += kCombT) {
        float c[kCombT];
        float4 d[kCombT][kCombV];
#pragma unroll
        for (int tt = 0; tt < kCombT; ++tt) {
            const int t = t0 + tt;
            c[tt] = t < k ? rw[b * k + t] : 0.0f;
            const float4 *dr = reinterpret_cast<const float4 *>(D + (long long)(b * k + min(t, k - 1)) * hidden);
#pragma unroll
            for (int kk = 0; kk < kCombV; ++kk) {
                const int i = threadIdx.x + kk * kCombThreads;
                d[tt][kk] = t < k && i < h4 ? dr[i] : make_float4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int tt = 0; tt < kCombT; ++tt) {
            if (t0 + tt >= k) break;
#pragma unroll
            for (int kk = 0; kk < kCombV; ++kk) {
                m[kk].x = fmaf(c[tt], d[tt][kk].x, m[kk].x); m[kk].y = fmaf(c[tt], d[tt][kk].y, m[kk].y);
                m[kk].z = fmaf(c[tt], d[tt][kk].z, m[kk].z); m[kk].w = fmaf(c[tt], d[tt][kk].w, m[kk].w);
            }
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kCombV; ++kk) {
        const int i = threadIdx.x + kk * kCombThreads;
        if (i < h4) {
            float4 a = v[kk];
            a.x += m[kk].x; a.y += m[kk].y; a.z += m[kk].z; a.w += m[kk].w;
            hr[i] = a;
            v[kk] = a;
            ss += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
        }
    }
    const float inv = rsqrtf(block_sum<kCombThreads>(ss, red) / (float)hidden + eps);
    const float4 *wr = reinterpret_cast<const float4 *>(w);
    float4 *orow = reinterpret_cast<float4 *>(out + (long long)b * hidden);
#pragma unroll
    for (int kk = 0; kk < kCombV; ++kk) {
        const int i = threadIdx.x + kk * kCombThreads;
        if (i < h4) {
            const float4 g = wr[i];
            orow[i] = make_float4(g.x * (v[kk].x * inv), g.y * (v[kk].y * inv),
                                  g.z * (v[kk].z * inv), g.w * (v[kk].w * inv));
        }
    }
}

int launch_moe_combine(float *h, const float *shared, const float *D, const float *rw, int n, int k, const float *w,
                       float eps, int hidden, float *out, hipStream_t s) {
    hipLaunchKernelGGL(moe_combine_kernel, dim3(n), dim3(kCombThreads), 0, s, h, shared, D, rw, k, w, eps,
                       hidden, out);
    return launch_status();
}

}  // namespace pg

using namespace pg;

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
