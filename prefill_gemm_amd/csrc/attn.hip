// Causal grouped-query attention over one prefill pass, and the KV append
// (nemotron_prefill.rs: `pb_kv_append`, `pb_attn`, `pb_attn_merge`).
//
// The pass holds n positions at absolute positions pos0 .. pos0 + n - 1; their
// K and V rows go into the caches [pos][nkv][hd] first.  Query head h of
// position b then reads KV head g = h / (nh / nkv) and every key j <= pos0 + b:
//     o[b][h] = sum_j softmax_j((scale * q[b][h]) . k[j][g]) v[j][g].
//
// Work split: a workgroup takes one KV head, a block of 64 queries (64 / rep
// positions times the rep query heads that share the KV head, so each K and V
// row staged in LDS serves all of them) and one range of keys (a split).  Per
// tile of 64 keys, K and V are staged in LDS; each wave scores its 16 queries
// with one key per lane (q read from LDS by broadcast), keeps an online
// softmax per query (running max m and sum l), and then accumulates p . V with
// the lanes over the head dimensions.  A split writes (m, l, acc) per query;
// the merge kernel rescales the splits to a common maximum and adds them in
// split order.  Everything is f32, as on the pages.
#include <stdint.h>

#include <algorithm>

#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kAttnQ = 64;                     // queries per workgroup
constexpr int kAttnQW = kAttnQ / kAttnWaves;   // queries per wave
constexpr int kAttnKT = 64;                    // keys per tile
constexpr float kAttnNoMax = -1e30f;           // running max before any key

// Maximum over the wave without LDS: quad, half-row and row exchanges by DPP,
// then the four rows' results read out by readlane (wave-uniform result).
__device__ __forceinline__ float wave_max_dpp(float v) {
    auto dpp = [](float x, int ctrl) __attribute__((always_inline)) {
        switch (ctrl) {  // the control must be a constant expression
            case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
            case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
            case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
            default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
        }
    };
    v = fmaxf(v, dpp(v, 0));  // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp(v, 1));  // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp(v, 2));  // row_half_mirror
    v = fmaxf(v, dpp(v, 3));  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int HD>
struct AttnCfg {
    static constexpr int kKStride = HD + 4;    // floats; keeps lane-per-key reads off one bank
    static constexpr int kKFloats = kAttnKT * kKStride;
    static constexpr int kVFloats = kAttnKT * HD;
    static constexpr int kQFloats = kAttnQ * HD;
    static constexpr int kPFloats = kAttnWaves * kAttnQW * kAttnKT;
    static constexpr int kLdsFloats = kKFloats + kVFloats + kQFloats + kPFloats;
};

// Grid (split, query block, KV head).  part: [split][n][nh][hd + 2] (acc, m, l).
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_prefill_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc, int n, int pos0,
    int nh, int nkv, float scale, int chunk, float *__restrict__ part) {
    using C = AttnCfg<HD>;
    extern __shared__ float lds[];
    float *sk = lds;
    float *sv = sk + C::kKFloats;
    float *sq = sv + C::kVFloats;
    float *sp = sq + C::kQFloats;
    const int split = blockIdx.x, qblk = blockIdx.y, g = blockIdx.z;
    const int rep = nh / nkv, P = kAttnQ / rep;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b0 = qblk * P;
    const int bl = min(n, b0 + P) - 1;                    // last position of the block
    const int j0 = split * chunk;
    const int j1 = min(j0 + chunk, pos0 + bl + 1);        // keys past the block's last limit add nothing

    // Queries of the block, scaled: query i = position b0 + i / rep, head g * rep + i % rep.
    for (int t = threadIdx.x; t < kAttnQ * (HD / 4); t += kAttnThreads) {
        const int i = t / (HD / 4), d4 = t % (HD / 4);
        const int b = b0 + i / rep, h = g * rep + i % rep;
        float4 v = make_float4(0, 0, 0, 0);
        if (b < n) v = reinterpret_cast<const float4 *>(q + ((long long)b * nh + h) * HD)[d4];
        reinterpret_cast<float4 *>(sq + i * HD)[d4] = make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
    }

    // The wave's queries: qi = wave * 16 + r.  Key limit of each: pos0 + its position.
    int lim[kAttnQW];
#pragma unroll
    for (int r = 0; r < kAttnQW; ++r) {
        const int i = wave * kAttnQW + r;
        lim[r] = pos0 + b0 + i / rep;  // keys j <= lim (positions past n are never written)
    }
    float m[kAttnQW], l[kAttnQW];
    constexpr int DL = HD / 64;  // dims per lane in the p . V step
    float acc[kAttnQW][DL];
#pragma unroll
    for (int r = 0; r < kAttnQW; ++r) {
        m[r] = kAttnNoMax;
        l[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[r][e] = 0.0f;
    }

    for (int t0 = j0; t0 < j1; t0 += kAttnKT) {
        __syncthreads();  // the previous tile's K, V and p are no longer read
        // Stage the tile's K and V rows (keys t0 .. t0 + 63; rows past j1 stage zeros).
        constexpr int kRow4 = HD / 4;
        for (int t = threadIdx.x; t < kAttnKT * kRow4; t += kAttnThreads) {
            const int kk = t / kRow4, d4 = t % kRow4;
            const int j = t0 + kk;
            float4 a = make_float4(0, 0, 0, 0), c = make_float4(0, 0, 0, 0);
            if (j < j1) {
                const long long off = ((long long)j * nkv + g) * HD;
                a = reinterpret_cast<const float4 *>(kc + off)[d4];
                c = reinterpret_cast<const float4 *>(vc + off)[d4];
            }
            reinterpret_cast<float4 *>(sk + kk * C::kKStride)[d4] = a;
            reinterpret_cast<float4 *>(sv + kk * HD)[d4] = c;
        }
        __syncthreads();

        // Scores: lane = key t0 + lane, 16 queries.
        float s[kAttnQW];
#pragma unroll
        for (int r = 0; r < kAttnQW; ++r) s[r] = 0.0f;
        const float *krow = sk + lane * C::kKStride;
        const float *qw = sq + wave * kAttnQW * HD;
        for (int d = 0; d < HD; d += 4) {
            const float4 kv = *reinterpret_cast<const float4 *>(krow + d);
#pragma unroll
            for (int r = 0; r < kAttnQW; ++r) {
                const float4 qv = *reinterpret_cast<const float4 *>(qw + r * HD + d);
                s[r] = fmaf(qv.x, kv.x, s[r]);
                s[r] = fmaf(qv.y, kv.y, s[r]);
                s[r] = fmaf(qv.z, kv.z, s[r]);
                s[r] = fmaf(qv.w, kv.w, s[r]);
            }
        }
        // Online softmax per query; masked keys (past the query's limit or the
        // split) weigh exactly 0.  The running sum stays a per-lane partial
        // (every lane rescales by the same factor) and is folded once at the end.
        const int j = t0 + lane;
        float *pw = sp + wave * kAttnQW * kAttnKT;
#pragma unroll
        for (int r = 0; r < kAttnQW; ++r) {
            const bool ok = j < j1 && j <= lim[r];
            const float sc = ok ? s[r] : -INFINITY;
            const float mn = fmaxf(m[r], wave_max_dpp(sc));
            const float al = expf(m[r] - mn);
            const float p = ok ? expf(sc - mn) : 0.0f;
            l[r] = l[r] * al + p;
#pragma unroll
            for (int e = 0; e < DL; ++e) acc[r][e] *= al;
            m[r] = mn;
            pw[r * kAttnKT + lane] = p;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's p writes land before its reads (lgkmcnt 0)
        __builtin_amdgcn_wave_barrier();
        // p . V: lane owns dims lane * DL .. lane * DL + DL - 1.
        for (int kk = 0; kk < kAttnKT; ++kk) {
            float vv[DL];
#pragma unroll
            for (int e = 0; e < DL; ++e) vv[e] = sv[kk * HD + lane * DL + e];
#pragma unroll
            for (int r = 0; r < kAttnQW; ++r) {
                const float p = pw[r * kAttnKT + kk];
#pragma unroll
                for (int e = 0; e < DL; ++e) acc[r][e] = fmaf(p, vv[e], acc[r][e]);
            }
        }
    }

    // Partials of the wave's queries for this split.
#pragma unroll
    for (int r = 0; r < kAttnQW; ++r) l[r] = wave_sum(l[r]);
#pragma unroll
    for (int r = 0; r < kAttnQW; ++r) {
        const int i = wave * kAttnQW + r;
        const int b = b0 + i / rep, h = g * rep + i % rep;
        if (b >= n) continue;
        float *o = part + (((long long)split * n + b) * nh + h) * (HD + 2);
#pragma unroll
        for (int e = 0; e < DL; ++e) o[lane * DL + e] = acc[r][e];
        if (lane == 0) {
            o[HD] = m[r];
            o[HD + 1] = l[r];
        }
    }
}

// One wave per (position, query head): the splits rescaled to their common
// maximum and added in split order.
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(const float *__restrict__ part, int n, int nh,
                                                                  int splits, float *__restrict__ o) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * kAttnWaves + (threadIdx.x >> 6);  // b * nh + h
    if (i >= n * nh) return;
    constexpr int DL = HD / 64;
    const long long stride = (long long)n * nh * (HD + 2);
    const float *p0 = part + (long long)i * (HD + 2);
    float mx = kAttnNoMax;
    for (int s = 0; s < splits; ++s) mx = fmaxf(mx, p0[s * stride + HD]);
    float den = 0.0f, num[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) num[e] = 0.0f;
    for (int s = 0; s < splits; ++s) {
        const float *ps = p0 + s * stride;
        const float f = expf(ps[HD] - mx);
        den = fmaf(ps[HD + 1], f, den);
#pragma unroll
        for (int e = 0; e < DL; ++e) num[e] = fmaf(ps[lane * DL + e], f, num[e]);
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) o[(long long)i * HD + lane * DL + e] = num[e] / den;
}

__global__ __launch_bounds__(256) void kv_append_kernel(const float4 *__restrict__ k, const float4 *__restrict__ v,
                                                        long long n4, float4 *__restrict__ kc,
                                                        float4 *__restrict__ vc) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long long)gridDim.x * blockDim.x) {
        kc[i] = k[i];
        vc[i] = v[i];
    }
}

// Keys per split: a multiple of the tile, with enough splits that the grid
// holds about two workgroups per compute unit.
static int attn_chunk(int ctx, int blocks) {
    const int tiles = ceil_div(ctx, kAttnKT);
    const int want = std::max(1, 512 / std::max(1, blocks));
    const int splits = std::min(tiles, want);
    return kAttnKT * ceil_div(tiles, splits);
}

template <int HD>
static int launch_attn(const float *q, const float *kc, const float *vc, int n, int pos0, int nh, int nkv,
                       float scale, float *o, float *part, int chunk, int splits, hipStream_t s) {
    constexpr size_t lds = (size_t)AttnCfg<HD>::kLdsFloats * sizeof(float);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_prefill_kernel<HD>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return PG_ELAUNCH;
    const int rep = nh / nkv;
    const dim3 grid(splits, ceil_div(n, kAttnQ / rep), nkv);
    hipLaunchKernelGGL(attn_prefill_kernel<HD>, grid, dim3(kAttnThreads), lds, s, q, kc, vc, n, pos0, nh, nkv, scale,
                       chunk, part);
    int rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(attn_merge_kernel<HD>, dim3(ceil_div(n * nh, kAttnWaves)), dim3(kAttnThreads), 0, s, part, n,
                       nh, splits, o);
    return launch_status();
}

}  // namespace pg

using namespace pg;

static bool attn_shape_ok(int n, int pos0, int nh, int nkv, int hd) {
    if (n <= 0 || pos0 < 0 || nh <= 0 || nkv <= 0 || nh % nkv) return false;
    return true;
}

static int attn_splits(int n, int pos0, int nh, int nkv, int *chunk) {
    const int rep = nh / nkv;
    const int blocks = ceil_div(n, kAttnQ / rep) * nkv;
    *chunk = attn_chunk(pos0 + n, blocks);
    return ceil_div(pos0 + n, *chunk);
}

extern "C" size_t attn_prefill_workspace_bytes(int32_t n, int32_t pos0, int32_t nh, int32_t nkv, int32_t hd) {
    if (!attn_shape_ok(n, pos0, nh, nkv, hd)) return 0;
    int chunk;
    const int splits = attn_splits(n, pos0, nh, nkv, &chunk);
    return (size_t)splits * n * nh * (hd + 2) * sizeof(float);
}

extern "C" int attn_prefill(const float *q, const float *kc, const float *vc, int32_t n, int32_t pos0, int32_t nh,
                            int32_t nkv, int32_t hd, float scale, float *o, void *workspace, size_t workspace_bytes,
                            pg_stream_t stream) {
    if (!q || !kc || !vc || !o) return PG_EINVAL;
    if (!attn_shape_ok(n, pos0, nh, nkv, hd)) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || ((uintptr_t)o & 3)) return PG_EINVAL;
    const int rep = nh / nkv;
    if ((hd != 64 && hd != 128) || kAttnQ % rep || n > 64) return PG_EUNSUPPORTED;
    if ((long long)(pos0 + n) * nkv * hd >= (1ll << 31)) return PG_EUNSUPPORTED;
    const size_t need = attn_prefill_workspace_bytes(n, pos0, nh, nkv, hd);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3)) return PG_EWORKSPACE;
    const char *oc = reinterpret_cast<const char *>(o), *wc = static_cast<const char *>(workspace);
    const size_t ob = (size_t)n * nh * hd * sizeof(float);
    if (oc < wc + need && wc < oc + ob) return PG_EINVAL;
    int chunk;
    const int splits = attn_splits(n, pos0, nh, nkv, &chunk);
    float *part = static_cast<float *>(workspace);
    hipStream_t s = as_stream(stream);
    return hd == 128 ? launch_attn<128>(q, kc, vc, n, pos0, nh, nkv, scale, o, part, chunk, splits, s)
                     : launch_attn<64>(q, kc, vc, n, pos0, nh, nkv, scale, o, part, chunk, splits, s);
}

extern "C" int attn_kv_append(const float *k, const float *v, int32_t n, int32_t width, int32_t pos0, float *kc,
                              float *vc, int32_t cap, pg_stream_t stream) {
    if (!k || !v || !kc || !vc) return PG_EINVAL;
    if (n <= 0 || width <= 0 || pos0 < 0 || pos0 + n > cap) return PG_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(kc) || !aligned16(vc) || width % 4) return PG_EINVAL;
    const long long n4 = (long long)n * width / 4;
    const long long at = (long long)pos0 * width / 4;
    const unsigned grid = (unsigned)std::min<long long>((n4 + 255) / 256, 2048);
    hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, as_stream(stream), reinterpret_cast<const float4 *>(k),
                       reinterpret_cast<const float4 *>(v), n4, reinterpret_cast<float4 *>(kc) + at,
                       reinterpret_cast<float4 *>(vc) + at);
    return launch_status();
}
