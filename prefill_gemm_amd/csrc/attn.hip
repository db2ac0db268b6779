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
// tile of 64 keys, K and V are staged in LDS; each wave takes 16 queries,
// forms their scores and p . V on the matrix cores in f32
// (v_mfma_f32_16x16x4f32: products and sums in f32, as the pages' arithmetic),
// and keeps an online softmax per query (running max m and sum l) on the vector
// ALU in between.  q enters scaled by scale * log2 e, so the scores are in
// base-2 units and every softmax weight is one hardware exp2 (v_exp_f32).  A split writes (m, l, acc) per query; the merge kernel
// rescales the splits to a common maximum and adds them in split order.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Reductions over the 16 lanes of one DPP row (quad, half-row and row
// exchanges); every lane of the row receives the result.
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v) {
    auto dpp = [](float x, int ctrl) __attribute__((always_inline)) {
        switch (ctrl) {  // the control must be a constant expression
            case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
            case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
            case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
            default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
        }
    };
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror
        const float o = dpp(v, c);
        v = MAX ? fmaxf(v, o) : v + o;
    }
    return v;
}

__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int HD>
struct AttnCfg {
    static constexpr int kKStride = HD + 4;        // floats per staged K row (padding spreads banks)
    static constexpr int kKFloats = kAttnKT * kKStride;
    static constexpr int kVStride = HD + 4;        // V staged as K: [key][dim]
    static constexpr int kVFloats = kAttnKT * kVStride;
    static constexpr int kPStride = kAttnKT + 4;   // p of a wave: [16 queries][key]
    static constexpr int kPFloats = kAttnWaves * kAttnQW * kPStride;
    static_assert(kPFloats <= kKFloats, "p reuses the K tile's space");
    static constexpr int kLdsFloats = kKFloats + kVFloats;
};

// Grid (split, query block, KV head).  part: [split][n][nh][hd + 2] (acc, m, l).
//
// Matrix-core fragments (v_mfma_f32_16x16x4f32: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16], and holds D[4 (l / 16) + v][l % 16], v < 4).  A wave's
// 16 queries are the rows.  q . k: step 4c + u contracts head dims
// 16c + 4k + u (k = lane group l / 16), so a lane reads its q row and its key's
// K row as float4 at dims 16c + 4k; q stays in registers.  p . V: step 4c + u
// contracts keys 16c + 4k + u, p read back from LDS as float4 of its row and V
// (staged as K is, a row per key) as four single values of its dim, one per
// key: a transposed copy would need 4-byte writes that meet 16-way LDS bank
// conflicts, the single reads meet none.  The softmax runs in the D
// layout: a row's 16 keys of a 16-key block sit in the 16 lanes of one DPP row.
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_prefill_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc, int n, int pos0,
    int nh, int nkv, float scale, int chunk, float *__restrict__ part, float *__restrict__ out) {
    using C = AttnCfg<HD>;
    constexpr int NC = HD / 16;   // 16-dim chunks (q . k) = 16-dim output blocks (p . V)
    constexpr int NKB = kAttnKT / 16;
    extern __shared__ float lds[];
    float *sk = lds;
    float *sv = sk + C::kKFloats;
    float *sp = sk;  // p takes the K tile's space once every wave has its scores
    const int split = blockIdx.x, qblk = blockIdx.y, g = blockIdx.z;
    const int rep = nh / nkv, P = kAttnQ / rep;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int b0 = qblk * P;
    const int bl = min(n, b0 + P) - 1;                    // last position of the block
    const int j0 = split * chunk;
    const int j1 = min(j0 + chunk, pos0 + bl + 1);        // keys past the block's last limit add nothing

    // A fragments of q . k: query 16 wave + r16 (position b0 + i / rep, head g rep + i % rep), scaled.
    f32x4 qf[NC];
    const float sl = scale * 1.44269504088896341f;  // base-2 scores: exp(x) = exp2(x log2 e)
    {
        const int i = kAttnQW * wave + r16;
        const int b = b0 + i / rep, h = g * rep + i % rep;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float4 v = make_float4(0, 0, 0, 0);
            if (b < n) v = *reinterpret_cast<const float4 *>(q + ((long long)b * nh + h) * HD + 16 * c + 4 * kg);
            qf[c] = f32x4{v.x * sl, v.y * sl, v.z * sl, v.w * sl};
        }
    }
    // The lane's D rows: queries 16 wave + 4 kg + v; their key limits.
    int lim[4];
    float m[4], l[4];
    f32x4 o[NC];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        lim[v] = pos0 + b0 + (kAttnQW * wave + 4 * kg + v) / rep;
        m[v] = kAttnNoMax;
        l[v] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float *pw = sp + wave * kAttnQW * C::kPStride;

    // K and V of a tile come into registers one tile ahead (each thread NR
    // float4 of each), so their memory latency hides behind the previous
    // tile's arithmetic; keys past j1 read as zeros.
    constexpr int kRow4 = HD / 4;
    constexpr int NR = kAttnKT * kRow4 / kAttnThreads;
    float4 ka[NR], va[NR];
    auto fetch = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int t = threadIdx.x + r * kAttnThreads;
            const int j = t0 + t / kRow4, d4 = t % kRow4;
            ka[r] = va[r] = make_float4(0, 0, 0, 0);
            if (j < j1) {
                const long long off = ((long long)j * nkv + g) * HD;
                ka[r] = reinterpret_cast<const float4 *>(kc + off)[d4];
                va[r] = reinterpret_cast<const float4 *>(vc + off)[d4];
            }
        }
    };
    if (j0 < j1) fetch(j0);

    for (int t0 = j0; t0 < j1; t0 += kAttnKT) {
        __syncthreads();  // the previous tile's K and V are no longer read
        // Stage keys t0 .. t0 + 63: K and V rows as they are.
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int t = threadIdx.x + r * kAttnThreads;
            const int kk = t / kRow4, d4 = t % kRow4;
            *reinterpret_cast<float4 *>(sk + kk * C::kKStride + 4 * d4) = ka[r];
            *reinterpret_cast<float4 *>(sv + kk * C::kVStride + 4 * d4) = va[r];
        }
        __syncthreads();
        if (t0 + kAttnKT < j1) fetch(t0 + kAttnKT);

        // Scores of the wave's 16 queries against the tile's 4 blocks of 16 keys.
        f32x4 sc[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sc[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const float *krow = sk + (16 * kb + r16) * C::kKStride + 4 * kg;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 kf = *reinterpret_cast<const f32x4 *>(krow + 16 * c);
#pragma unroll
                for (int u = 0; u < 4; ++u) sc[kb] = mfma_f32_16x16x4(qf[c][u], kf[u], sc[kb]);
            }
        }
        __syncthreads();  // every wave is done with K: its space takes p
        // Online softmax per row; masked keys weigh exactly 0.  Sums stay per lane.
        // The reference maximum m moves only when a row's tile maximum exceeds it
        // by more than 8 (weights up to 2^8), so most tiles rescale nothing.
        float s[4][NKB], mxr[4];
        bool need = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int j = t0 + 16 * kb + r16;
                s[v][kb] = (j < j1 && j <= lim[v]) ? sc[kb][v] : -INFINITY;
                mx = fmaxf(mx, s[v][kb]);
            }
            mxr[v] = row16_reduce<true>(mx);
            need |= mxr[v] > m[v] + 8.0f;
        }
        if (__ballot(need)) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float mn = fmaxf(m[v], mxr[v]);
                const float al = __builtin_amdgcn_exp2f(m[v] - mn);
                l[v] *= al;
                m[v] = mn;
#pragma unroll
                for (int c = 0; c < NC; ++c) o[c][v] *= al;
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float ps = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const float p = s[v][kb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[v][kb] - m[v]);
                ps += p;
                pw[(4 * kg + v) * C::kPStride + 16 * kb + r16] = p;
            }
            l[v] += ps;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's p writes land before its reads (lgkmcnt 0)
        __builtin_amdgcn_wave_barrier();
        // o += p . V over the tile's keys.
#pragma unroll
        for (int c2 = 0; c2 < NKB; ++c2) {
            const f32x4 pf = *reinterpret_cast<const f32x4 *>(pw + r16 * C::kPStride + 16 * c2 + 4 * kg);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float *vcol = sv + (16 * c2 + 4 * kg) * C::kVStride + 16 * c + r16;
                const f32x4 vf{vcol[0], vcol[C::kVStride], vcol[2 * C::kVStride], vcol[3 * C::kVStride]};
#pragma unroll
                for (int u = 0; u < 4; ++u) o[c] = mfma_f32_16x16x4(pf[u], vf[u], o[c]);
            }
        }
    }

    // Partials of the lane's rows for this split: o[c][v] is (query 16 wave + 4 kg + v, dim 16 c + r16).
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float lsum = row16_reduce<false>(l[v]);
        const int i = kAttnQW * wave + 4 * kg + v;
        const int b = b0 + i / rep, h = g * rep + i % rep;
        if (b >= n) continue;
        if (out) {  // one split: the result itself, no merge
            float *dst = out + ((long long)b * nh + h) * HD;
#pragma unroll
            for (int c = 0; c < NC; ++c) dst[16 * c + r16] = o[c][v] / lsum;
            continue;
        }
        float *dst = part + (((long long)split * n + b) * nh + h) * (HD + 2);
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[16 * c + r16] = o[c][v];
        if (r16 == 0) {
            dst[HD] = m[v];
            dst[HD + 1] = lsum;
        }
    }
}

// One wave per (position, query head): the splits rescaled to their common
// maximum and added in split order.  Lane s fetches split s's maximum and sum
// (splits <= 64), so the maximum and the denominator are one wave reduction
// each; the partial rows are requested sixteen splits at a time, the first
// sixteen together with the maxima and sums (one round trip for up to 16 splits).
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(const float *__restrict__ part, int n, int nh,
                                                                  int splits, float *__restrict__ o) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * kAttnWaves + (threadIdx.x >> 6);  // b * nh + h
    if (i >= n * nh) return;
    constexpr int DL = HD / 64;
    constexpr int kBatch = 16;
    const long long stride = (long long)n * nh * (HD + 2);
    const float *p0 = part + (long long)i * (HD + 2);
    float a[kBatch][DL];
    auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int sk = min(s0 + k, splits - 1);
#pragma unroll
            for (int e = 0; e < DL; ++e) a[k][e] = p0[sk * stride + lane * DL + e];
        }
    };
    fetch(0);  // requested together with the maxima and sums below: one round trip
    const bool mine = lane < splits;
    const float ms = mine ? p0[lane * stride + HD] : kAttnNoMax;
    const float ls = mine ? p0[lane * stride + HD + 1] : 0.0f;
    const float mx = wave_max(ms);
    const float f = mine ? __builtin_amdgcn_exp2f(ms - mx) : 0.0f;  // split `lane`'s factor
    float den = 0.0f, num[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) num[e] = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += kBatch) {
        if (s0 > 0) fetch(s0);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (s0 + k >= splits) break;
            const float fk = __shfl(f, s0 + k, kWave);
            const float lk = __shfl(ls, s0 + k, kWave);
            den = fmaf(lk, fk, den);
#pragma unroll
            for (int e = 0; e < DL; ++e) num[e] = fmaf(a[k][e], fk, num[e]);
        }
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

// Keys per split: a multiple of the tile, with enough splits (at most 64) that
// the grid holds about two workgroups per compute unit.
static int attn_chunk(int ctx, int blocks) {
    const int tiles = ceil_div(ctx, kAttnKT);
    const int want = std::min(64, std::max(1, 512 / std::max(1, blocks)));  // the merge takes <= 64 splits
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
    // A single split writes the output itself (no merge launch).
    hipLaunchKernelGGL(attn_prefill_kernel<HD>, grid, dim3(kAttnThreads), lds, s, q, kc, vc, n, pos0, nh, nkv, scale,
                       chunk, part, splits == 1 ? o : nullptr);
    int rc = launch_status();
    if (rc || splits == 1) return rc;
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
