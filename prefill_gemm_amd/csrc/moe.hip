// Routed-MoE pass (moe_grouped).  nemotron_prefill.rs: `pb_f32_mm` (router
// product over the pass), `pb_route` (top-k by k rounds of a workgroup max,
// the lower expert index winning an exact tie, the winner masked),
// `pb_lists` (per expert, the pass's entries j = position * k + slot that
// chose it, ascending), `pb_q8_bank` (expert banks: workgroup per (row block,
// expert), an expert with no entries returns at once), `pb_add_rms` with
// add = 2 (the slot-ordered weighted sum into the residual, then the norm).
// Differences from the page: the router scores are softmax probabilities of
// the logits (ranking is done on the logits, which softmax preserves), and each
// expert's weights stream through the matrix cores once for all its entries
// instead of once per entry.
#include <math.h>

#include <type_traits>

#include "expert_q8.h"
#include "pg_device.h"
#include "pg_host.h"

namespace pg {

int launch_moe_combine(float *h, const float *shared, const float *D, const float *rw, int n, int k, const float *w,
                       float eps, int hidden, float *out, hipStream_t s);

constexpr int kRouterPos = 8;  // positions per router workgroup
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

// logits[b][e] in the fixed f32 order: lane l chains fused multiply-adds over
// the 4-column groups l, l+64, ...; the 64 lane sums fold pairwise for
// s = 32, 16, ..., 1 (lane l += lane l+s); the logit is lane 0's value.
// Grid (ceil(E / 4), ceil(n / 8)); wave -> expert, 8 positions per workgroup.
// The groups go in batches of kRouterBatch per lane: a batch's router and
// activation loads for all 8 positions are issued before any of them is used
// (one round trip per batch instead of one per group and position); each
// position's chain still runs over its groups in ascending order.
constexpr int kRouterBatch = 4;

__global__ __launch_bounds__(256) void router_logits_kernel(const float *__restrict__ X,
                                                            const float *__restrict__ Wr, int n,
                                                            int H, int E,
                                                            float *__restrict__ logits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const int G4 = H >> 2;
    const int b0 = blockIdx.y * kRouterPos;
    const float4 *wr = reinterpret_cast<const float4 *>(Wr + (long long)e * H);
    float acc[kRouterPos];
#pragma unroll
    for (int bb = 0; bb < kRouterPos; ++bb) acc[bb] = 0.0f;
    for (int g0 = lane; g0 < G4; g0 += 64 * kRouterBatch) {
        float4 w[kRouterBatch], x[kRouterPos][kRouterBatch];
#pragma unroll
        for (int k = 0; k < kRouterBatch; ++k) {
            const int g = g0 + 64 * k;
            w[k] = g < G4 ? wr[g] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
            for (int bb = 0; bb < kRouterPos; ++bb) {
                const int b = min(b0 + bb, n - 1);
                x[bb][k] = g < G4 ? reinterpret_cast<const float4 *>(X + (long long)b * H)[g]
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int k = 0; k < kRouterBatch; ++k) {
            if (g0 + 64 * k >= G4) break;  // past the row: the chain ends (no extra terms)
#pragma unroll
            for (int bb = 0; bb < kRouterPos; ++bb) {
                float a = acc[bb];
                a = fmaf(w[k].x, x[bb][k].x, a);
                a = fmaf(w[k].y, x[bb][k].y, a);
                a = fmaf(w[k].z, x[bb][k].z, a);
                a = fmaf(w[k].w, x[bb][k].w, a);
                acc[bb] = a;
            }
        }
    }
#pragma unroll
    for (int bb = 0; bb < kRouterPos; ++bb) {
        float v = acc[bb];
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
            const float o = __shfl_down(v, s, kWave);
            v = v + o;
        }
        const int b = b0 + bb;
        if (lane == 0 && b < n) logits[(long long)b * E + e] = v;
    }
}

// The sigmoid router's choice value decides integers (the chosen experts), so
// the sigmoid is one fixed sequence of binary32 operations whose every step is
// correctly rounded (fma, rint, ldexp, add, divide): any IEEE implementation
// of the same sequence gets the same bits.  exp(x) = 2^k e^r with the
// reduction of Cody and Waite ("Software Manual for the Elementary
// Functions", 1980): k = rint(x log2 e), r = x - k ln2 in two fused steps with
// ln2 = head (16 significant bits) + binary32 tail; e^r from its Taylor series
// through r^7 by Horner's rule, one fma a term.  x is clamped to [-80, 80]
// first, so nothing in the sequence is subnormal or infinite.
__device__ __forceinline__ float sigmoid_seq_f32(float l) {
#pragma clang fp contract(off)
    constexpr float kLog2E = 1.44269502162933349609375f;
    constexpr float kLn2Head = 0.693145751953125f;
    constexpr float kLn2Tail = 1.428606765330187045037746429443359375e-06f;
    // 1/7!, 1/6!, ..., 1/1!, 1/0! rounded to binary32, highest power first
    constexpr float kTaylor[8] = {1.0f / 5040.0f, 1.0f / 720.0f, 1.0f / 120.0f, 1.0f / 24.0f,
                                  1.0f / 6.0f,    0.5f,           1.0f,           1.0f};
    const float x = fminf(fmaxf(-l, -80.0f), 80.0f);
    const float kf = rintf(x * kLog2E);
    const float r = fmaf(-kf, kLn2Tail, fmaf(-kf, kLn2Head, x));
    float poly = kTaylor[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) poly = fmaf(poly, r, kTaylor[i]);
    const float ex = ldexpf(poly, (int)kf);
    return 1.0f / (1.0f + ex);
}

// One wave per position.  Softmax router (SIG = false): softmax over all E
// logits, then k rounds that take the largest remaining logit (lower index on
// an exact tie) and mask it.  Sigmoid router (SIG = true; nemotron_prefill.rs,
// `pb_route`): the choice value is sigmoid_seq_f32(l) + bias[e] (one binary32
// add), the k rounds rank it
// the same way, and slot t's weight is sigmoid(l_sel) / den * scale with
// den = (sum of the chosen sigmoids in slot order) + 1e-20 if norm, else 1.
// V = logits per lane (E <= 64 V); a lane's experts are lane, lane + 64, ...
template <int V, bool SIG>
__global__ __launch_bounds__(64) void route_kernel(const float *__restrict__ logits, int E, int k,
                                                   int renorm, const float *__restrict__ bias, float scale,
                                                   int32_t *__restrict__ sel, float *__restrict__ rw) {
    const int b = blockIdx.x, lane = threadIdx.x;
    float v[V], sg[V];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = lane + 64 * i;
        const float l = e < E ? logits[(long long)b * E + e] : -INFINITY;
        if (SIG) {
            sg[i] = e < E ? sigmoid_seq_f32(l) : 0.0f;
            v[i] = e < E ? sg[i] + bias[e] : -INFINITY;
        } else {
            v[i] = l;
            mx = fmaxf(mx, v[i]);
        }
    }
    float z = 0.0f;
    if (!SIG) {
        mx = wave_max(mx);
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (lane + 64 * i < E) z += expf(v[i] - mx);
        z = wave_sum(z);
    }

    uint32_t taken = 0;
    float psum = 0.0f;
    for (int t = 0; t < k; ++t) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && (bi < 0 || v[i] > bv)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
            const float ov = __shfl_xor(bv, s, kWave);
            const int oi = __shfl_xor(bi, s, kWave);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        float p;
        if (SIG) {
            float mine = 0.0f;  // the owner lane's sigmoid of the chosen expert
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (i == (bi >> 6)) mine = sg[i];
            p = __shfl(mine, bi & 63, kWave);
        } else {
            p = expf(bv - mx) / z;
        }
        psum += p;
        if (lane == 0) {
            sel[b * k + t] = bi;
            rw[b * k + t] = p;
        }
    }
    if (lane == 0) {
        if (SIG) {
            const float den = renorm ? psum + 1e-20f : 1.0f;
            for (int t = 0; t < k; ++t) rw[b * k + t] = rw[b * k + t] / den * scale;
        } else if (renorm) {
            for (int t = 0; t < k; ++t) rw[b * k + t] = rw[b * k + t] / psum;
        }
    }
}

// Router kernel for E experts (softmax, or sigmoid + bias when bias is given).
static int launch_route(const float *logits, int n, int E, int k, int renorm, const float *bias, float scale,
                        int32_t *sel, float *rw, hipStream_t s) {
    const bool sig = bias != nullptr;
    auto go = [&](auto vtag) {
        constexpr int V = decltype(vtag)::value;
        if (sig)
            hipLaunchKernelGGL((route_kernel<V, true>), dim3(n), dim3(64), 0, s, logits, E, k, renorm, bias, scale,
                               sel, rw);
        else
            hipLaunchKernelGGL((route_kernel<V, false>), dim3(n), dim3(64), 0, s, logits, E, k, renorm, bias, scale,
                               sel, rw);
    };
    if (E <= 64) go(std::integral_constant<int, 1>{});
    else if (E <= 128) go(std::integral_constant<int, 2>{});
    else if (E <= 256) go(std::integral_constant<int, 4>{});
    else go(std::integral_constant<int, kMaxExperts / kWave>{});
    return launch_status();
}

// One wave per expert: walk the n*k entries in ascending order, 64 at a time,
// and append the ones that chose this expert (ballot + prefix count).
__global__ __launch_bounds__(256) void group_kernel(const int32_t *__restrict__ sel, int nk, int E,
                                                    int cap, int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ lists) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    int base = 0;
    for (int j0 = 0; j0 < nk; j0 += 64) {
        const int j = j0 + lane;
        const bool hit = j < nk && sel[j] == e;
        const unsigned long long mask = __ballot(hit);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (hit && base + below < cap) lists[(long long)e * cap + base + below] = j;
        base += __popcll(mask);
    }
    if (lane == 0) counts[e] = base;
}

struct MoeLayout {
    size_t u, d, total;
};

// Workspace: the entries' up rows U [n k][I] and down rows D [n k][H].
static MoeLayout moe_layout(int n, int H, int I, int k) {
    MoeLayout L{};
    const size_t nk = (size_t)n * k;
    L.u = 0;
    L.d = round_up(nk * I * sizeof(float), 256);
    L.total = L.d + round_up(nk * H * sizeof(float), 256);
    return L;
}

}  // namespace pg

using namespace pg;

extern "C" size_t moe_grouped_workspace_bytes(int32_t n, int32_t H, int32_t I, int32_t E,
                                              int32_t top_k) {
    (void)E;
    if (n <= 0 || H <= 0 || I <= 0 || top_k <= 0 || H % 32 || I % 32) return 0;
    return moe_layout(n, H, I, top_k).total;
}

// The pass behind moe_grouped (router_bias NULL: softmax router) and
// moe_grouped_sigmoid (router_bias given: sigmoid + bias router; shared: the
// dense term the combine adds before the slots, NULL: none).
static int moe_run(const float *X, int32_t n, int32_t H, const float *Wr, int32_t E, int32_t top_k,
                   int32_t renorm, const float *router_bias, float scale, const int8_t *up_q,
                   const float *up_scale, const float *up_bias, int32_t I, const int8_t *down_q,
                   const float *down_scale, const float *down_bias, const float *shared, float *h,
                   const float *w_norm, float eps, float *out, float *logits, int32_t *sel, float *route_w,
                   int32_t *counts, int32_t *lists, void *workspace, size_t workspace_bytes,
                   pg_stream_t stream) {
    if (!X || !Wr || !up_q || !up_scale || !up_bias || !down_q || !down_scale || !down_bias ||
        !h || !w_norm || !out || !logits || !sel || !route_w || !counts || !lists)
        return PG_EINVAL;
    if (n <= 0 || H <= 0 || I <= 0 || E <= 0 || top_k <= 0) return PG_EINVAL;
    if (!aligned16(X) || !aligned16(Wr) || !aligned16(up_q) || !aligned16(down_q) ||
        !aligned16(h) || !aligned16(w_norm) || !aligned16(out))
        return PG_EINVAL;
    if (h == out) return PG_EINVAL;
    if (n > 64 || H % 32 || I % 32 || H > 16384 || E > kMaxExperts || top_k > kMaxTopK ||
        top_k > E)
        return PG_EUNSUPPORTED;
    const MoeLayout L = moe_layout(n, H, I, top_k);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return PG_EWORKSPACE;
    hipStream_t s = as_stream(stream);
    char *ws = static_cast<char *>(workspace);
    const int nk = n * top_k;
    float *U = reinterpret_cast<float *>(ws + L.u);
    float *D = reinterpret_cast<float *>(ws + L.d);

    hipLaunchKernelGGL(router_logits_kernel, dim3(ceil_div(E, 4), ceil_div(n, kRouterPos)),
                       dim3(256), 0, s, X, Wr, n, H, E, logits);
    int rc = launch_status();
    if (rc) return rc;
    if ((rc = launch_route(logits, n, E, top_k, renorm, router_bias, scale, sel, route_w, s))) return rc;
    hipLaunchKernelGGL(group_kernel, dim3(ceil_div(E, 4)), dim3(256), 0, s, sel, nk, E, n, counts,
                       lists);
    if ((rc = launch_status())) return rc;

    ExpertBank up{};
    up.q = up_q;
    up.scale = up_scale;
    up.bias = up_bias;
    up.rows = I;
    up.cols = H;
    up.q_stride = (long long)I * H;
    up.s_stride = (long long)I * (H / 32);
    up.x = X;
    up.ldx = H;
    up.src_div = top_k;
    up.counts = counts;
    up.lists = lists;
    up.cap = n;
    up.experts = E;
    up.out = U;
    up.ldo = I;
    up.act = 1;
    if ((rc = launch_expert_bank(up, s))) return rc;

    ExpertBank dn = up;
    dn.q = down_q;
    dn.scale = down_scale;
    dn.bias = down_bias;
    dn.rows = H;
    dn.cols = I;
    dn.q_stride = (long long)H * I;
    dn.s_stride = (long long)H * (I / 32);
    dn.x = U;
    dn.ldx = I;
    dn.src_div = 1;
    dn.out = D;
    dn.ldo = H;
    dn.act = 0;
    if ((rc = launch_expert_bank(dn, s))) return rc;

    return launch_moe_combine(h, shared, D, route_w, n, top_k, w_norm, eps, H, out, s);
}

extern "C" int moe_grouped(const float *X, int32_t n, int32_t H, const float *Wr, int32_t E,
                           int32_t top_k, int32_t renorm, const int8_t *up_q,
                           const float *up_scale, const float *up_bias, int32_t I,
                           const int8_t *down_q, const float *down_scale, const float *down_bias,
                           float *h, const float *w_norm, float eps, float *out, float *logits,
                           int32_t *sel, float *route_w, int32_t *counts, int32_t *lists,
                           void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    return moe_run(X, n, H, Wr, E, top_k, renorm, nullptr, 1.0f, up_q, up_scale, up_bias, I, down_q, down_scale,
                   down_bias, nullptr, h, w_norm, eps, out, logits, sel, route_w, counts, lists, workspace,
                   workspace_bytes, stream);
}

extern "C" int moe_grouped_sigmoid(const float *X, int32_t n, int32_t H, const float *Wr, int32_t E,
                                   int32_t top_k, const float *router_bias, int32_t renorm, float scale,
                                   const int8_t *up_q, const float *up_scale, const float *up_bias, int32_t I,
                                   const int8_t *down_q, const float *down_scale, const float *down_bias,
                                   const float *shared, float *h, const float *w_norm, float eps, float *out,
                                   float *logits, int32_t *sel, float *route_w, int32_t *counts,
                                   int32_t *lists, void *workspace, size_t workspace_bytes,
                                   pg_stream_t stream) {
    if (!router_bias) return PG_EINVAL;
    if (shared && (!aligned16(shared) || overlaps(shared, (size_t)n * H * 4, out, (size_t)n * H * 4) ||
                   overlaps(shared, (size_t)n * H * 4, h, (size_t)n * H * 4)))
        return PG_EINVAL;
    return moe_run(X, n, H, Wr, E, top_k, renorm, router_bias, scale, up_q, up_scale, up_bias, I, down_q,
                   down_scale, down_bias, shared, h, w_norm, eps, out, logits, sel, route_w, counts, lists,
                   workspace, workspace_bytes, stream);
}

extern "C" int moe_route_sigmoid(const float *logits, const float *router_bias, int32_t n, int32_t E,
                                 int32_t top_k, int32_t renorm, float scale, int32_t *sel, float *route_w,
                                 pg_stream_t stream) {
    if (!logits || !router_bias || !sel || !route_w) return PG_EINVAL;
    if (n <= 0 || E <= 0 || top_k <= 0) return PG_EINVAL;
    if (E > kMaxExperts || top_k > kMaxTopK || top_k > E) return PG_EUNSUPPORTED;
    return launch_route(logits, n, E, top_k, renorm, router_bias, scale, sel, route_w, as_stream(stream));
}
