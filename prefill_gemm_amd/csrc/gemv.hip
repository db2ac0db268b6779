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
#include <type_traits>

#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// What a q8 GEMV does around its product (template argument MODE):
//  kPlain    y = act(W x)
//  kAddNorm  y = act(W x), x = rmsnorm(h + delta) * w built while staging;
//            every workgroup forms the same sum of squares in the same order
//            and multiplies its finished dot products by the scalar 1/rms
//  kResid    y = act(W x); then for rows r < n: h_out[r] = h[r] + y[r],
//            x_out[r] = w[r] * h_out[r], and parts[j] = the sum of h_out^2
//            over the rows 8j .. 8j + 7 (the rows of workgroup j; one
//            part per workgroup keeps what every consumer workgroup reads small)
//  kScaled   y = act((W x) / sqrt(sum_j parts[j] / cols + eps)), j < n: the
//            consumer of a kResid product (x = its x_out), which completes
//            the RMSNorm without another pass over the activations
enum GemvMode { kPlain = 0, kAddNorm = 1, kResid = 2, kScaled = 3 };

// Norm parts per thread that a kScaled product requests up front (2 x 256
// threads cover the 512 parts of a 4096-row residual; more are read after).
constexpr int kPartsAhead = 2;

struct Fuse {
    const float *h;      // residual [cols] (kAddNorm) or [n] (kResid)
    const float *delta;  // kAddNorm: added to h first (NULL: nothing)
    const float *w;      // norm weight
    float eps;
    float *h_out;        // kAddNorm / kResid: h + delta or h + y (NULL: not written)
    float *x_out;        // kAddNorm: the normed x; kResid: w * h_out (NULL: not written)
    float *parts;        // kResid: written; kScaled: read
    int n;               // kResid: rows feeding the residual; kScaled: number of parts
};

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
// it adds nothing.  Weights are read with non-temporal loads: each byte is
// used once, and the staged activation and small vectors keep the caches.
// What happens around the product is MODE (GemvMode above).
template <int RW, int U, int MODE>
__global__ __launch_bounds__(kGemvThreads) void gemv_q8_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
    int rows, int cols, const float *__restrict__ x, float *__restrict__ y, int act, Fuse nm) {
    constexpr bool NORM = MODE == kAddNorm;
    extern __shared__ float4 sx[];
    __shared__ float red[kGemvWaves];
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
                    w[u][rr] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(qr[rr] + 16 * s));
                    sc[u][rr] = sr[rr][s >> 1];
                    bi[u][rr] = br[rr][s >> 1];
                }
            }
        }
    };
    load(0, wa, sa, ba);

    // kScaled: the first kPartsAhead norm parts a thread adds are requested
    // before the activation, so that both arrive in one round trip.
    float ss = 0.0f;
    float pa[kPartsAhead];
    if (MODE == kScaled) {
#pragma unroll
        for (int k = 0; k < kPartsAhead; ++k) {
            const int j = threadIdx.x + kGemvThreads * k;
            pa[k] = j < nm.n ? nm.parts[j] : 0.0f;
        }
    }
    for (int s = threadIdx.x; s < steps * 64; s += kGemvThreads) {
        float4 a[4];
        float sum = 0.0f;
        if (NORM) {
            // This workgroup writes h + delta (and later x) for its share of segments.
            const bool mine = (unsigned)s % gridDim.x == blockIdx.x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float4 v = make_float4(0, 0, 0, 0);
                if (s < nseg) {
                    v = reinterpret_cast<const float4 *>(nm.h)[4 * s + j];
                    if (nm.delta) {
                        const float4 d = reinterpret_cast<const float4 *>(nm.delta)[4 * s + j];
                        v.x += d.x; v.y += d.y; v.z += d.z; v.w += d.w;
                    }
                    if (nm.h_out && mine) reinterpret_cast<float4 *>(nm.h_out)[4 * s + j] = v;
                    const float4 g = reinterpret_cast<const float4 *>(nm.w)[4 * s + j];
                    ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
                    v = make_float4(g.x * v.x, g.y * v.y, g.z * v.z, g.w * v.w);
                }
                a[j] = v;
                sum += (v.x + v.y) + (v.z + v.w);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = s < nseg ? reinterpret_cast<const float4 *>(x)[4 * s + j] : make_float4(0, 0, 0, 0);
                sum += (a[j].x + a[j].y) + (a[j].z + a[j].w);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sx[xslot<4>(s, j)] = a[j];
        seg_sum[s] = sum;
    }
    if (MODE == kScaled) {
        // Opaque to the compiler, so that no add of a part (and its wait for
        // the memory counter, which covers the weights requested earlier) is
        // moved ahead of the activation staging.
#pragma unroll
        for (int k = 0; k < kPartsAhead; ++k) asm volatile("" : "+v"(pa[k]));
#pragma unroll
        for (int k = 0; k < kPartsAhead; ++k) ss += pa[k];
        for (int j = threadIdx.x + kGemvThreads * kPartsAhead; j < nm.n; j += kGemvThreads) ss += nm.parts[j];
    }
    if (NORM || MODE == kScaled) {
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
    }
    __syncthreads();
    float inv = 1.0f;
    if (NORM || MODE == kScaled) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kGemvWaves; ++i) t += red[i];
        inv = rsqrtf(t / (float)cols + nm.eps);
    }
    if (NORM) {
        if (nm.x_out) {
            for (int s = threadIdx.x; s < nseg; s += kGemvThreads) {
                if ((unsigned)s % gridDim.x != blockIdx.x) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a = sx[xslot<4>(s, j)];
                    reinterpret_cast<float4 *>(nm.x_out)[4 * s + j] =
                        make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
                }
            }
        }
    }

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
    float sq = 0.0f;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const float v = apply_act(act, wave_sum(acc[rr]) * inv);
        const int r = r0 + rr;
        if (lane == rr && r < rows) y[r] = v;
        if (MODE == kResid && r < nm.n) {
            const float hp = nm.h[r] + v;
            if (lane == rr) {
                if (nm.h_out) nm.h_out[r] = hp;
                if (nm.x_out) nm.x_out[r] = nm.w[r] * hp;
            }
            sq += hp * hp;
        }
    }
    if (MODE == kResid) {
        // The workgroup's 4 * RW rows (waves in order) make one part.
        if (lane == 0) red[wave] = sq;
        __syncthreads();
        if (threadIdx.x == 0 && blockIdx.x * kGemvWaves * RW < nm.n) {
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < kGemvWaves; ++i) t += red[i];
            nm.parts[blockIdx.x] = t;
        }
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

constexpr int kQ8Rw = 2, kQ8U = 1, kQ8ULong = 2;
constexpr int kQ8LongRow = 8192;  // columns above which a batch takes kQ8ULong steps
// q8_2f weights (gemma_batch.rs, `q8_2f_mm_r2` doc comment and epilogue): the
// column field folds into the staged activation, x'[c] = f16(cf[c]) * x[c],
// the row scale multiplies the finished sum.  Same streaming and batching as
// gemv_q8_kernel, without per-block factors: a 16-column segment is 16 plain
// fused multiply-adds of the decoded int8 with x'.
template <int RW, int U>
__global__ __launch_bounds__(kGemvThreads) void gemv_q82_kernel(
    const int8_t *__restrict__ q, const uint16_t *__restrict__ rs, const uint16_t *__restrict__ cf,
    int rows, int cols, const float *__restrict__ x, float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 4;
    const int steps = (nseg + 63) >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * kGemvWaves + wave) * RW;
    const int8_t *qr[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) qr[rr] = q + (long long)min(r0 + rr, rows - 1) * cols;
    u32x4 wa[U][RW], wb[U][RW];
    auto load = [&](int i0, u32x4 (&w)[U][RW]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u < steps) {
                const int s = min(lane + 64 * (i0 + u), nseg - 1);
#pragma unroll
                for (int rr = 0; rr < RW; ++rr)
                    w[u][rr] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(qr[rr] + 16 * s));
            }
        }
    };
    load(0, wa);
    for (int s = threadIdx.x; s < steps * 64; s += kGemvThreads) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 a = make_float4(0, 0, 0, 0);
            if (s < nseg) {
                const float4 v = reinterpret_cast<const float4 *>(x)[4 * s + j];
                const uint2 h = reinterpret_cast<const uint2 *>(cf)[4 * s + j];  // 4 binary16
                _Float16 c[4];
                __builtin_memcpy(c, &h, 8);
                a = make_float4((float)c[0] * v.x, (float)c[1] * v.y, (float)c[2] * v.z, (float)c[3] * v.w);
            }
            sx[xslot<4>(s, j)] = a;
        }
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
                float xv[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 a = sx[(i * 4 + j) * 64 + lane];
                    xv[4 * j] = a.x; xv[4 * j + 1] = a.y; xv[4 * j + 2] = a.z; xv[4 * j + 3] = a.w;
                }
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
        const int r = r0 + rr;
        const float v = wave_sum(acc[rr]);
        if (lane == rr && r < rows) {
            const _Float16 sr = __builtin_bit_cast(_Float16, rs[r]);
            y[r] = apply_act(act, (float)sr * v);
        }
    }
}

// f16: one row per wave (4096-column rows: the whole row in one batch of 4 x 2 steps).
constexpr int kF16Rw = 1, kF16U = 4;

// q4tp weights (nemotron_prefill.rs, the q4tp expert bank `pb_q4_bank`): per
// row, 4-bit codes two to a byte (column c in the low half of byte c/2 when c
// is even), the integer weight being code - 8; a binary16 base and step in one
// 32-bit word; a 5-bit code per 32-column group, least significant bit first,
// giving the group scale 2^(base + code * step).  A lane's step covers one
// group: 16 bytes of codes, the group scale from two code bytes, and
//     acc += scale * (sum_c nib[c] * x[c] - 8 * sum_c x[c]),
// the "- 8" folded into the group's activation sum (formed once per workgroup
// while x is staged).  Each 32-bit word's nibbles are split into its even and
// odd columns with two masks, and every byte becomes f32 in one conversion.
//
// Persistent: a few workgroups per compute unit stage x once, then each wave
// walks its items (RW rows x U steps; row block j of a wave is
// gw + j * total_waves), requesting item t + 1 before it computes item t.
// Loads go through buffer resources; an item past the wave's last one gets an
// empty resource (zeros, no memory traffic), so every load is issued
// unconditionally and each compute waits for exactly its own data.
constexpr int kQ4Rw = 2, kQ4U = 1, kQ4Occ = 2;
constexpr int kQ4Threads = 512;
constexpr int kQ4Waves = kQ4Threads / kWave;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t q4_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <int RW, int U>
__global__ __launch_bounds__(kQ4Threads) void gemv_q4tp_kernel(
    const uint8_t *__restrict__ nib, const uint32_t *__restrict__ params, const uint8_t *__restrict__ codes,
    int rows, int cols, const float *__restrict__ x, float *__restrict__ y, int act) {
    extern __shared__ float4 sx[];
    const int nseg = cols >> 5;  // groups per row
    const int steps = (nseg + 63) >> 6;
    const int nch = (steps + U - 1) / U;
    const int cstride = (5 * nseg + 7) >> 3;
    float *gsum = reinterpret_cast<float *>(sx + steps * 8 * 64);
    const int lane = threadIdx.x & 63;
    // Wave-uniform (the buffer resources below must be scalar).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nrb = (rows + RW - 1) / RW;
    const int gw = blockIdx.x * kQ4Waves + wave, tw = gridDim.x * kQ4Waves;
    const int T = gw < nrb ? ((nrb - gw + tw - 1) / tw) * nch : 0;
    const uint32_t half = (uint32_t)cols >> 1;
    const uint32_t nbytes = (uint32_t)rows * half;

    // A group's 5-bit code comes from one 4-byte window that starts at the
    // byte holding its first bit, moved back to end inside the code buffer when
    // needed (the field then still lies inside the window); the window's byte
    // address need not be 4-aligned.  Dead items read the last row's window
    // (cached).  The window's word stays as loaded until the compute, where the
    // code is cut out of it (doing that at the load would wait for the load).
    const uint32_t ctotal = (uint32_t)rows * (uint32_t)cstride;
    u32x4 wa[U][RW], wb[U][RW];
    uint32_t ca[U][RW], cb[U][RW], pa[RW], pb[RW];
    auto load = [&](int t, u32x4 (&w)[U][RW], uint32_t (&c)[U][RW], uint32_t (&p)[RW])
                    __attribute__((always_inline)) {
        const bool live = t < T;
        const int tt = live ? t : 0;
        const int rb = gw + (tt / nch) * tw, ch = tt % nch;
        const __amdgpu_buffer_rsrc_t rn = q4_rsrc(nib, live ? nbytes : 0u);
        const __amdgpu_buffer_rsrc_t rp = q4_rsrc(params, live ? (uint32_t)rows * 4u : 0u);
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const uint32_t r = (uint32_t)min(rb * RW + rr, rows - 1);
            p[rr] = __builtin_amdgcn_raw_buffer_load_b32(rp, 4u * r, 0, 0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = min(lane + 64 * (ch * U + u), nseg - 1);
                w[u][rr] = __builtin_amdgcn_raw_buffer_load_b128(rn, r * half + 16u * (uint32_t)s, 0, 0);
                const uint32_t at = r * (uint32_t)cstride + ((5u * (uint32_t)s) >> 3);
                uint32_t win;
                __builtin_memcpy(&win, codes + min(at, ctotal - 4u), 4);
                c[u][rr] = win;
            }
        }
    };
    load(0, wa, ca, pa);
    // Stage x: a thread's eight float4 are all requested before any is used
    // (one round trip); groups past the row stage zeros.
    for (int s = threadIdx.x; s < steps * 64; s += kQ4Threads) {
        const float4 *xs4 = reinterpret_cast<const float4 *>(x) + 8 * min(s, nseg - 1);
        float4 a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = xs4[j];
        const bool in = s < nseg;
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (!in) a[j] = make_float4(0, 0, 0, 0);
            sx[xslot<8>(s, j)] = a[j];
            t += (a[j].x + a[j].y) + (a[j].z + a[j].w);
        }
        gsum[s] = t;
    }
    __syncthreads();

    float acc[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) acc[rr] = 0.0f;
    // Item t: its chunk's U steps for the RW rows; the last chunk of a row
    // block folds the sums across the wave and writes y.  An item past the
    // wave's last one is computed on zeros and writes nothing (its rows are
    // at or past `rows`).
    auto compute = [&](int t, const u32x4 (&w)[U][RW], const uint32_t (&c)[U][RW], const uint32_t (&p)[RW])
                       __attribute__((always_inline)) {
        const int rb = gw + (t / nch) * tw, ch = t % nch;
        float base[RW], step[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            base[rr] = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[rr] & 0xFFFFu));
            step[rr] = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[rr] >> 16));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = ch * U + u;
            const int ic = min(i, steps - 1);
            const int s = lane + 64 * i;
            float xv[32];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 a = sx[(ic * 8 + j) * 64 + lane];
                xv[4 * j] = a.x; xv[4 * j + 1] = a.y; xv[4 * j + 2] = a.z; xv[4 * j + 3] = a.w;
            }
            const float xs8 = 8.0f * gsum[min(s, nseg - 1)];
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const uint32_t word[4] = {w[u][rr].x, w[u][rr].y, w[u][rr].z, w[u][rr].w};
                float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t lo = word[k] & 0x0F0F0F0Fu, hi = (word[k] >> 4) & 0x0F0F0F0Fu;
                    // Keep the two masked words whole so each byte converts with one
                    // v_cvt_f32_ubyteN instead of an extract and a conversion.
                    asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        d0 = fmaf((float)((lo >> (8 * b)) & 0xFFu), xv[8 * k + 2 * b], d0);
                        d1 = fmaf((float)((hi >> (8 * b)) & 0xFFu), xv[8 * k + 2 * b + 1], d1);
                    }
                }
                uint32_t win = c[u][rr];
                asm volatile("" : "+v"(win));  // cut the code here, not where the window loads
                const uint32_t r = (uint32_t)min(rb * RW + rr, rows - 1);
                const uint32_t at = r * (uint32_t)cstride + ((5u * (uint32_t)min(s, nseg - 1)) >> 3);
                const uint32_t sh = 8u * (at - min(at, ctotal - 4u)) + ((5u * (uint32_t)s) & 7u);
                const uint32_t code = (win >> sh) & 31u;
                // Hardware exp2 (exact at integer exponents; a scale below 2^-126 reads as
                // 0).  Groups past the row (s >= nseg) weigh nothing.
                const float sc = s < nseg ? __builtin_amdgcn_exp2f(fmaf((float)code, step[rr], base[rr])) : 0.0f;
                acc[rr] = fmaf(sc, (d0 + d1) - xs8, acc[rr]);
            }
        }
        if (ch == nch - 1) {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const float v = wave_sum(acc[rr]);
                const int r = rb * RW + rr;
                if (lane == rr && r < rows) y[r] = apply_act(act, v);
                acc[rr] = 0.0f;
            }
        }
    };
    for (int t = 0; t < T; t += 2) {
        load(t + 1, wb, cb, pb);
        __builtin_amdgcn_sched_barrier(0);
        compute(t, wa, ca, pa);
        __builtin_amdgcn_sched_barrier(0);
        load(t + 2, wa, ca, pa);
        __builtin_amdgcn_sched_barrier(0);
        compute(t + 1, wb, cb, pb);
        __builtin_amdgcn_sched_barrier(0);
    }
}

static int gemv_grid(int rows, int rw) { return ceil_div(rows, kGemvWaves * rw); }

// Compute units of the current device (read once).
static int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

}  // namespace pg

using namespace pg;

// Dynamic LDS of the q8 kernel: staged x (16 bytes per float4, 4 per segment)
// and one segment sum per segment, for ceil(cols / 1024) steps of 64 segments.
static size_t gemv_q8_lds(int cols) {
    const int steps = ceil_div(cols / 16, 64);
    return (size_t)steps * 4 * 64 * sizeof(float4) + (size_t)steps * 64 * sizeof(float);
}

// Allow the largest dynamic LDS a kernel can ask for (cols = 32768); the
// static reduction slots come on top, within the 160 KB of a compute unit.
static int allow_lds(const void *kernel, size_t bytes) {
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess)
        return PG_OK;
    (void)hipGetLastError();  // do not leave the error for a later launch check to find
    return PG_ELAUNCH;
}

template <int U, int MODE>
static int launch_mode_u(const int8_t *q, const float *scale, const float *bias, int rows, int cols,
                         const float *x, float *y, int act, const Fuse &nm, pg_stream_t stream) {
    static const int ok = allow_lds(reinterpret_cast<const void *>(gemv_q8_kernel<kQ8Rw, U, MODE>),
                                    gemv_q8_lds(32768));
    if (ok != PG_OK) return PG_ELAUNCH;
    hipLaunchKernelGGL((gemv_q8_kernel<kQ8Rw, U, MODE>), dim3(gemv_grid(rows, kQ8Rw)), dim3(kGemvThreads),
                       gemv_q8_lds(cols), as_stream(stream), q, scale, bias, rows, cols, x, y, act, nm);
    return launch_status();
}

// Steps per weight batch: rows up to 8192 columns take one step a batch (more
// workgroups resident, each issuing sooner), longer rows two (measured on the
// hidden-4096 frame: 4096-column products 4-11% faster at one, the
// 14336-column product 5% faster at two).  The rows per workgroup, and with them
// the residual mode's norm parts, do not depend on it.
template <int MODE>
static int launch_mode(const int8_t *q, const float *scale, const float *bias, int rows, int cols,
                       const float *x, float *y, int act, const Fuse &nm, pg_stream_t stream) {
    if (cols > kQ8LongRow)
        return launch_mode_u<kQ8ULong, MODE>(q, scale, bias, rows, cols, x, y, act, nm, stream);
    return launch_mode_u<kQ8U, MODE>(q, scale, bias, rows, cols, x, y, act, nm, stream);
}

// [a, a + an) and [b, b + bn) bytes overlap.
extern "C" int gemv_q8(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                       int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream) {
    if (!q || !scale || !bias || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(x) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    if (overlaps(y, (size_t)rows * sizeof(float), x, (size_t)cols * sizeof(float))) return PG_EINVAL;
    return launch_mode<kPlain>(q, scale, bias, rows, cols, x, y, act, Fuse{}, stream);
}

extern "C" int gemv_q8_addnorm(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                               int32_t cols, const float *h, const float *delta, const float *w,
                               float eps, float *h_out, float *x_out, float *y, int32_t act,
                               pg_stream_t stream) {
    if (!q || !scale || !bias || !h || !w || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || !(eps >= 0.0f)) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(h) || !aligned16(w) || !aligned16(y)) return PG_EINVAL;
    if ((delta && !aligned16(delta)) || (h_out && !aligned16(h_out)) || (x_out && !aligned16(x_out)))
        return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    // Outputs are written while other workgroups still read h, delta and w.
    const size_t vb = (size_t)cols * sizeof(float), yb = (size_t)rows * sizeof(float);
    const void *ins[3] = {h, delta, w};
    for (const void *in : ins) {
        if (overlaps(h_out, vb, in, vb) || overlaps(x_out, vb, in, vb) || overlaps(y, yb, in, vb))
            return PG_EINVAL;
    }
    if (overlaps(h_out, vb, x_out, vb) || overlaps(h_out, vb, y, yb) || overlaps(x_out, vb, y, yb))
        return PG_EINVAL;
    const Fuse nm{h, delta, w, eps, h_out, x_out, nullptr, 0};
    return launch_mode<kAddNorm>(q, scale, bias, rows, cols, nullptr, y, act, nm, stream);
}

extern "C" int32_t gemv_q8_norm_parts(int32_t hidden) {
    return hidden > 0 ? ceil_div(hidden, kGemvWaves * kQ8Rw) : 0;
}

extern "C" int gemv_q8_residual(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                                int32_t cols, const float *x, float *y, int32_t act, const float *h,
                                const float *w, int32_t hidden, float *h_out, float *xw, float *parts,
                                pg_stream_t stream) {
    if (!q || !scale || !bias || !x || !y || !h || !w || !xw || !parts) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || hidden <= 0 || hidden > rows) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(x) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    // Row r's residual is read and written by one lane, so h_out may be h; nothing
    // else may overlap (x is read by every workgroup while the others write).
    const size_t hb = (size_t)hidden * sizeof(float), yb = (size_t)rows * sizeof(float);
    const size_t pb = (size_t)ceil_div(hidden, kGemvWaves * kQ8Rw) * sizeof(float);
    const size_t xb = (size_t)cols * sizeof(float);
    struct Span { const void *p; size_t n; };
    const Span sp[7] = {{x, xb}, {y, yb}, {h, hb}, {w, hb}, {h_out, hb}, {xw, hb}, {parts, pb}};
    for (int i = 0; i < 7; ++i)
        for (int j = i + 1; j < 7; ++j) {
            if (i == 2 && j == 4 && h_out == h) continue;    // in place
            if (i <= 3 && j <= 3 && i != 1 && j != 1) continue;  // inputs may share memory
            if (overlaps(sp[i].p, sp[i].n, sp[j].p, sp[j].n)) return PG_EINVAL;
        }
    const Fuse nm{h, nullptr, w, 0.0f, h_out, xw, parts, hidden};
    return launch_mode<kResid>(q, scale, bias, rows, cols, x, y, act, nm, stream);
}

extern "C" int gemv_q8_normed(const int8_t *q, const float *scale, const float *bias, int32_t rows,
                              int32_t cols, const float *xw, const float *parts, float eps, float *y,
                              int32_t act, pg_stream_t stream) {
    if (!q || !scale || !bias || !xw || !parts || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0 || !(eps >= 0.0f)) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(xw) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    const int nparts = ceil_div(cols, kGemvWaves * kQ8Rw);
    const size_t yb = (size_t)rows * sizeof(float);
    if (overlaps(y, yb, xw, (size_t)cols * sizeof(float)) || overlaps(y, yb, parts, (size_t)nparts * sizeof(float)))
        return PG_EINVAL;
    const Fuse nm{nullptr, nullptr, nullptr, eps, nullptr, nullptr, const_cast<float *>(parts), nparts};
    return launch_mode<kScaled>(q, scale, bias, rows, cols, xw, y, act, nm, stream);
}

extern "C" int gemv_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field, int32_t rows,
                        int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream) {
    if (!q || !row_scale || !col_field || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(x) || ((uintptr_t)col_field & 7) || ((uintptr_t)row_scale & 1))
        return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 16 || cols > 32768) return PG_EUNSUPPORTED;
    if (overlaps(y, (size_t)rows * sizeof(float), x, (size_t)cols * sizeof(float))) return PG_EINVAL;
    const size_t lds = (size_t)ceil_div(cols / 16, 64) * 4 * 64 * sizeof(float4);
    auto go = [&](auto utag) {
        constexpr int U = decltype(utag)::value;
        static const int ok = allow_lds(reinterpret_cast<const void *>(gemv_q82_kernel<kQ8Rw, U>),
                                        (size_t)ceil_div(32768 / 16, 64) * 4 * 64 * sizeof(float4));
        if (ok != PG_OK) return (int)PG_ELAUNCH;
        hipLaunchKernelGGL((gemv_q82_kernel<kQ8Rw, U>), dim3(gemv_grid(rows, kQ8Rw)), dim3(kGemvThreads), lds,
                           as_stream(stream), q, row_scale, col_field, rows, cols, x, y, act);
        return launch_status();
    };
    // Steps per weight batch as for the block format (longer rows take more).
    return cols > kQ8LongRow ? go(std::integral_constant<int, kQ8ULong>{}) : go(std::integral_constant<int, kQ8U>{});
}

extern "C" int gemv_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t rows,
                         int32_t cols, const float *x, float *y, int32_t act, pg_stream_t stream) {
    if (!nib || !params || !codes || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(nib) || !aligned16(x) || ((uintptr_t)params & 3)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32 || cols > 32768) return PG_EUNSUPPORTED;
    if (overlaps(y, (size_t)rows * sizeof(float), x, (size_t)cols * sizeof(float))) return PG_EINVAL;
    if ((size_t)rows * (size_t)cols / 2 > 0x7FFFFFFFu) return PG_EUNSUPPORTED;  // 32-bit buffer offsets
    if ((size_t)rows * (size_t)((5 * (cols / 32) + 7) / 8) < 4) return PG_EUNSUPPORTED;  // 4-byte code windows
    auto bytes = [](int c) { return (size_t)ceil_div(c / 32, 64) * (8 * 64 * sizeof(float4) + 64 * sizeof(float)); };
    static const int ok = allow_lds(reinterpret_cast<const void *>(gemv_q4tp_kernel<kQ4Rw, kQ4U>), bytes(32768));
    if (ok != PG_OK) return PG_ELAUNCH;
    const int grid = std::min(ceil_div(ceil_div(rows, kQ4Rw), kQ4Waves), kQ4Occ * device_cus());
    hipLaunchKernelGGL((gemv_q4tp_kernel<kQ4Rw, kQ4U>), dim3(grid), dim3(kQ4Threads), bytes(cols),
                       as_stream(stream), nib, params, codes, rows, cols, x, y, act);
    return launch_status();
}

extern "C" int gemv_f16(const uint16_t *w, int32_t rows, int32_t cols, const float *x, float *y,
                        int32_t act, pg_stream_t stream) {
    if (!w || !x || !y) return PG_EINVAL;
    if (rows <= 0 || cols <= 0) return PG_EINVAL;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 8 || cols > 32768) return PG_EUNSUPPORTED;
    if (overlaps(y, (size_t)rows * sizeof(float), x, (size_t)cols * sizeof(float))) return PG_EINVAL;
    const size_t lds = (size_t)ceil_div(cols / 8, 64) * 2 * 64 * sizeof(float4);
    static const int ok = allow_lds(reinterpret_cast<const void *>(gemv_f16_kernel<kF16Rw, kF16U>),
                                    (size_t)ceil_div(32768 / 8, 64) * 2 * 64 * sizeof(float4));
    if (ok != PG_OK) return PG_ELAUNCH;
    hipLaunchKernelGGL((gemv_f16_kernel<kF16Rw, kF16U>), dim3(gemv_grid(rows, kF16Rw)),
                       dim3(kGemvThreads), lds, as_stream(stream), w, rows, cols, x, y, act);
    return launch_status();
}
