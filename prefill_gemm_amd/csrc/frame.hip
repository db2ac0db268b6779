// The q8 decode layer frame at one position as ONE persistent launch
// (decode_frame_q8).
//
// embryo_wide.wgsl (header comment): every dispatch boundary costs several
// microseconds, so the token frame fuses its stages; nemotron_prefill.rs
// (`pb_add_rms`, add = 1) places a residual add + RMSNorm between matrix
// stages.  The frame is four matrix-vector products, each needing the whole
// output of the one before:
//     qkv = Wqkv x0;  h1 = h + qkv[:H];  x1 = rmsnorm(h1) w1
//     u = relu^2(Wup x1);  d = Wdown u;  h2 = h1 + d;  x2 = rmsnorm(h2) w2
//     logits = Whead x2;   h <- h2
// One workgroup per compute unit runs all four products on a contiguous
// share of each matrix's rows, with a grid-wide barrier between products.
// Before wave 0 of a workgroup finishes the product and takes the barrier,
// the other waves have already requested the first weights of their next
// share (weights do not depend on the barrier), so those loads overlap the
// barrier.  After the barrier, wave 0 requests the activation before its own
// weights: a compute unit's memory requests are served in order, so a load
// queued behind weight requests waits for them.  The two norms are split
// the way gemv_q8_residual / gemv_q8_normed split them: a residual product
// writes w * h' and one sum of h'^2 per workgroup; the next product
// multiplies its dot products by 1 / rms, every workgroup adding the sums in
// the same order.  Values handed between workgroups are stored and loaded
// at device scope, so the barrier needs no cache-wide fences.
//
// Matrix-vector product of one wave: it owns units of two streams, each
// stream S steps of 1024 columns (16 bytes a lane: one half block of 16
// columns per lane).  A unit is two rows, or, when a share has too few rows
// to give every wave work, the two column halves of one row.  Loads go
// through a register ring D steps deep that runs across unit boundaries.
// Per 16-column segment:
//     acc += scale * sum_c q[c] x[c] + bias * sum_c x[c]
// with x and its segment sums staged in LDS (lane-interleaved, so a wave's
// 64 lanes read consecutive 16-byte slots).  Finished dot products go to LDS;
// wave 0 applies the product's epilogue for the whole share.
#include <algorithm>

#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kFD = 8;  // ring depth, in steps
constexpr int kFPre = 8;  // ring slots requested before a grid barrier
constexpr int kFStep = 1024;       // columns per step
constexpr int kFMaxCols = 16384;   // LDS holds one activation vector of this size
constexpr int kFMaxShare = 2048;   // rows of one product per workgroup

struct FMat {
    const int8_t *q;
    const float *scale;
    const float *bias;
    int rows, cols;
};

struct FrameArgs {
    FMat W[4];  // qkv, up, down, head
    const float *w1, *w2;
    float eps;
    const float *x0;
    float *h;
    float *qkv, *u, *d, *logits;
    float *xw1, *xw2;
    float *parts;     // [2][gridDim.x]: per-workgroup sums of h'^2 of the two residual products
    unsigned *sync;   // barrier counters (kSync* word offsets)
    int hidden;
    unsigned spin_limit;
    int split[4];     // per product: units are row halves (1) or row pairs (0)
};

// One product as seen by one wave.  The weights are read through buffer
// resources: the row and step go into the scalar offset, so a lane's vector
// offsets are the same for every load (and out-of-range reads return zero).
struct FPhase {
    const int8_t *q;
    const float *scale, *bias;
    int nq, ns;        // bytes of q and of scale (= of bias)
    int cols, nb;
    int r0, r1;        // this workgroup's rows [r0, r1)
    int S;             // steps per stream
    int split;         // 1: unit g = the halves of row r0 + g; 0: rows r0 + 2g, r0 + 2g + 1
    int units;         // units of this wave
    int wave;
};

__device__ __forceinline__ int share_per(int rows) {
    return ((rows + (int)gridDim.x - 1) / (int)gridDim.x + 1) & ~1;
}

__device__ __forceinline__ FPhase make_phase(const FMat &W, int split, int wave) {
    FPhase F;
    F.cols = W.cols;
    F.nb = W.cols >> 5;
    F.q = W.q;
    F.scale = W.scale;
    F.bias = W.bias;
    F.nq = W.rows * W.cols;
    F.ns = W.rows * F.nb * 4;
    const int per = share_per(W.rows);
    F.r0 = min(W.rows, (int)blockIdx.x * per);
    F.r1 = min(W.rows, F.r0 + per);
    F.split = split;
    F.S = (W.cols / kFStep) >> split;
    const int nunits = split ? F.r1 - F.r0 : (F.r1 - F.r0 + 1) >> 1;
    F.units = nunits > wave ? (nunits - wave + kFWaves - 1) / kFWaves : 0;
    F.wave = wave;
    return F;
}

// Register ring of one wave: D steps of two streams.
struct FRing {
    u32x4 q[kFD][2];
    float s[kFD][2], b[kFD][2];
};

// Position in a wave's (unit, step) stream.
struct FPos {
    int unit, step;
};

__device__ __forceinline__ void fadvance(FPos &p, int S) {
    if (++p.step == S) {
        p.step = 0;
        ++p.unit;
    }
}

__device__ __forceinline__ void unit_rows(const FPhase &F, int unit, int &ra, int &rb) {
    const int g = F.wave + kFWaves * unit;
    ra = F.r0 + (F.split ? g : 2 * g);
    rb = F.split ? ra : ra + 1;
}

// A raw buffer resource over `bytes` bytes at p; reads at offsets past the
// end return zero and make no memory request.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t frsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// Loads of stream position p into ring slot U (non-temporal: each weight
// byte is used once).  Lane l reads bytes 16 l .. 16 l + 15 of the step and
// the scale and bias of its half block; the row and step go into the scalar
// offset.  A stream position past the wave's last unit, or the second row
// of a pair that falls outside the share, is read through an empty resource:
// zeros, no memory traffic (nothing is stored for it).
constexpr int kFNT = 2;    // buffer cache policy: non-temporal
constexpr int kFDev = 16;  // buffer cache policy: device scope
template <int U>
__device__ __forceinline__ void fload(const FPhase &F, const FPos p, FRing &R, const int lane) {
    int ra, rb;
    unit_rows(F, p.unit, ra, rb);
    const bool va = p.unit < F.units, vb = va && rb < F.r1;
    const int sa = p.step, sb = p.step + (F.split ? F.S : 0);
    const int vq = 16 * lane, vs = 4 * (lane >> 1);
    R.q[U][0] = __builtin_amdgcn_raw_buffer_load_b128(frsrc(F.q, va ? F.nq : 0), vq, ra * F.cols + sa * kFStep, kFNT);
    R.q[U][1] = __builtin_amdgcn_raw_buffer_load_b128(frsrc(F.q, vb ? F.nq : 0), vq, rb * F.cols + sb * kFStep, kFNT);
    const int oa = 4 * (ra * F.nb + sa * (kFStep / 32)), ob = 4 * (rb * F.nb + sb * (kFStep / 32));
    const int nsa = va ? F.ns : 0, nsb = vb ? F.ns : 0;
    R.s[U][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(frsrc(F.scale, nsa), vs, oa, kFNT));
    R.s[U][1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(frsrc(F.scale, nsb), vs, ob, kFNT));
    R.b[U][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(frsrc(F.bias, nsa), vs, oa, kFNT));
    R.b[U][1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(frsrc(F.bias, nsb), vs, ob, kFNT));
}

// Positions B .. E - 1 of a product into ring slots B .. E - 1 (the ring
// holds positions 0 .. D - 1 once both halves have been issued in order).
template <int B = 0, int E = kFD>
__device__ __forceinline__ void fprefetch(const FPhase &F, FRing &R, const int lane) {
    static_for<E - B>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = B + decltype(uc)::value;
        fload<u>(F, FPos{u / F.S, u % F.S}, R, lane);
    });
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Total over the 64 lanes as a wave-uniform value: inside each row of 16
// lanes swap neighbours (quad permutations 1032 and 2301, then the half-row
// and row mirrors), which leaves the row's sum in all of its lanes; then the
// four row sums are added in a fixed order.
__device__ __forceinline__ float wave_total(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Dot product of 16 decoded weights with 16 staged activations.
__device__ __forceinline__ float dot16(const u32x4 w, const float (&xv)[16]) {
    float f[16];
    q16_to_f32(w, f);
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
        d0 = fmaf(f[k], xv[k], d0);
        d1 = fmaf(f[k + 1], xv[k + 1], d1);
    }
    return d0 + d1;
}

__device__ __forceinline__ void read_x(const float4 *sx, int step, int lane, float (&xv)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 a = sx[(step * 4 + j) * 64 + lane];
        xv[4 * j] = a.x;
        xv[4 * j + 1] = a.y;
        xv[4 * j + 2] = a.z;
        xv[4 * j + 3] = a.w;
    }
}

// Stream this wave's units of one product.  On entry the ring holds the
// loads of positions 0 .. D - 1; on exit it has been consumed and the dot
// products of this wave's rows are in yl[row - r0].
template <bool SPLIT>
__device__ __forceinline__ void fstream(const FPhase &F, FRing &R, const float4 *sx, const float *ssum, float *yl,
                                        const int lane) {
    const int T = F.units * F.S;
    const int Tpad = (T + kFD - 1) / kFD * kFD;
    FPos cp{0, 0}, lp{0, 0};
#pragma unroll
    for (int k = 0; k < kFD; ++k) fadvance(lp, F.S);
    float accA = 0.0f, accB = 0.0f;
    auto compute = [&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        // One slot at a time: the scheduler would otherwise hoist the LDS
        // reads of every slot and run out of registers.
        __builtin_amdgcn_sched_barrier(0);
        float xv[16];
        read_x(sx, cp.step, lane, xv);
        const float xsa = ssum[cp.step * 64 + lane];
        accA = fmaf(R.s[u][0], dot16(R.q[u][0], xv), accA);
        accA = fmaf(R.b[u][0], xsa, accA);
        float xsb = xsa;
        if (SPLIT) {
            read_x(sx, cp.step + F.S, lane, xv);
            xsb = ssum[(cp.step + F.S) * 64 + lane];
        }
        accB = fmaf(R.s[u][1], dot16(R.q[u][1], xv), accB);
        accB = fmaf(R.b[u][1], xsb, accB);
        if (cp.step == F.S - 1) {
            int ra, rb;
            unit_rows(F, cp.unit, ra, rb);
            if (SPLIT) {
                const float y = wave_total(accA + accB);
                if (lane == 0 && ra < F.r1) yl[ra - F.r0] = y;
            } else {
                const float ya = wave_total(accA), yb = wave_total(accB);
                if (lane == 0 && ra < F.r1) yl[ra - F.r0] = ya;
                if (lane == 0 && rb < F.r1) yl[rb - F.r0] = yb;
            }
            accA = 0.0f;
            accB = 0.0f;
        }
        fadvance(cp, F.S);
    };
    for (int t0 = 0; t0 + kFD < Tpad; t0 += kFD) {
        static_for<kFD>([&](auto uc) __attribute__((always_inline)) {
            compute(uc);
            fload<decltype(uc)::value>(F, lp, R, lane);
            fadvance(lp, F.S);
        });
    }
    if (Tpad > 0) static_for<kFD>([&](auto uc) __attribute__((always_inline)) { compute(uc); });
}

// Staging of x (cols floats) into LDS: float4 j of segment s at slot
// ((s / 64) * 4 + j) * 64 + s % 64, and the segment sums.  Thread t takes
// segments t, t + threads, ...; the loads and the LDS stores are separate
// calls so that a wave can request other data in between.  x is read at
// device scope (it may have been written by other workgroups of the launch);
// segments past the end read as zeros.
constexpr int kFStageIt = (kFMaxCols / 16 + kFThreads - 1) / kFThreads;
struct FStage {
    float4 a[kFStageIt][4];
};

__device__ __forceinline__ void stage_load(const float *x, int cols, FStage &st) {
    const __amdgpu_buffer_rsrc_t rx = frsrc(x, cols * 4);
#pragma unroll
    for (int it = 0; it < kFStageIt; ++it) {
        const int s = threadIdx.x + it * kFThreads;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            st.a[it][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, 64 * s + 16 * j, 0, kFDev));
    }
}

__device__ __forceinline__ void stage_store(const FStage &st, int cols, float4 *sx, float *ssum) {
    const int nseg = cols >> 4;
#pragma unroll
    for (int it = 0; it < kFStageIt; ++it) {
        const int s = threadIdx.x + it * kFThreads;
        if (s < nseg) {
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sx[((s >> 6) * 4 + j) * 64 + (s & 63)] = st.a[it][j];
                sum += (st.a[it][j].x + st.a[it][j].y) + (st.a[it][j].z + st.a[it][j].w);
            }
            ssum[s] = sum;
        }
    }
}

__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void wg_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Values handed between workgroups inside the launch (h, w * h, u, the norm
// parts) are written and read at device scope: the stores write through to
// where every compute unit sees them and the loads do not hit a stale cached
// copy.  That is what lets the grid barrier go without the device-wide
// release and acquire fences, which write back and invalidate whole caches.
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid-wide barrier (wave 0 of every workgroup), in two levels so that no
// counter takes more than a sixteenth of the arrivals: workgroup b counts
// itself into group b % 16; the last of a group counts the group into the
// top counter; the last group publishes the barrier's number, which every
// workgroup polls.  Counts accumulate over the launch (the n-th barrier
// waits for n arrivals per member).  The counters come in two sets used by
// alternate launches; a launch clears the other set.  The values a workgroup
// hands on were stored at device scope; waiting for those stores to complete
// before counting in orders them before the arrival.  The spin is bounded
// and counts a wait that gave up instead of hanging.
constexpr int kFGroups = 16;
constexpr int kSyncLaunch = 0;     // launch counter: its parity picks the set
constexpr int kSyncTimeouts = 2;   // barrier waits that gave up
constexpr int kSyncSet0 = 64;      // word offset of counter set 0 (set 1 follows)
constexpr int kSyncSetWords = 1024;
constexpr int kSyncTop = 512;      // within a set; group g's counter is at 32 g
constexpr int kSyncGen = 544;
constexpr int kSyncWords = kSyncSet0 + 2 * kSyncSetWords;

__device__ __forceinline__ unsigned ldu_dev(const unsigned *p) {
    return __hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stu_dev(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned addu_dev(unsigned *p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void grid_arrive_wait(unsigned *sync, unsigned *set, unsigned n, unsigned spin_limit,
                                                 int lane) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) {
        const unsigned G = gridDim.x, g = blockIdx.x % kFGroups;
        const unsigned groups = min(G, (unsigned)kFGroups);
        const unsigned members = G / kFGroups + (g < G % kFGroups ? 1u : 0u);
        if (addu_dev(&set[32 * g], 1u) == n * members - 1 && addu_dev(&set[kSyncTop], 1u) == n * groups - 1)
            stu_dev(&set[kSyncGen], n);
        unsigned spins = 0;
        while (ldu_dev(&set[kSyncGen]) < n) {
            if (++spins > spin_limit) {
                addu_dev(&sync[kSyncTimeouts], 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __asm__ volatile("" ::: "memory");
}

// Epilogue of a residual product (wave 0): out[r] = y; for r < hidden
// h[r] += y, xw[r] = w[r] * h[r]; part = sum of the new h[r]^2 (lanes take
// rows r0 + lane + 64 k in order, then a fixed butterfly).
__device__ __forceinline__ void epi_resid(const FPhase &F, const float *yl, const float *hl, const float *wl,
                                          float *out, float *h, float *xw, int hidden, float *part, int lane) {
    float sq = 0.0f;
    for (int i = lane; i < F.r1 - F.r0; i += kWave) {
        const int r = F.r0 + i;
        const float y = yl[i];
        out[r] = y;
        if (r < hidden) {
            const float hp = hl[i] + y;
            st_dev(h + r, hp);
            st_dev(xw + r, wl[i] * hp);
            sq = fmaf(hp, hp, sq);
        }
    }
    sq = wave_sum(sq);
    if (lane == 0) st_dev(part, sq);
}

__device__ __forceinline__ void epi_scaled(const FPhase &F, const float *yl, float inv, int act, float *out, int lane) {
    for (int i = lane; i < F.r1 - F.r0; i += kWave) st_dev(out + F.r0 + i, apply_act(act, inv * yl[i]));
}

// h[r] and w[r] of the share's residual rows into LDS (wave 0).
__device__ __forceinline__ void load_resid_rows(const FPhase &F, const float *h, const float *w, int hidden,
                                                float *hl, float *wl, int lane) {
    for (int i = lane; i < F.r1 - F.r0; i += kWave) {
        const int r = F.r0 + i;
        if (r < hidden) {
            hl[i] = ld_dev(h + r);
            wl[i] = w[r];
        }
    }
}

// 1 / rms from the per-workgroup parts (wave 0; the same order everywhere).
__device__ __forceinline__ float inv_rms(const float *parts, int hidden, float eps, int lane) {
    float t = 0.0f;
    for (int i = lane; i < (int)gridDim.x; i += kWave) t += ld_dev(parts + i);
    t = wave_sum(t);
    return rsqrtf(t / (float)hidden + eps);
}

template <class Fn>
__device__ __forceinline__ void with_split(int split, Fn &&fn) {
    if (split) fn(std::integral_constant<bool, true>{});
    else fn(std::integral_constant<bool, false>{});
}

__global__ __launch_bounds__(kFThreads) void decode_frame_kernel(FrameArgs A) {
    extern __shared__ float4 fsx[];
    __shared__ float s_inv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = A.hidden;
    const int maxS = max(max(A.W[0].cols, A.W[1].cols), max(A.W[2].cols, A.W[3].cols)) / kFStep;
    float *ssum = reinterpret_cast<float *>(fsx + maxS * 4 * 64);
    float *yl = ssum + maxS * 64;
    float *hl = yl + kFMaxShare;
    float *wl = hl + kFMaxShare;

    float *const outs[4] = {A.qkv, A.u, A.d, A.logits};

    // This launch's counter set; the launch counter moves on after the first
    // barrier, when every workgroup has read it.
    const unsigned launch = ldu_dev(&A.sync[kSyncLaunch]);
    unsigned *const set = A.sync + kSyncSet0 + (launch & 1) * kSyncSetWords;

    FRing R;
    FStage st;
    // Product 0 (QKV): weights first, then x0; wave 1 fetches the residual
    // rows and norm weights of the share.
    FPhase cur = make_phase(A.W[0], A.split[0], wave);
    fprefetch(cur, R, lane);
    stage_load(A.x0, A.W[0].cols, st);
    stage_store(st, A.W[0].cols, fsx, ssum);
    if (wave == 1 % kFWaves) load_resid_rows(cur, A.h, A.w1, H, hl, wl, lane);
    lds_barrier();
    with_split(A.split[0], [&](auto sp) __attribute__((always_inline)) {
        fstream<decltype(sp)::value>(cur, R, fsx, ssum, yl, lane);
    });
    lds_barrier();

    // Between products: waves 1.. request the next weights; wave 0 finishes
    // the product (epilogue stores), crosses the grid barrier, then requests
    // the activation before its own weights so that it does not wait for
    // them to stage it.
    static_for<3>([&](auto pc) __attribute__((always_inline)) {
        constexpr int ph = decltype(pc)::value + 1;
        const FPhase nxt = make_phase(A.W[ph], A.split[ph], wave);
        if (wave != 0) {
            fprefetch<0, kFPre>(nxt, R, lane);
        } else {
            if (ph == 1 || ph == 3)
                epi_resid(cur, yl, hl, wl, outs[ph - 1], A.h, ph == 1 ? A.xw1 : A.xw2, H,
                          A.parts + (ph == 1 ? 0 : gridDim.x) + blockIdx.x, lane);
            else
                epi_scaled(cur, yl, s_inv, 1, outs[ph - 1], lane);
            grid_arrive_wait(A.sync, set, ph, A.spin_limit, lane);
            if (ph == 1 && blockIdx.x == 0 && lane == 0) {
                unsigned *other = A.sync + kSyncSet0 + ((launch + 1) & 1) * kSyncSetWords;
                for (int g = 0; g < kFGroups; ++g) stu_dev(&other[32 * g], 0u);
                stu_dev(&other[kSyncTop], 0u);
                stu_dev(&other[kSyncGen], 0u);
                stu_dev(&A.sync[kSyncLaunch], launch + 1);
            }
        }
        wg_barrier();
        // Stage this product's activation: x1 = xw1 / rms, u, x2 = xw2 / rms.
        const float *xin = ph == 1 ? A.xw1 : ph == 2 ? A.u : A.xw2;
        stage_load(xin, A.W[ph].cols, st);
        if (wave == 0) fprefetch(nxt, R, lane);
        else fprefetch<kFPre, kFD>(nxt, R, lane);
        stage_store(st, A.W[ph].cols, fsx, ssum);
        if (wave == 1 % kFWaves) {
            if (ph == 2) {
                load_resid_rows(nxt, A.h, A.w2, H, hl, wl, lane);
            } else {
                const float inv = inv_rms(A.parts + (ph == 1 ? 0 : gridDim.x), H, A.eps, lane);
                if (lane == 0) s_inv = inv;
            }
        }
        lds_barrier();
        with_split(A.split[ph], [&](auto sp) __attribute__((always_inline)) {
            fstream<decltype(sp)::value>(nxt, R, fsx, ssum, yl, lane);
        });
        lds_barrier();
        cur = nxt;
    });

    if (wave == 0) epi_scaled(cur, yl, s_inv, 0, A.logits, lane);
}

__global__ void frame_sync_clear_kernel(unsigned *sync) {
    for (int i = threadIdx.x; i < kSyncWords; i += blockDim.x) sync[i] = 0u;
}

}  // namespace pg

using namespace pg;

namespace {

int frame_grid() {
    static int g = -1;
    if (g < 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        g = cus;
    }
    return g;
}

size_t frame_lds(int maxcols) {
    const int S = maxcols / kFStep;
    return (size_t)S * 4 * 64 * sizeof(float4) + (size_t)S * 64 * sizeof(float) + 3 * (size_t)kFMaxShare * sizeof(float);
}

// Units are row halves when that shortens the busiest wave's stream.
int choose_split(int rows, int cols, int grid) {
    const int per = ((rows + grid - 1) / grid + 1) & ~1;
    const int S = cols / kFStep;
    if (S % 2) return 0;
    const int pairs = ceil_div(ceil_div(per, 2), kFWaves) * S;
    const int halves = ceil_div(per, kFWaves) * (S / 2);
    return halves < pairs ? 1 : 0;
}

constexpr size_t kSyncBytes = round_up((size_t)kSyncWords * 4, 256);
constexpr size_t kFLdsMin = 80 * 1024 + 16;  // more than half of a compute unit's LDS

}  // namespace

extern "C" size_t decode_frame_q8_workspace_bytes(int32_t hidden, int32_t inter) {
    const int g = frame_grid();
    if (hidden <= 0 || inter <= 0 || g <= 0) return 0;
    return kSyncBytes + round_up((size_t)2 * g * sizeof(float), 256) + 2 * round_up((size_t)hidden * sizeof(float), 256);
}

extern "C" int decode_frame_q8_workspace_init(void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    if (!workspace || workspace_bytes < kSyncBytes || !aligned16(workspace)) return PG_EWORKSPACE;
    hipLaunchKernelGGL(frame_sync_clear_kernel, dim3(1), dim3(256), 0, as_stream(stream),
                       static_cast<unsigned *>(workspace));
    return launch_status();
}

extern "C" int decode_frame_q8_status(const void *workspace, size_t workspace_bytes, pg_stream_t stream) {
    if (!workspace || workspace_bytes < kSyncBytes || !aligned16(workspace)) return PG_EWORKSPACE;
    unsigned gave_up = 0;
    hipStream_t s = as_stream(stream);
    if (hipMemcpyAsync(&gave_up, static_cast<const unsigned *>(workspace) + kSyncTimeouts, sizeof(gave_up),
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return PG_ELAUNCH;
    return gave_up ? PG_ETIMEOUT : PG_OK;
}

extern "C" int decode_frame_q8(const pg_q8 *qkv_w, const pg_q8 *up_w, const pg_q8 *down_w, const pg_q8 *head_w,
                               const float *w1, const float *w2, float eps, const float *x0, float *h, float *qkv,
                               float *u, float *d, float *logits, void *workspace, size_t workspace_bytes,
                               pg_stream_t stream) {
    if (!qkv_w || !up_w || !down_w || !head_w || !w1 || !w2 || !x0 || !h || !qkv || !u || !d || !logits)
        return PG_EINVAL;
    if (!(eps >= 0.0f)) return PG_EINVAL;
    const pg_q8 *Ws[4] = {qkv_w, up_w, down_w, head_w};
    for (const pg_q8 *W : Ws) {
        if (!W->q || !W->scale || !W->bias || W->rows <= 0 || W->cols <= 0) return PG_EINVAL;
        if (!aligned16(W->q) || !aligned16(W->scale) || !aligned16(W->bias)) return PG_EINVAL;
        if (W->cols % kFStep || W->cols > kFMaxCols) return PG_EUNSUPPORTED;
        if ((size_t)W->rows * (size_t)W->cols >= (size_t)1 << 31) return PG_EUNSUPPORTED;
    }
    const int H = qkv_w->cols;
    if (qkv_w->rows < H || up_w->cols != H || down_w->cols != up_w->rows || down_w->rows != H || head_w->cols != H)
        return PG_EINVAL;
    const float *ins[] = {w1, w2, x0, h, qkv, u, d, logits};
    for (const float *p : ins)
        if (!aligned16(p)) return PG_EINVAL;
    const int g = frame_grid();
    if (g <= 0) return PG_ELAUNCH;
    for (const pg_q8 *W : Ws)
        if (ceil_div(W->rows, g) + 1 > kFMaxShare) return PG_EUNSUPPORTED;
    const size_t need = decode_frame_q8_workspace_bytes(H, up_w->rows);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PG_EWORKSPACE;
    {   // workgroups write the outputs while others still read the inputs
        const size_t hb = (size_t)H * sizeof(float);
        const Span sp[] = {{x0, hb}, {h, hb}, {w1, hb}, {w2, hb}, {qkv, (size_t)qkv_w->rows * sizeof(float)},
                           {u, (size_t)up_w->rows * sizeof(float)}, {d, hb},
                           {logits, (size_t)head_w->rows * sizeof(float)}, {workspace, need}};
        if (any_overlap(sp)) return PG_EINVAL;
    }

    char *ws = static_cast<char *>(workspace);
    FrameArgs A{};
    for (int i = 0; i < 4; ++i) {
        A.W[i] = FMat{Ws[i]->q, Ws[i]->scale, Ws[i]->bias, Ws[i]->rows, Ws[i]->cols};
        A.split[i] = choose_split(Ws[i]->rows, Ws[i]->cols, g);
    }
    A.w1 = w1;
    A.w2 = w2;
    A.eps = eps;
    A.x0 = x0;
    A.h = h;
    A.qkv = qkv;
    A.u = u;
    A.d = d;
    A.logits = logits;
    A.sync = reinterpret_cast<unsigned *>(ws);
    A.parts = reinterpret_cast<float *>(ws + kSyncBytes);
    A.xw1 = reinterpret_cast<float *>(ws + kSyncBytes + round_up((size_t)2 * g * sizeof(float), 256));
    A.xw2 = A.xw1 + round_up((size_t)H * sizeof(float), 256) / sizeof(float);
    A.hidden = H;
    A.spin_limit = 1u << 20;
    const int maxcols = std::max(std::max(qkv_w->cols, up_w->cols), std::max(down_w->cols, head_w->cols));
    // One workgroup per compute unit, all resident at once: every launch
    // asks for more LDS than two workgroups could share, and the occupancy
    // query confirms that one fits.  (A plain launch, so that the call can be
    // captured into a graph; the bounded barrier waits cover a device whose
    // compute units are held by other work.)
    static const int resident = [] {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(decode_frame_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)frame_lds(kFMaxCols)) != hipSuccess)
            return 0;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(decode_frame_kernel),
                                                         kFThreads, kFLdsMin) != hipSuccess)
            return 0;
        return n;
    }();
    if (resident < 1) return PG_ELAUNCH;
    hipLaunchKernelGGL(decode_frame_kernel, dim3(g), dim3(kFThreads), std::max(frame_lds(maxcols), kFLdsMin),
                       as_stream(stream), A);
    return launch_status();
}
