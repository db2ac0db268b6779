// Token choice of every position over its logits (nemotron_prefill.rs,
// `pb_argmax`, used by the verify passes): ids[b] is the smallest index of the
// row's largest logit, counting only logits above -3.0e38 (the search starts
// from that value at index 0, so NaN never wins and a row with no such logit
// gives 0).
//
// One 1024-thread workgroup per position: a 32000-entry row is 125 KB, and the
// whole row is requested at once (kArgBatch float4 loads a thread before any
// comparison).  Each thread walks its entries in ascending order with a strict
// comparison, so it keeps the first index of its maximum; the workgroup then
// folds (value, index) pairs, a larger value or an equal value at a smaller
// index winning, which is the same choice as one sequential scan.
#include <stdint.h>

#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kArgThreads = 1024;
constexpr int kArgBatch = 8;
constexpr float kArgFloor = -3.0e38f;

struct Best {
    float v;
    uint32_t i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ void take(Best &b, float v, uint32_t i) {
    if (v > b.v) {
        b.v = v;
        b.i = i;
    }
}

// VEC: rows are read as float4 (vocab % 4 == 0 and a 16-byte aligned base).
template <bool VEC>
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const float *__restrict__ L, int vocab,
                                                             uint32_t *__restrict__ ids) {
    __shared__ float sv[kArgThreads / kWave];
    __shared__ uint32_t si[kArgThreads / kWave];
    const int b = blockIdx.x;
    const float *row = L + (long long)b * vocab;
    Best best{kArgFloor, 0u};
    if (VEC) {
        const int n4 = vocab >> 2;
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int base = 0; base < n4; base += kArgThreads * kArgBatch) {
            float4 v[kArgBatch];
#pragma unroll
            for (int k = 0; k < kArgBatch; ++k) {
                const int i = base + threadIdx.x + k * kArgThreads;
                v[k] = i < n4 ? r4[i] : make_float4(kArgFloor, kArgFloor, kArgFloor, kArgFloor);
            }
#pragma unroll
            for (int k = 0; k < kArgBatch; ++k) {
                const uint32_t i = 4u * (uint32_t)(base + threadIdx.x + k * kArgThreads);
                take(best, v[k].x, i);
                take(best, v[k].y, i + 1);
                take(best, v[k].z, i + 2);
                take(best, v[k].w, i + 3);
            }
        }
    } else {
        for (int base = 0; base < vocab; base += kArgThreads * kArgBatch) {
            float v[kArgBatch];
#pragma unroll
            for (int k = 0; k < kArgBatch; ++k) {
                const int i = base + threadIdx.x + k * kArgThreads;
                v[k] = i < vocab ? row[i] : kArgFloor;
            }
#pragma unroll
            for (int k = 0; k < kArgBatch; ++k) take(best, v[k], (uint32_t)(base + threadIdx.x + k * kArgThreads));
        }
    }
    // Fold across the wave, then across the waves.
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const Best o{__shfl_xor(best.v, off), (uint32_t)__shfl_xor((int)best.i, off)};
        best = better(best, o);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = best.v;
        si[wave] = best.i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        Best t{sv[0], si[0]};
        for (int w = 1; w < kArgThreads / kWave; ++w) t = better(t, Best{sv[w], si[w]});
        ids[b] = t.i;
    }
}

}  // namespace pg

using namespace pg;

extern "C" int argmax_rows(const float *logits, int32_t n, int32_t vocab, uint32_t *ids, pg_stream_t stream) {
    if (!logits || !ids) return PG_EINVAL;
    if (n <= 0 || vocab <= 0) return PG_EINVAL;
    if (((uintptr_t)logits & 3) || ((uintptr_t)ids & 3)) return PG_EINVAL;
    const char *l0 = reinterpret_cast<const char *>(logits), *i0 = reinterpret_cast<const char *>(ids);
    const size_t lb = (size_t)n * vocab * sizeof(float), ib = (size_t)n * sizeof(uint32_t);
    if (i0 < l0 + lb && l0 < i0 + ib) return PG_EINVAL;
    const bool vec = vocab % 4 == 0 && aligned16(logits);
    if (vec)
        hipLaunchKernelGGL(argmax_kernel<true>, dim3(n), dim3(kArgThreads), 0, as_stream(stream), logits, vocab, ids);
    else
        hipLaunchKernelGGL(argmax_kernel<false>, dim3(n), dim3(kArgThreads), 0, as_stream(stream), logits, vocab, ids);
    return launch_status();
}
