// The achievable HBM read rate: a kernel that only streams bytes in, the
// ceiling the bandwidth-bound products are measured against (MI355X's
// published 8 TB/s is the peak; this is what a plain read reaches).
#include "pg_device.h"
#include "pg_host.h"

namespace pg {

constexpr int kProbeThreads = 512;
constexpr int kProbeBatch = 8;  // 16-byte loads in flight per lane

// Workgroup g reads the contiguous span of 16-byte units [g*per, min((g+1)*per, units)),
// kProbeBatch loads per lane in flight, non-temporal (each byte is read once).  The
// words are folded into one value per workgroup so that no load is dead.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                                    long long units, long long per,
                                                                    float *__restrict__ sink) {
    const long long lo = (long long)blockIdx.x * per;
    const long long hi = min(lo + per, units);
    uint32_t acc = 0;
    for (long long i = lo + threadIdx.x; i < hi; i += (long long)kProbeThreads * kProbeBatch) {
        u32x4 v[kProbeBatch];
#pragma unroll
        for (int b = 0; b < kProbeBatch; ++b) {
            const long long j = i + (long long)b * kProbeThreads;
            v[b] = j < hi ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int b = 0; b < kProbeBatch; ++b) acc ^= v[b].x ^ v[b].y ^ v[b].z ^ v[b].w;
    }
    for (int s = 32; s >= 1; s >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, s, kWave);
    if ((threadIdx.x & 63) == 0) atomicXor(reinterpret_cast<unsigned *>(sink) + blockIdx.x, acc);
}

}  // namespace pg

using namespace pg;

extern "C" int pg_stream_read(const void *src, size_t bytes, int32_t workgroups, float *sink,
                              pg_stream_t stream) {
    if (!src || !sink || bytes == 0 || workgroups <= 0) return PG_EINVAL;
    if (!aligned16(src) || bytes % 16) return PG_EINVAL;
    const long long units = (long long)(bytes / 16);
    const long long per = (units + workgroups - 1) / workgroups;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0, as_stream(stream),
                       static_cast<const u32x4 *>(src), units, per, sink);
    return launch_status();
}
