// Device-side building blocks shared by the libpg kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's uint4 is a struct whose copies become memcpy).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 32;  // columns sharing one scale and one bias

// Relu^2 on a finished product (act == 1), identity otherwise.
__device__ __forceinline__ float apply_act(int act, float v) {
    if (act == 1) {
        float t = fmaxf(v, 0.0f);
        return t * t;
    }
    return v;
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, kWave));
    return v;
}

// Two f32 values that are exact in bf16 (e.g. small integers): keep their high
// halves, `lo` in bits 0..15 and `hi` in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Sixteen int8 weights (one 16-byte load, columns c0..c0+15 of a row) as the
// two bf16x8 matrix-core operands: columns c0..c0+7 and c0+8..c0+15.  Integers
// in [-128, 127] are exact in bf16.
__device__ __forceinline__ void q16_to_bf16(const u32x4 w, bf16x8 &k0, bf16x8 &k1) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t p[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int v = (int)in[j];
        const float f0 = (float)(int8_t)(v);
        const float f1 = (float)(int8_t)(v >> 8);
        const float f2 = (float)(int8_t)(v >> 16);
        const float f3 = (float)(v >> 24);
        p[2 * j] = pack_bf16_exact(f0, f1);
        p[2 * j + 1] = pack_bf16_exact(f2, f3);
    }
    __builtin_memcpy(&k0, &p[0], 16);
    __builtin_memcpy(&k1, &p[4], 16);
}

// Sixteen int8 as f32 into `f`, column order.
__device__ __forceinline__ void q16_to_f32(const u32x4 w, float f[16]) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int v = (int)in[j];
        f[4 * j + 0] = (float)(int8_t)(v);
        f[4 * j + 1] = (float)(int8_t)(v >> 8);
        f[4 * j + 2] = (float)(int8_t)(v >> 16);
        f[4 * j + 3] = (float)(v >> 24);
    }
}

// Sixteen 4-bit codes n (two 32-bit words, columns 0..7 then 8..15: the low
// half of byte j is column 2j, the high half column 2j + 1) as the bf16
// values n, exact (integers below 16; unsigned byte to f32, the high half).
__device__ __forceinline__ void nib16_to_bf16(const uint32_t w0, const uint32_t w1, bf16x8 &k0, bf16x8 &k1) {
    const uint32_t in[2] = {w0, w1};
    uint32_t p[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t lo = in[k] & 0x0F0F0F0Fu, hi = (in[k] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            p[4 * k + j] = pack_bf16_exact((float)((lo >> (8 * j)) & 0xFFu), (float)((hi >> (8 * j)) & 0xFFu));
    }
    k0 = __builtin_bit_cast(bf16x8, u32x4{p[0], p[1], p[2], p[3]});
    k1 = __builtin_bit_cast(bf16x8, u32x4{p[4], p[5], p[6], p[7]});
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 a, const bf16x8 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round-to-nearest-even bf16 of an f32 (the gfx950 packed converter).
__device__ __forceinline__ __bf16 to_bf16(float f) { return (__bf16)f; }

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, so that f can
// index register arrays with a compile-time constant.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace pg
