// Matrix-core product of a q8-block weight panel with up to 64 staged
// activation rows (the batched prefill product and the grouped expert banks).
//
// The pages' prompt GEMM (gemma_batch.rs, `q8_2f_mm_r2`; nemotron_prefill.rs,
// `pb_q8_bank`) walks every weight once per pass, folds the per-column factor
// into the staged activations and multiplies the row factor onto the finished
// sum.  On gfx950 the same contraction runs on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16):
//  - a weight q in [-127, 127] is an exact bf16 integer (B operand);
//  - an activation x enters as the pair x_hi = bf16(x), x_lo = bf16(x - x_hi)
//    (A operand, two products), exact to about 2^-17 relative;
//  - the matrix core accumulates one 32-column block in f32; the block's
//    scale then multiplies that block sum on the vector ALU (scale belongs to
//    the weight row, so it cannot ride inside the contraction);
//  - the bias term sum_blk bias[r][blk] * Xsum[m][blk] is one more
//    contraction over blocks (K = 16 blocks a step), with Xsum the staged
//    per-block activation sum (hi + lo) and the bias rounded to bf16.
//
// Tile: a workgroup is 4 waves over 128 weight rows; each wave owns 32 rows
// (the 32 columns of the MFMA output) and all A rows (MT tiles of 32).  The A
// operand is staged through LDS, kChunk blocks per buffer, double buffered;
// each wave streams its own weights straight from HBM, 16 bytes a lane.
#pragma once

#include <utility>

#include "pg_device.h"

namespace pg {

// Staging layout of activation rows (written by stage_x_kernel):
//  xp: 64 bytes per (row, block blk, half h): [hi: k-step 0 | k-step 1][lo: k-step 0 | k-step 1],
//      8 bf16 each; element i of k-step ks of half h is column 32 blk + 16 h + 8 ks + i.
//      Record (row, blk, h) starts at uint4 index ((row * nb + blk) * 2 + h) * 4.
//  xs: 64 bytes per (row, group g of 16 blocks): [h][part][8 bf16], element i of half h is
//      the sum of the row's X over block 16 g + 8 h + i (zero past the last block).
//  The row after the last is all zeros; tile rows past the valid count read it.
//  This "row" layout serves gathered A rows (expert entries).  The dense pass
//  (A row m = position m) uses the "fragment" layout instead, in which the 64
//  lanes of one matrix-core fragment are contiguous (one 1 KB load a fragment):
//  xp: [blk][mt][fi = part * 2 + ks][lane = m % 32 + 32 h] 16 bytes each;
//  xs: [g][mt][part][lane = m % 32 + 32 h] 16 bytes each; rows past n are zero.
struct MmaPanel {
    const int8_t *q;
    const float *scale;
    const float *bias;
    int rows, cols;
    const u32x4 *xp;
    const u32x4 *xs;
    int zero_row;
    const int32_t *src_list;  // A row m reads staged row src_list[m] / src_div (NULL: row m)
    int src_div;
    int m_valid;              // A rows in use (<= 64)
    float *out;               // out[orow(m) * ldo + r]
    long long ldo;
    const int32_t *out_list;  // orow(m) = out_list[m] (NULL: m)
    int act;
    int frag;                 // 1: fragment layout (dense rows, MT tiles staged), 0: row layout
};

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

constexpr int kPanelRows = 128;
constexpr int kChunk = 4;

template <int MT>
__device__ __forceinline__ int lds_index(int buf, int kbl, int mt, int fi, int lane) {
    return (((buf * kChunk + kbl) * MT + mt) * 4 + fi) * 64 + lane;
}

// One workgroup's share of the product: weight rows [r_base, r_base + 128),
// blocks [kb0, kb1), all A rows.  Software pipeline, per chunk c of kChunk blocks:
//   - the A fragments of chunk c+1 (in registers since two chunks ago) go to
//     LDS buffer (c+1) & 1 and chunk c+3 is requested into the freed registers;
//   - chunk c is contracted from LDS buffer c & 1 and the weight registers of
//     ring slot c % WCH, which are then refilled with chunk c + WCH;
//   - one barrier closes the chunk.
// Every load is unconditional (block index clamped into the range, so the
// loads past the end re-read the last block) and every register array is
// indexed by compile-time constants, so nothing leaves the register file.
template <int MT, int WCH>
__device__ __forceinline__ void mma_panel(const MmaPanel &P, const int r_base, const int kb0,
                                          const int kb1, u32x4 *lds) {
    static_assert(WCH % 2 == 0, "the ring walk keeps the LDS buffer parity static");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb = P.cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int ml = lane & 31;
    const int h = lane >> 5;

    // Staged row behind A-tile row m = 32 mt + ml (the rows this lane loads).
    int srow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 32 * mt + ml;
        srow[mt] = m < P.m_valid ? (P.src_list ? P.src_list[m] / P.src_div : m) : P.zero_row;
    }

    // The weight row this lane feeds to the matrix core and owns in the output.
    // Addresses are a wave-uniform base (scalar registers) plus a 32-bit lane
    // offset, so the per-block address arithmetic stays off the vector ALU.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int row_base = r_base + wave_u * 32;
    const int r = row_base + ml;
    const bool r_ok = r < P.rows;
    const int rl = r_ok ? r : P.rows - 1;
    const int q_off = (rl - row_base) * P.cols + 16 * h;
    const int s_off = (rl - row_base) * nb;
    const int8_t *q_wave = P.q + (long long)row_base * P.cols;
    const float *sc_wave = P.scale + (long long)row_base * nb;
    const float *birow = P.bias + (long long)rl * nb;

    // This lane's A fragment of tile mt and block blk is
    //   a_base + blk * a_step + mt * a_mt + a_off[mt]   (a_off: lane part),
    // its block-sum fragment of group g and part p is
    //   P.xs + g * s_step + p * s_part + s_lane[mt].
    long long a_step, a_mt, s_step;
    int s_part;
    int a_off[MT], s_lane[MT];
    const u32x4 *a_base;
    if (P.frag) {
        a_base = P.xp + wave_u * 64;
        a_step = MT * 4 * 64;
        a_mt = 4 * 64;
        s_step = MT * 2 * 64;
        s_part = 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            a_off[mt] = lane;
            s_lane[mt] = mt * 2 * 64 + lane;
        }
    } else {
        a_base = P.xp + wave_u;
        a_step = 8;
        a_mt = 0;
        s_step = 4;
        s_part = 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            a_off[mt] = (srow[mt] * nb * 2 + h) * 4;
            s_lane[mt] = srow[mt] * ng * 4 + 2 * h;
        }
    }

    const int nblk = kb1 - kb0;
    const int nchunks = (nblk + kChunk - 1) / kChunk;
    auto blk_of = [&](int c, int kbl) __attribute__((always_inline)) { return min(kb0 + c * kChunk + kbl, kb1 - 1); };

    u32x4 wq[WCH][kChunk];
    float ws[WCH][kChunk];
    u32x4 st[2][kChunk * MT];

    auto load_w = [&](int c, u32x4 (&q)[kChunk], float (&s)[kChunk]) __attribute__((always_inline)) {
#pragma unroll
        for (int kbl = 0; kbl < kChunk; ++kbl) {
            const int b = blk_of(c, kbl);
            q[kbl] = *reinterpret_cast<const u32x4 *>(q_wave + (long long)b * 32 + q_off);
            s[kbl] = sc_wave[(long long)b + s_off];
        }
    };
    auto load_a = [&](int c, u32x4 (&dst)[kChunk * MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kChunk * MT; ++i) {
            const int kbl = i / MT, mt = i % MT;
            const u32x4 *base = a_base + (long long)blk_of(c, kbl) * a_step + mt * a_mt;
            dst[i] = base[a_off[mt]];
        }
    };
    auto store_a = [&](int buf, const u32x4 (&src)[kChunk * MT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kChunk * MT; ++i)
            lds[lds_index<MT>(buf, i / MT, i % MT, wave, lane)] = src[i];
    };

    // Prologue: weights of the first WCH chunks, A of chunk 0 in LDS, A of
    // chunks 1 and 2 on their way.
#pragma unroll
    for (int u = 0; u < WCH; ++u) load_w(u, wq[u], ws[u]);
    load_a(0, st[0]);
    store_a(0, st[0]);
    load_a(1, st[1]);
    load_a(2, st[0]);

    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
    const f32x16 zero{};

    // Bias term over the blocks [kb0, kb1): K = 16 blocks a step, blocks of
    // the step outside the range contribute a zero bias.
    for (int g = kb0 >> 4; g * 16 < kb1; ++g) {
        bf16x8 bb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = 16 * g + 8 * h + i;
            const bool in = blk >= kb0 && blk < kb1;
            const float v = birow[in ? blk : kb0];
            bb[i] = to_bf16(in ? v : 0.0f);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x4 *xr = P.xs + g * s_step;
            acc[mt] = mfma_bf16(as_bf16x8(xr[s_lane[mt]]), bb, acc[mt]);
            acc[mt] = mfma_bf16(as_bf16x8(xr[s_lane[mt] + s_part]), bb, acc[mt]);
        }
    }
    __syncthreads();

    auto chunk_step = [&](auto uc, const int c0) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        const int c = c0 + u;
        if (c < nchunks) {
            store_a((u + 1) & 1, st[(u + 1) & 1]);
            load_a(c + 3, st[(u + 1) & 1]);
            // A block past kb1 (last chunk only) re-reads the last block and is
            // weighted by zero, which keeps the chunk one branch-free stretch.
#pragma unroll
            for (int kbl = 0; kbl < kChunk; ++kbl) {
                bf16x8 b0, b1;
                q16_to_bf16(wq[u][kbl], b0, b1);
                const float s = kb0 + c * kChunk + kbl < kb1 ? ws[u][kbl] : 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 *f = lds + lds_index<MT>(u & 1, kbl, mt, 0, lane);
                    f32x16 t = mfma_bf16(as_bf16x8(f[0]), b0, zero);
                    t = mfma_bf16(as_bf16x8(f[64]), b1, t);
                    t = mfma_bf16(as_bf16x8(f[128]), b0, t);
                    t = mfma_bf16(as_bf16x8(f[192]), b1, t);
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][v] = fmaf(s, t[v], acc[mt][v]);
                }
            }
            load_w(c + WCH, wq[u], ws[u]);
        }
        __syncthreads();
    };
    for (int c0 = 0; c0 < nchunks; c0 += WCH) static_for<WCH>([&](auto uc) __attribute__((always_inline)) { chunk_step(uc, c0); });

    // Output: element v of tile mt is A row 32 mt + 8 (v / 4) + 4 h + (v % 4), column r.
    if (r_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
                if (m < P.m_valid) {
                    const long long orow = P.out_list ? P.out_list[m] : m;
                    P.out[orow * P.ldo + r] = apply_act(P.act, acc[mt][v]);
                }
            }
    }
}

}  // namespace pg
