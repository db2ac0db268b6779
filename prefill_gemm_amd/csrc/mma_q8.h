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

#include "pg_device.h"

namespace pg {

// Staging layout of activation rows (written by stage_x_kernel):
//  xp: 64 bytes per (row, block blk, half h): [hi: k-step 0 | k-step 1][lo: k-step 0 | k-step 1],
//      8 bf16 each; element i of k-step ks of half h is column 32 blk + 16 h + 8 ks + i.
//      Record (row, blk, h) starts at uint4 index ((row * nb + blk) * 2 + h) * 4.
//  xs: 64 bytes per (row, group g of 16 blocks): [h][part][8 bf16], element i of half h is
//      the sum of the row's X over block 16 g + 8 h + i (zero past the last block).
//  The row after the last is all zeros; tile rows past the valid count read it.
struct MmaPanel {
    const int8_t *q;
    const float *scale;
    const float *bias;
    int rows, cols;
    const uint4 *xp;
    const uint4 *xs;
    int zero_row;
    const int32_t *src_list;  // A row m reads staged row src_list[m] / src_div (NULL: row m)
    int src_div;
    int m_valid;              // A rows in use (<= 64)
    float *out;               // out[orow(m) * ldo + r]
    long long ldo;
    const int32_t *out_list;  // orow(m) = out_list[m] (NULL: m)
    int act;
};

constexpr int kPanelRows = 128;
constexpr int kChunk = 4;

template <int MT>
__device__ __forceinline__ int lds_index(int buf, int kbl, int mt, int fi, int lane) {
    return (((buf * kChunk + kbl) * MT + mt) * 4 + fi) * 64 + lane;
}

template <int MT>
__device__ __forceinline__ void mma_panel(const MmaPanel &P, const int r_base, const int kb0,
                                          const int kb1, uint4 *lds) {
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
    const int r = r_base + wave * 32 + ml;
    const bool r_ok = r < P.rows;
    const long long rl = r_ok ? r : P.rows - 1;
    const int8_t *qrow = P.q + rl * P.cols + 16 * h;
    const float *scrow = P.scale + rl * nb;
    const float *birow = P.bias + rl * nb;

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
            const float v = (blk >= kb0 && blk < kb1) ? birow[blk] : 0.0f;
            bb[i] = to_bf16(v);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 *xr = P.xs + ((long long)srow[mt] * ng + g) * 4 + 2 * h;
            acc[mt] = mfma_bf16(as_bf16x8(xr[0]), bb, acc[mt]);
            acc[mt] = mfma_bf16(as_bf16x8(xr[1]), bb, acc[mt]);
        }
    }

    // Main contraction.  Thread `tid` stages, for every (block, tile) of a
    // chunk, the fragment of type fi = wave (hi/lo x k-step) for its lane.
    const int nblk = kb1 - kb0;
    const int nchunks = (nblk + kChunk - 1) / kChunk;
    uint4 st[kChunk * MT];
    uint4 wq[kChunk], wq_n[kChunk];
    float ws[kChunk], ws_n[kChunk];

    auto load_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < kChunk * MT; ++i) {
            const int kbl = i / MT, mt = i % MT;
            const int blk = kb0 + c * kChunk + kbl;
            if (blk < kb1)
                st[i] = P.xp[(((long long)srow[mt] * nb + blk) * 2 + h) * 4 + wave];
        }
    };
    auto store_a = [&](int c, int buf) {
#pragma unroll
        for (int i = 0; i < kChunk * MT; ++i) {
            const int kbl = i / MT, mt = i % MT;
            const int blk = kb0 + c * kChunk + kbl;
            if (blk < kb1) lds[lds_index<MT>(buf, kbl, mt, wave, lane)] = st[i];
        }
    };
    auto load_w = [&](int c, uint4 *q, float *s) {
#pragma unroll
        for (int kbl = 0; kbl < kChunk; ++kbl) {
            const int blk = kb0 + c * kChunk + kbl;
            if (blk < kb1) {
                q[kbl] = *reinterpret_cast<const uint4 *>(qrow + blk * 32);
                s[kbl] = scrow[blk];
            }
        }
    };

    load_a(0);
    load_w(0, wq, ws);
    store_a(0, 0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) {
            load_a(c + 1);
            load_w(c + 1, wq_n, ws_n);
        }
#pragma unroll
        for (int kbl = 0; kbl < kChunk; ++kbl) {
            const int blk = kb0 + c * kChunk + kbl;
            if (blk < kb1) {
                bf16x8 b0, b1;
                q16_to_bf16(wq[kbl], b0, b1);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 *f = lds + lds_index<MT>(buf, kbl, mt, 0, lane);
                    f32x16 t = mfma_bf16(as_bf16x8(f[0]), b0, zero);
                    t = mfma_bf16(as_bf16x8(f[64]), b1, t);
                    t = mfma_bf16(as_bf16x8(f[128]), b0, t);
                    t = mfma_bf16(as_bf16x8(f[192]), b1, t);
                    const float s = ws[kbl];
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][v] = fmaf(s, t[v], acc[mt][v]);
                }
            }
        }
        if (more) {
            store_a(c + 1, buf ^ 1);
#pragma unroll
            for (int kbl = 0; kbl < kChunk; ++kbl) {
                wq[kbl] = wq_n[kbl];
                ws[kbl] = ws_n[kbl];
            }
        }
        __syncthreads();
    }

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
