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

constexpr int kPanelRows = 128;
constexpr int kChunk = 4;

template <int MT>
__device__ __forceinline__ int lds_index(int buf, int kbl, int mt, int fi, int lane) {
    return (((buf * kChunk + kbl) * MT + mt) * 4 + fi) * 64 + lane;
}

// One workgroup's share of the product: weight rows [r_base, r_base + 128),
// blocks [kb0, kb1), all A rows.  The workgroup is 4 row groups x kKSplit
// consumer waves plus one producer wave:
//  - the producer copies the A fragments of chunk c+1 from global memory
//    straight into LDS buffer (c+1) & 1 (global_load_lds_dwordx4, no
//    registers) while the consumers work on chunk c;
//  - consumer (g, k) owns the 32 weight rows of row group g and, inside every
//    chunk, the blocks k, k + kKSplit, ...; it streams those weights through a
//    register ring WCH chunks deep and contracts them against LDS buffer c & 1;
//  - after the last chunk the kKSplit partial sums of a row group meet in LDS
//    and the k = 0 wave adds them (in order k = 0, 1, ...) and stores.
// Splitting K inside the workgroup puts two consumer waves on every SIMD, so
// one wave's matrix-core chain overlaps the other's vector work, without
// reading any weight or activation twice.  Consumers issue only weight loads,
// so their in-order vmcnt waits cover just the weights they are about to use;
// the producer waits for its own copies before each barrier.  Producer and
// consumers run separate loops that pass the same number of barriers (one per
// chunk, plus one before the first and one before the reduction).  Every load
// address is clamped into range (blocks past kb1 re-read the last block and
// are weighted by zero) and register arrays are indexed by compile-time
// constants only.
constexpr int kKSplit = 2;
constexpr int kRowGroups = 4;
constexpr int kConsumers = kRowGroups * kKSplit;
constexpr int kMmaThreads = (kConsumers + 1) * 64;

template <int MT, int WCH>
__device__ __forceinline__ void mma_panel(const MmaPanel &P, const int r_base, const int kb0,
                                          const int kb1, u32x4 *lds) {
    static_assert(kChunk % kKSplit == 0, "a chunk splits evenly between the K halves");
    constexpr int kPer = kChunk / kKSplit;  // blocks per chunk per consumer
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = P.cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int ml = lane & 31;
    const int h = lane >> 5;
    const int nblk = kb1 - kb0;
    const int nchunks = (nblk + kChunk - 1) / kChunk;
    auto blk_of = [&](int c, int kbl) __attribute__((always_inline)) {
        return min(kb0 + c * kChunk + kbl, kb1 - 1);
    };

    // Staged row behind A-tile row m = 32 mt + ml.
    int srow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 32 * mt + ml;
        srow[mt] = m < P.m_valid ? (P.src_list ? P.src_list[m] / P.src_div : m) : P.zero_row;
    }

    if (wave == kConsumers) {
        // ---------------- producer: A fragments into LDS, one chunk ahead
        auto copy_chunk = [&](int c, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int kbl = 0; kbl < kChunk; ++kbl) {
                const long long b = blk_of(c, kbl);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) {
                        const u32x4 *src = P.frag
                            ? P.xp + ((b * MT + mt) * 4 + fi) * 64 + lane
                            : P.xp + (((long long)srow[mt] * nb + b) * 2 + h) * 4 + fi;
                        __builtin_amdgcn_global_load_lds(
                            (const void *)src,
                            (__attribute__((address_space(3))) void *)(lds + lds_index<MT>(buf, kbl, mt, fi, 0)),
                            16, 0, 0);
                    }
            }
        };
        copy_chunk(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) copy_chunk(c + 1, (c + 1) & 1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        __syncthreads();  // the consumers' reduction barrier
        return;
    }

    // ---------------- consumers
    const int rg = wave % kRowGroups;
    const int kh = wave / kRowGroups;
    // The weight row this lane feeds to the matrix core and owns in the output.
    // Addresses are a wave-uniform base (scalar registers) plus a 32-bit lane offset.
    const int row_base = r_base + rg * 32;
    const int r = row_base + ml;
    const bool r_ok = r < P.rows;
    const int rl = r_ok ? r : P.rows - 1;
    const int q_off = (rl - row_base) * P.cols + 16 * h;
    const int s_off = (rl - row_base) * nb;
    const int8_t *q_wave = P.q + (long long)row_base * P.cols;
    const float *sc_wave = P.scale + (long long)row_base * nb;
    const float *birow = P.bias + (long long)rl * nb;

    u32x4 wq[WCH][kPer];
    float ws[WCH][kPer];
    auto load_w = [&](int c, u32x4 (&q)[kPer], float (&s)[kPer]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int b = blk_of(c, kh + kKSplit * j);
            q[j] = *reinterpret_cast<const u32x4 *>(q_wave + (long long)b * 32 + q_off);
            s[j] = sc_wave[(long long)b + s_off];
        }
    };
#pragma unroll
    for (int u = 0; u < WCH; ++u) load_w(u, wq[u], ws[u]);

    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
    const f32x16 zero{};

    // Bias term over the blocks [kb0, kb1) (k = 0 waves): K = 16 blocks a step,
    // blocks of the step outside the range contribute a zero bias.  Block-sum
    // fragment of group g, part p for tile mt: row layout
    // xs[(srow * ng + g) * 4 + 2 h + p], fragment layout xs[((g * MT + mt) * 2 + p) * 64 + lane].
    if (kh == 0) {
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
                const long long i0 = P.frag ? (((long long)g * MT + mt) * 2) * 64 + lane
                                            : ((long long)srow[mt] * ng + g) * 4 + 2 * h;
                const long long i1 = P.frag ? i0 + 64 : i0 + 1;
                acc[mt] = mfma_bf16(as_bf16x8(P.xs[i0]), bb, acc[mt]);
                acc[mt] = mfma_bf16(as_bf16x8(P.xs[i1]), bb, acc[mt]);
            }
        }
    }
    __syncthreads();

    auto chunk_step = [&](auto uc, const int c0) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        const int c = c0 + u;
        if (c < nchunks) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int kbl = kh + kKSplit * j;
                const u32x4 *f = lds + lds_index<MT>(c & 1, kbl, 0, 0, lane);
                bf16x8 b0, b1;
                q16_to_bf16(wq[u][j], b0, b1);
                f32x16 t[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 *fm = f + mt * 4 * 64;
                    t[mt] = mfma_bf16(as_bf16x8(fm[0]), b0, zero);
                    t[mt] = mfma_bf16(as_bf16x8(fm[64]), b1, t[mt]);
                    t[mt] = mfma_bf16(as_bf16x8(fm[128]), b0, t[mt]);
                    t[mt] = mfma_bf16(as_bf16x8(fm[192]), b1, t[mt]);
                }
                // A block past kb1 (last chunk only) re-reads the last block and is
                // weighted by zero, which keeps the chunk one branch-free stretch.
                const float s = kb0 + c * kChunk + kbl < kb1 ? ws[u][j] : 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][v] = fmaf(s, t[mt][v], acc[mt][v]);
            }
            load_w(c + WCH, wq[u], ws[u]);
            __syncthreads();
        }
    };
    for (int c0 = 0; c0 < nchunks; c0 += WCH)
        static_for<WCH>([&](auto uc) __attribute__((always_inline)) { chunk_step(uc, c0); });

    // Partial sums of the K halves meet in LDS (the stage buffers are free now):
    // slot [rg][k-1][mt][v][lane] for k >= 1.
    float *red = reinterpret_cast<float *>(lds);
    if (kh > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[((((rg * (kKSplit - 1) + kh - 1) * MT + mt) * 16 + v) * 64) + lane] = acc[mt][v];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int k = 1; k < kKSplit; ++k)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mt][v] += red[((((rg * (kKSplit - 1) + k - 1) * MT + mt) * 16 + v) * 64) + lane];

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
