// Matrix-core engine of the batched prefill product over one pass of up to 64
// positions (prefill_gemm_q8): every weight is read from HBM once per pass.
//
// nemotron_prefill.rs (module doc) sets the pass at PB_MAX = 64 positions so
// that one stream of the weights serves all of them; gemma_batch.rs
// (`q8_2f_mm_r2`) folds the per-column factor into the staged activations and
// multiplies the row factor onto the finished sum.  Here the same contraction
// runs on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16):
//  - a weight q in [-128, 127] is an exact bf16 integer (B operand, one weight
//    row per output column of the instruction);
//  - an activation x enters as x_hi = bf16(x) and x_lo = bf16(x - x_hi)
//    (A operand, two products), exact to about 2^-17 relative;
//  - the matrix core sums one 32-column block in f32, and the block's scale
//    multiplies that block sum on the vector ALU (the scale belongs to one
//    weight row and one block, so it cannot ride inside the contraction);
//  - the bias term sum_blk bias[r][blk] * Xsum[m][blk] is a second
//    contraction over blocks, K = 16 blocks an instruction, with the staged
//    block sums (hi + lo) and the bias split hi + lo as well.
//
// Work of one workgroup: 128 weight rows x a range of blocks x all positions,
// 2 NK waves.  Wave (rh, kq) owns rows 64 rh .. 64 rh + 63 (two matrix-core
// row tiles, so every activation fragment read from LDS feeds two weight
// tiles) and blocks kq * 4/NK .. of every stage of four blocks; at the end
// the NK partial sums of a row half meet in LDS, every K wave adding one
// quarter of each tile.  With NK = 4 two waves share every SIMD, so one
// wave's matrix-core chain overlaps the other's vector work.  Workgroup ids
// go to the chiplets in turn; the kernel maps them so that each chiplet takes
// a contiguous run of (split, panel) items and its L2 holds the staged
// activations of one or two K ranges.
//
// Memory path.  Every byte moves from global memory straight into LDS
// (buffer loads to LDS, no registers), shared out over all waves, NX - 1
// (activations, from L2) or NW - 1 (weights, from HBM) stages ahead:
//  - weights: one instruction copies 8 rows x 128 contiguous bytes (the
//    stage's four blocks of each row), so HBM sees whole lines of a row in one
//    request; the lane -> (row, 16-byte piece) assignment is permuted so that
//    the matrix-core reads (lane = row, one 16-byte piece) hit distinct LDS
//    banks;
//  - scales and biases: 16 rows x 4 blocks (4 bytes a lane) per instruction;
//  - activation fragments and block sums: as staged, 1 KB per instruction.
// Each stage requests the next activations at its start and the weights (and a
// bias share) once its matrix-core work is issued, so the activations are
// never queued behind that stage's weight requests.  A wave waits for its own
// copies of stage c + 1 (memory counter) before the stage barrier; copies are
// issued in the same order every stage, so the wait is one constant.  Blocks past the range inside a stage are weighted by
// zero, and copies for stages past the end go through empty buffer
// resources (zeros, no memory traffic), which keeps every stage one
// branch-free stretch.
//
// K splits.  When a product has too few 128-row panels to fill the device,
// workgroups split its blocks; every split writes its partial tile and the
// panel's last split to arrive adds all of them in split order (so the result
// does not depend on timing) and runs the epilogue (DenseMode).
#pragma once

#include "pg_device.h"

namespace pg {

// What the finished panel tile y[m][r] (positions m < n, the panel's rows)
// becomes (DenseArgs::mode):
//  kDensePlain   out[m][r] = act(y)
//  kDenseResid   out[m][r] = y; for r < hidden: h' = H[m][r] + y is written
//                back to H, w[r] * h' is staged as column r of the next
//                product's activations, and sumsq[panel][m] = the sum of h'^2
//                over the panel's rows (its part of the next RMSNorm)
//  kDenseScaled  v = act(y / sqrt(sum_p sumsq_in[p][m] / hidden + eps)) (p in
//                order); out[m][r] = v, staged as column r of the next
//                product's activations when nxp is set
// so that an add + RMSNorm between two products runs in the first one's
// epilogue and the second one's scaling, with no pass of its own.
enum DenseMode { kDensePlain = 0, kDenseResid = 1, kDenseScaled = 2 };

// Weight formats of the engine (template argument FMT):
//  kFmtQ8   int8 + f32 scale + f32 bias per 32 columns (w = scale q + bias);
//  kFmtQ82  q8_2f: int8 body, f16 row scale on the finished sum (the f16
//           column field is already folded into the staged activations);
//  kFmtQ4   q4tp: 4-bit codes (w = 2^(base + code_g step) (nib - 8)), the
//           nibble n entering the matrix cores as the exact bf16 n, and the
//           - 8 through the bias contraction: per group the bias is
//           -8 * scale, so scale (sum n x) - 8 scale sum x = scale sum (n - 8) x.
enum DenseFmt { kFmtQ8 = 0, kFmtQ82 = 1, kFmtQ4 = 2 };

struct DenseArgs {
    const int8_t *q;
    const float *scale;
    const float *bias;
    const uint16_t *rs;  // q8_2f variant: binary16 row scales (scale and bias unused)
    // q4tp variant (q, scale, bias unused): nibbles [rows][cols / 2], parameter
    // words [rows] (binary16 base low, step high), 5-bit group codes
    // [rows][code_stride] (least significant bit first, bit 5 g for group g)
    const uint8_t *nib;
    const uint32_t *params;
    const uint8_t *codes;
    int code_stride;
    uint32_t code_bytes;  // rows * code_stride
    int rows, cols;
    const u32x4 *xp;  // staged A fragments [nb][mts][4][64] (see stage_x_frag_kernel)
    const u32x4 *xs;  // staged block sums [ng][mts][2][64]
    int mts;          // position tiles staged (>= MT)
    int n;            // positions in use
    float *out;       // out[m * ldo + r]
    long long ldo;
    int act;
    // K splits: split s of panel p writes its partial tile [m][128] to
    // parts + ((s * n + m) * panels + p) * 128; the last split of the panel to
    // arrive (tickets[p], zeroed before the launch) adds them in split order
    // and runs the epilogue.
    int splits;
    int split;  // this workgroup's split
    float *parts;
    unsigned *tickets;
    // epilogue
    int mode;
    float *H;               // kDenseResid: residual [n][hidden], updated in place
    const float *w;         // kDenseResid: norm weight [hidden]
    int hidden;             // columns of the residual / of the RMSNorm
    float *sumsq;           // kDenseResid: [ceil(hidden / 128)][n] written
    const float *sumsq_in;  // kDenseScaled: [ceil(hidden / 128)][n] read
    float eps;
    u32x4 *nxp;             // next product's staged fragments (NULL: none)
    __bf16 *nxs;            // next product's staged block sums
    int nnb;                // next product's blocks (its cols / 32)
    // Pass size on the device (nemotron_prefill.rs keeps n and pos0 in its
    // `Meta` uniform so that the pass is built once): meta = {n, pos0}, read at
    // launch; out and H then address row pos0 of the prompt's buffers, which
    // hold rows_total rows.  NULL: n above is the pass size.
    const int *meta;
    int rows_total;
    int nl;                 // positions the layouts of parts / sumsq are sized for
};

// Resolve a device-side pass size into P (n, out, H); false if the pass is
// empty or outside the buffers (then nothing is to be done).
__device__ __forceinline__ bool dense_resolve_meta(DenseArgs &P) {
    if (!P.meta) return true;
    const int n = __builtin_amdgcn_readfirstlane(P.meta[0]);
    const int pos0 = __builtin_amdgcn_readfirstlane(P.meta[1]);
    if (n < 1 || n > P.nl || pos0 < 0 || pos0 > P.rows_total - n) return false;
    P.n = n;
    P.out += (long long)pos0 * P.ldo;
    if (P.H) P.H += (long long)pos0 * P.hidden;
    return true;
}

// Fragment layout of the staged activations: the 64 lanes of one matrix-core
// fragment are contiguous (one 1 KB load a fragment).
//  xp: [blk][mt][fi = part * 2 + ks][lane = m % 32 + 32 h], 16 bytes each:
//      part 0 = hi, 1 = lo; element i of k-step ks of half h is column
//      32 blk + 16 h + 8 ks + i;
//  xs: [g][mt][part][lane = m % 32 + 32 h], 16 bytes each: element i of half h
//      is the sum of row m over block 16 g + 8 h + i (zero past the last block).
// Rows m >= n are zero.
//
// Fragment-layout record of one half block (16 columns, half h of block blk)
// of A row m: the hi/lo bf16 pair of each value, and (h == 0 lane) the
// block's sum.  Lanes 2i and 2i + 1 hold the two halves of one block.
__device__ __forceinline__ void put_frag_half(const float v[16], int m, int blk, int h, int nb, int mts,
                                              u32x4 *__restrict__ xp, __bf16 *__restrict__ xs) {
    const int mt = m >> 5, lane = (m & 31) + 32 * h;
    __bf16 hi[16], lo[16];
    float half_sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        hi[i] = to_bf16(v[i]);
        lo[i] = to_bf16(v[i] - (float)hi[i]);
        half_sum += v[i];
    }
    if (blk < nb) {
        u32x4 rec[4];
        __builtin_memcpy(&rec[0], &hi[0], 16);
        __builtin_memcpy(&rec[1], &hi[8], 16);
        __builtin_memcpy(&rec[2], &lo[0], 16);
        __builtin_memcpy(&rec[3], &lo[8], 16);
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) xp[(((long long)blk * mts + mt) * 4 + fi) * 64 + lane] = rec[fi];
    }
    const float block_sum = half_sum + __shfl_xor(half_sum, 1, kWave);
    if (h == 0) {
        const __bf16 s_hi = to_bf16(block_sum);
        const __bf16 s_lo = to_bf16(block_sum - (float)s_hi);
        const int g = blk >> 4, hh = (blk >> 3) & 1, i = blk & 7;
        const int sl = (m & 31) + 32 * hh;
        xs[((((long long)g * mts + mt) * 2 + 0) * 64 + sl) * 8 + i] = s_hi;
        xs[((((long long)g * mts + mt) * 2 + 1) * 64 + sl) * 8 + i] = s_lo;
    }
}

template <int MT, int NK, int NX, int NW>
struct DenseCfg {
    static constexpr int kWaves = 2 * NK;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kRows = 128;
    static constexpr int kKB = 4;                        // blocks per stage
    static constexpr int kStagesPerGroup = 4;            // 16 blocks: one bias group
    // LDS map, in 16-byte slots.
    static constexpr int kXStage = kKB * MT * 4 * 64;    // activation fragments of a stage
    static constexpr int kWq = 16 * 64;                  // 128 rows x 128 bytes
    static constexpr int kWs = 128;                      // 128 rows x 4 scales
    static constexpr int kWStage = kWq + kWs;
    static constexpr int kBGroup = 512;                  // 128 rows x 16 biases of a group
    static constexpr int kXBase = 0;
    static constexpr int kWBase = NX * kXStage;
    static constexpr int kBBase = kWBase + NW * kWStage;  // bias ring: 2 groups
    static constexpr int kSBase = kBBase + 2 * kBGroup;   // block-sum ring: 2 groups
    static constexpr int kSGroup = 2 * MT * 64;
    static constexpr int kLdsU4 = kSBase + 2 * kSGroup;
    static constexpr int kRedU4 = (NK - 1) * 2 * 2 * MT * 16 * 64 / 4;  // K partials of both row halves
    static constexpr int kBPW = 4 / NK;                  // blocks per wave per stage
    static constexpr int kXPer = 16 * MT / kWaves;       // activation fragments per wave per stage
    static constexpr int kQPer = 16 / kWaves;            // weight copies (8 rows each)
    static constexpr int kSPer = 8 / kWaves;             // scale copies (16 rows each)
    static constexpr int kBPer = 32 / kWaves / 4;        // bias copies (4 rows x 16) per wave per stage
    static_assert(NK == 4, "K waves per row half: one block per wave per stage");
    static constexpr int kTileU4 = 64 * 128 / 4;          // the finished panel tile [m][128] f32
    static constexpr int kTileBase = kRedU4;
    static_assert(kRedU4 + kTileU4 + 17 <= kLdsU4, "the partial sums, the tile and its scalars fit the ring");
    static_assert(kLdsU4 * 16 <= 160 * 1024, "LDS of one compute unit");
    // Copies one wave issues per stage, and the memory-counter wait that
    // leaves in flight only the copies issued after stage c + 1's activations.
    static constexpr int kXCopies = kXPer + 1;
    static constexpr int kWCopies = kQPer + kSPer + kBPer;
    static constexpr int kWait = kWCopies + (NX - 2) * (kXCopies + kWCopies);
    static_assert(NX >= 2 && NW > NX, "weights are requested further ahead than activations");
    static_assert(kWait <= 63, "outstanding copies fit the memory counter");
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): out-of-range lanes read zero.
__device__ __forceinline__ i32x4 buf_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32) & 0xffff, (int32_t)bytes, 0x00020000};
}

// Copy SIZE (16 or 4) bytes a lane from buffer offset voff (per lane, range
// checked) to LDS at lds_wave_base + SIZE * lane.  Written as inline assembly
// so that the compiler does not see an LDS store it cannot place: it would
// otherwise wait for every outstanding copy before each LDS read, which
// serialises the rings.  Completion is tracked by hand (wait_vm) before the
// stage barriers.  lds_addr is the LDS byte address of lane 0's destination.
template <int SIZE, bool NT = false>
__device__ __forceinline__ void lds_copy(const i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    if constexpr (SIZE == 16 && NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(m0), "v"(voff),
                     "s"(rsrc)
                     : "memory", "m0");
    else if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff),
                     "s"(rsrc)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff),
                     "s"(rsrc)
                     : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS slot (16 bytes) of row (0..127) and 16-byte piece s (0..7) of a weight
// stage.  Copy instruction i = row / 8 holds rows 8i .. 8i + 7; its lane l
// carries row 8i + ((l / 8) ^ (i & 1)) and piece (l % 8) ^ (row % 8).  For a
// fixed piece, 16 consecutive rows land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int wq_slot(int row, int s) {
    const int i = row >> 3, r8 = row & 7;
    return i * 64 + 8 * (r8 ^ (i & 1)) + (s ^ r8);
}

// The panel's finished tile and its epilogue (DenseArgs::mode).  With K
// splits, every split has written its partial tile; the last to arrive adds
// them in split order into LDS, the others leave.  Then thread t takes
// position m = t / 8 and the 16 rows 16 (t % 8) .. of the panel (threads 2i,
// 2i + 1 hold the two halves of one 32-row block of the next product's
// columns).
template <int MT, int NK, int NX, int NW, int FMT = kFmtQ8>
__device__ __forceinline__ void dense_finish(const DenseArgs &P, const int r_base, u32x4 *lds) {
    using C = DenseCfg<MT, NK, NX, NW>;
    constexpr bool Q82 = FMT == kFmtQ82;
    static_assert(C::kThreads == 512, "one thread per (position, 16 rows) of a 64 x 128 tile");
    float *tile = reinterpret_cast<float *>(lds + C::kTileBase);
    float *s_inv = reinterpret_cast<float *>(lds + C::kTileBase + C::kTileU4);  // [64]
    unsigned &s_ticket = *reinterpret_cast<unsigned *>(lds + C::kTileBase + C::kTileU4 + 16);
    const int t = threadIdx.x;
    const int panel = r_base / C::kRows;
    const int prow = min(C::kRows, P.rows - r_base);  // rows of this panel
    if (P.splits > 1) {
        // This split's tile goes out as 16-byte chunks (chunk c: position
        // c / 32, rows 4 (c % 32) ..), written at device scope so that the
        // panel's last split reads them from another compute unit.
        __syncthreads();  // the tile is complete
        const int panels = (P.rows + C::kRows - 1) / C::kRows;
        const int chunks = P.n * 32;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            P.parts, (short)0, P.splits * P.nl * panels * C::kRows * 4, 0x00020000);
        auto chunk_off = [&](int sp, int c) __attribute__((always_inline)) {
            return (((sp * P.nl + (c >> 5)) * panels + panel) * C::kRows + 4 * (c & 31)) * 4;
        };
        constexpr int kC = 64 * 32 / C::kThreads;  // chunks per thread (n <= 64)
        constexpr int kDev = 16;                    // buffer cache policy: device scope
#pragma unroll
        for (int k = 0; k < kC; ++k) {
            const int c = t + k * C::kThreads;
            if (c < chunks)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4 *>(tile + 4 * c), rp,
                                                       chunk_off(P.split, c), 0, kDev);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this split's partial has landed
        __syncthreads();
        if (t == 0) s_ticket = __hip_atomic_fetch_add(P.tickets + panel, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_ticket != (unsigned)P.splits - 1) return;
        // Last split: y = sum_s parts[s] in split order, the loads of four
        // splits in flight at a time.
        constexpr int kS = 4;
        float4 y[kC];
#pragma unroll
        for (int k = 0; k < kC; ++k) y[k] = make_float4(0, 0, 0, 0);
        for (int s0 = 0; s0 < P.splits; s0 += kS) {
            u32x4 v[kS][kC];
#pragma unroll
            for (int si = 0; si < kS; ++si)
#pragma unroll
                for (int k = 0; k < kC; ++k) {
                    const int c = t + k * C::kThreads;
                    v[si][k] = (s0 + si < P.splits && c < chunks)
                                   ? __builtin_amdgcn_raw_buffer_load_b128(rp, chunk_off(s0 + si, c), 0, kDev)
                                   : u32x4{0, 0, 0, 0};
                }
#pragma unroll
            for (int si = 0; si < kS; ++si)
#pragma unroll
                for (int k = 0; k < kC; ++k) {
                    if (s0 + si >= P.splits) continue;
                    const float4 a = __builtin_bit_cast(float4, v[si][k]);
                    if (s0 + si == 0) {
                        y[k] = a;
                    } else {
                        y[k].x += a.x; y[k].y += a.y; y[k].z += a.z; y[k].w += a.w;
                    }
                }
        }
#pragma unroll
        for (int k = 0; k < kC; ++k) {
            const int c = t + k * C::kThreads;
            if (c < chunks) *reinterpret_cast<float4 *>(tile + 4 * c) = y[k];
        }
    }
    if (P.mode == kDenseScaled && t < 64) {
        // The panels' sums in panel order, the loads of 16 panels in flight.
        float ss = 0.0f;
        const int np = (P.hidden + C::kRows - 1) / C::kRows;
        const int m = min(t, P.n - 1);
        for (int p0 = 0; p0 < np; p0 += 16) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = p0 + k < np ? P.sumsq_in[(p0 + k) * P.nl + m] : 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) ss += v[k];
        }
        s_inv[t] = rsqrtf(ss / (float)P.hidden + P.eps);
    }
    __syncthreads();

    const int m = t >> 3, j = (t >> 1) & 3, hh = t & 1;
    if (m >= P.mts * 32) return;
    const int rl0 = 32 * j + 16 * hh, r0 = r_base + rl0;
    // Rows of this item inside the matrix (the last panel may end inside an
    // item; rows past the end hold zeros).
    const int cnt = m < P.n ? max(0, min(16, prow - rl0)) : 0;
    const bool live = cnt > 0;
    float v[16];
    if (live) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 a = *reinterpret_cast<const float4 *>(tile + m * 128 + rl0 + 4 * q4);
            v[4 * q4] = a.x; v[4 * q4 + 1] = a.y; v[4 * q4 + 2] = a.z; v[4 * q4 + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    float *o = P.out + (long long)m * P.ldo + r0;
    auto store16 = [&](const float (&x)[16]) __attribute__((always_inline)) {
        if (cnt == 16 && (P.ldo & 3) == 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4 *>(o + 4 * q4) = make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < cnt) o[i] = x[i];
        }
    };
    if (P.mode == kDensePlain) {
        if (Q82) {
            // q8_2f: the row scale multiplies the finished sum.
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = min(r0 + i, P.rows - 1);
                v[i] *= (float)__builtin_bit_cast(_Float16, P.rs[r]);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = apply_act(P.act, v[i]);
        store16(v);
        return;
    }
    if (P.mode == kDenseScaled) {
        const float inv = s_inv[m];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = i < cnt ? apply_act(P.act, inv * v[i]) : 0.0f;
        store16(v);
        if (P.nxp && r0 < 16 * ((P.nnb + 15) / 16) * 32)
            put_frag_half(v, m, r0 >> 5, hh, P.nnb, P.mts, P.nxp, P.nxs);
        return;
    }
    // kDenseResid (hidden % 32 == 0: an item below hidden is whole)
    store16(v);
    float sq = 0.0f;
    if (r0 < P.hidden) {
        float x[16];
        float *hp = P.H + (long long)m * P.hidden + r0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            float4 a = make_float4(0, 0, 0, 0), g = make_float4(0, 0, 0, 0);
            if (live) {
                a = *reinterpret_cast<const float4 *>(hp + 4 * q4);
                g = *reinterpret_cast<const float4 *>(P.w + r0 + 4 * q4);
                a.x += v[4 * q4]; a.y += v[4 * q4 + 1]; a.z += v[4 * q4 + 2]; a.w += v[4 * q4 + 3];
                *reinterpret_cast<float4 *>(hp + 4 * q4) = a;
            }
            sq += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
            x[4 * q4] = g.x * a.x; x[4 * q4 + 1] = g.y * a.y; x[4 * q4 + 2] = g.z * a.z; x[4 * q4 + 3] = g.w * a.w;
        }
        put_frag_half(x, m, r0 >> 5, hh, P.nnb, P.mts, P.nxp, P.nxs);
    }
    // The eight threads of position m, in a fixed butterfly.
    sq += __shfl_xor(sq, 1, kWave);
    sq += __shfl_xor(sq, 2, kWave);
    sq += __shfl_xor(sq, 4, kWave);
    if ((t & 7) == 0 && r_base < P.hidden && m < P.n) P.sumsq[panel * P.nl + m] = sq;
}

template <int MT, int NK, int NX, int NW, int FMT = kFmtQ8>
__device__ __forceinline__ void dense_panel(const DenseArgs &P, const int r_base, const int kb0,
                                            const int kb1, u32x4 *lds) {
    using C = DenseCfg<MT, NK, NX, NW>;
    constexpr bool Q82 = FMT == kFmtQ82, Q4 = FMT == kFmtQ4;
    constexpr int KB = C::kKB;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = P.cols >> 5;
    const int ng = (nb + 15) >> 4;
    const int nst = (kb1 - kb0 + 15) / 16 * C::kStagesPerGroup;

    // ------------------------------------------------------------ copies
    // Per-lane buffer offsets at stage 0; a stage adds a wave-uniform step.
    // Reads past a row's blocks (the tail stage of a range) fetch valid bytes
    // that are weighted by zero; reads past a buffer's end return zero.
    // Copies for stages past the range go through empty resources: they
    // return zeros at once and move no memory.
    // q8_2f: no block scales or biases; their copies go through empty
    // resources (zeros, no memory traffic), so every count of copies stays.
    // q4tp: the nibbles take the weight copies (one per wave carries data,
    // 16 rows x 64 bytes), a 16-byte window of each row's group codes takes the
    // scale copies, and there are no bias copies at all (the compute writes
    // the group biases itself), so the memory-counter waits drop kBPer a stage.
    const i32x4 rq = Q4 ? buf_rsrc(P.nib, (uint32_t)P.rows * (uint32_t)(P.cols >> 1))
                        : buf_rsrc(P.q, (uint32_t)P.rows * (uint32_t)P.cols);
    const i32x4 rs = Q4 ? buf_rsrc(P.codes, (uint32_t)P.rows * (uint32_t)P.code_stride)
                        : buf_rsrc(P.scale, Q82 ? 0u : (uint32_t)P.rows * nb * 4u);
    const i32x4 rb = buf_rsrc(P.bias, (Q82 || Q4) ? 0u : (uint32_t)P.rows * nb * 4u);
    constexpr int kWaitF = Q4 ? C::kWait - C::kBPer : C::kWait;
    const i32x4 rx = buf_rsrc(P.xp, (uint32_t)nb * P.mts * 4096u);
    const i32x4 rxs = buf_rsrc(P.xs, (uint32_t)ng * P.mts * 2048u);
    auto live_rsrc = [](i32x4 r, bool live) __attribute__((always_inline)) {
        r[2] = live ? r[2] : 0;
        return r;
    };
    // LDS byte address of slot i (16 bytes) of the ring.
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4 *)lds;
    auto laddr = [&](int slot) __attribute__((always_inline)) { return lbase + 16u * (uint32_t)slot; };
    uint32_t oq[C::kQPer], os[C::kSPer];
#pragma unroll
    for (int k = 0; k < C::kQPer; ++k) {
        const int i = C::kQPer * w + k;
        if (Q4) {
            // rows 16 w + lane / 4, block (lane & 3) of the stage (16 bytes of nibbles)
            // position p = lane & 3 of row r's four slots holds block p ^ ((r % 16) / 4),
            // so that the 32 rows a matrix-core read touches spread over the LDS banks
            oq[k] = (uint32_t)(r_base + 16 * w + (lane >> 2)) * (uint32_t)(P.cols >> 1) +
                    (uint32_t)(kb0 + ((lane & 3) ^ ((lane >> 4) & 3))) * 16u;
        } else {
            const int r8 = (lane >> 3) ^ (i & 1);
            const int s = (lane & 7) ^ r8;
            oq[k] = (uint32_t)(r_base + 8 * i + r8) * (uint32_t)P.cols +
                    (uint32_t)(kb0 * 32 + (s >> 1) * 32 + (s & 1) * 16);
        }
    }
#pragma unroll
    for (int k = 0; k < C::kSPer; ++k)
        os[k] = ((uint32_t)(r_base + 16 * (C::kSPer * w + k) + (lane >> 2)) * (uint32_t)nb +
                 (uint32_t)(kb0 + (lane & 3))) * 4u;
    // Fragment g = w * kXPer + f of a stage is block g / (4 MT), fragment g % (4 MT).
    const uint32_t ox = ((uint32_t)(kb0 * P.mts * 4) * 64u + lane) * 16u;
    const int fs = w % (2 * MT);
    const uint32_t oxs = ((uint32_t)((((kb0 >> 4) * P.mts + fs % MT) * 2 + fs / MT) * 64) + lane) * 16u;

    // Activation fragments of stage c and one block-sum fragment of its group
    // (fragment w mod 2 MT), into X slot c % NX.
    auto copy_x = [&](int c) __attribute__((always_inline)) {
        const int xslot = C::kXBase + (c % NX) * C::kXStage;
        const uint32_t step = (uint32_t)(c * KB * P.mts) * 4096u;
        const i32x4 rxc = live_rsrc(rx, c < nst), rxsc = live_rsrc(rxs, c < nst);
#pragma unroll
        for (int f = 0; f < C::kXPer; ++f) {
            const int g = w * C::kXPer + f;
            const uint32_t src = (uint32_t)((g / (4 * MT)) * P.mts * 4 + g % (4 * MT)) * 1024u;
            lds_copy<16>(rxc, ox + step + src, laddr(xslot + g * 64));
        }
        const int it = c / C::kStagesPerGroup;
        lds_copy<16>(rxsc, oxs + (uint32_t)(it * P.mts) * 2048u, laddr(C::kSBase + (it & 1) * C::kSGroup + fs * 64));
    };
    // Weights and scales of stage c for this wave's rows, into W slot c % NW
    // (layout: q pieces by wq_slot, then [row][4] scales), and this wave's
    // share of the biases of the next group (4 rows x 16 blocks a copy, layout
    // [row][16]) into bias slot (group + 1) % 2.
    const uint32_t ob = ((uint32_t)(r_base + (lane >> 4)) * (uint32_t)nb + (uint32_t)(kb0 + 16 + (lane & 15))) * 4u;
    auto copy_b = [&](int it, int p) __attribute__((always_inline)) {
        if (Q4) return;  // q4tp: the group biases are written by the compute
        // rows 4p .. 4p + 3 of group it
        lds_copy<4>(live_rsrc(rb, it * C::kStagesPerGroup < nst), ob + (uint32_t)(4 * p) * (uint32_t)nb * 4u + (uint32_t)(16 * (it - 1)) * 4u,
                    laddr(C::kBBase + (it & 1) * C::kBGroup + p * 16));
    };
    // q4tp: lane l of the wave's code copy: row 16 w + l / 4, dword l & 3 of the
    // 16 bytes from the aligned dword holding the row's first code bit of the stage.
    const uint32_t crow = (uint32_t)(r_base + 16 * w + (lane >> 2)) * (uint32_t)P.code_stride;
    auto code_off = [&](int c) __attribute__((always_inline)) {
        const uint32_t byte = (uint32_t)(5 * (kb0 + c * KB)) >> 3;
        return ((crow + byte) & ~3u) + 4u * (uint32_t)(lane & 3);
    };
    auto copy_w = [&](int c) __attribute__((always_inline)) {
        const int wslot = C::kWBase + (c % NW) * C::kWStage;
        const uint32_t sq = (uint32_t)(c * KB) * 32u, ss = (uint32_t)(c * KB) * 4u;
        const i32x4 rqc = live_rsrc(rq, c < nst), rsc = live_rsrc(rs, c < nst);
#pragma unroll
        // weights non-temporal: each is used once, which keeps the activations in L2
        for (int k = 0; k < C::kQPer; ++k) {
            if (Q4)  // one copy a wave carries the stage's nibbles; the rest are empty
                lds_copy<16, true>(k == 0 ? rqc : live_rsrc(rqc, false), oq[k] + (uint32_t)(c * KB) * 16u,
                                   laddr(wslot + (C::kQPer * w + k) * 64));
            else
                lds_copy<16, true>(rqc, oq[k] + sq, laddr(wslot + (C::kQPer * w + k) * 64));
        }
#pragma unroll
        for (int k = 0; k < C::kSPer; ++k) {
            if (Q4)
                lds_copy<4>(rsc, code_off(c), laddr(wslot + C::kWq + (C::kSPer * w + k) * 16));
            else
                lds_copy<4>(rsc, os[k] + ss, laddr(wslot + C::kWq + (C::kSPer * w + k) * 16));
        }
    };

    // Prologue: W(0), X(0), X(1 .. NX - 2), W(1 .. NW - 2).
    copy_w(0);
    copy_x(0);
    for (int c = 1; c < NX - 1; ++c) copy_x(c);
    for (int c = 1; c < NW - 1; ++c) copy_w(c);
#pragma unroll
    for (int k = 0; k < 4 * C::kBPer; ++k) copy_b(0, (4 * w + k / C::kBPer) * C::kBPer + k % C::kBPer);
    // Stage 0 only: the copies issued after X(0) (the other prologue stages and
    // group 0's biases) may still be in flight; the stage-end waits cover them.
    wait_vm<(NX - 2) * C::kXCopies + (NW - 2) * (C::kQPer + C::kSPer) + (Q4 ? 0 : 4 * C::kBPer)>();
    __builtin_amdgcn_s_barrier();

    // ------------------------------------------------------------ compute
    const int rh = w & 1, kq = w >> 1;
    const int h = lane >> 5;
    const int ml = lane & 31;
    // q4tp: base and step of this lane's two rows (binary16 halves of the parameter word)
    float qb0 = 0.0f, qs0 = 0.0f, qb1 = 0.0f, qs1 = 0.0f;
    if constexpr (Q4) {
        const uint32_t p0 = P.params[min(r_base + 64 * rh + ml, P.rows - 1)];
        const uint32_t p1 = P.params[min(r_base + 64 * rh + ml + 32, P.rows - 1)];
        qb0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p0 & 0xFFFFu));
        qs0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p0 >> 16));
        qb1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p1 & 0xFFFFu));
        qs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(p1 >> 16));
    }
    f32x16 acc[2][MT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x16{};
    const f32x16 zero{};
    // Software pipeline over the two row tiles: a stage's matrix-core chain of
    // tile 0 runs while the vector ALU applies the previous stage's tile-1
    // scale and converts tile 1's weights; tile 1's chain runs while tile 0's
    // scale is applied.  Tile 1's products (t1, scale s1) carry over the barrier.
    f32x16 t1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) t1[mt] = zero;
    float s1 = 0.0f;

    // Bias term of group g on the calling K wave: sum over the group's blocks of
    // bias[r][blk] * (block sum of x)[m][blk] (hi + lo on both sides); zero past kb1.
    auto bias_mfma = [&](int g) __attribute__((always_inline)) {
            // Bias term of the group on one K wave (in turn); zero past kb1.
            const u32x4 *sf = lds + C::kSBase + (g & 1) * C::kSGroup + lane;
            const float *bg = reinterpret_cast<const float *>(lds + C::kBBase + (g & 1) * C::kBGroup);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int row = 64 * rh + 32 * rt + ml;
                const float4 b0 = *reinterpret_cast<const float4 *>(bg + 16 * row + 8 * h);
                const float4 b1 = *reinterpret_cast<const float4 *>(bg + 16 * row + 8 * h + 4);
                const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                bf16x8 bh, bl;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float v = kb0 + 16 * g + 8 * h + i < kb1 ? bv[i] : 0.0f;
                    const __bf16 vh = to_bf16(v);
                    bh[i] = vh;
                    bl[i] = to_bf16(v - (float)vh);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 sh = as_bf16x8(sf[mt * 64]), sl = as_bf16x8(sf[(MT + mt) * 64]);
                    acc[rt][mt] = mfma_bf16(sh, bh, acc[rt][mt]);
                    acc[rt][mt] = mfma_bf16(sl, bh, acc[rt][mt]);
                    acc[rt][mt] = mfma_bf16(sh, bl, acc[rt][mt]);
                }
            }
    };

    for (int c = 0; c < nst; ++c) {
        const int u = c % C::kStagesPerGroup;
        const int it = c / C::kStagesPerGroup;
        // Refill the activation slot stage c - 1 used (every wave is past it).
        // The weight refill waits until this stage's matrix-core work is issued:
        // a compute unit returns its requests in order, so activations requested
        // ahead of weights arrive without waiting for them.
        copy_x(c + NX - 1);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4 *xst = lds + C::kXBase + (c % NX) * C::kXStage + lane;
        const u32x4 *wst = lds + C::kWBase + (c % NW) * C::kWStage;
        const float *sst = reinterpret_cast<const float *>(wst + C::kWq);

        const int kbl = kq;  // one block per wave per stage
        const bool live = kb0 + c * KB + kbl < kb1;
        u32x4 a[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) a[mt][fi] = xst[((kbl * MT + mt) * 4 + fi) * 64];
        const int row0 = 64 * rh + ml, row1 = row0 + 32;
        u32x4 q0, q1;
        if constexpr (Q4) {
            // 8 bytes (columns 16 h .. 16 h + 15 of block kbl) of each row's nibbles
            const uint8_t *wb = reinterpret_cast<const uint8_t *>(wst);
            auto nslot = [&](int r) __attribute__((always_inline)) {
                return 128 * (r >> 4) + 4 * (r & 15) + (kbl ^ ((r >> 2) & 3));
            };
            const uint2 v0 = *reinterpret_cast<const uint2 *>(wb + 16 * nslot(row0) + 8 * h);
            const uint2 v1 = *reinterpret_cast<const uint2 *>(wb + 16 * nslot(row1) + 8 * h);
            q0 = u32x4{v0.x, v0.y, 0u, 0u};
            q1 = u32x4{v1.x, v1.y, 0u, 0u};
        } else {
            q0 = wst[wq_slot(row0, 2 * kbl + h)];
            q1 = wst[wq_slot(row1, 2 * kbl + h)];
        }
        auto to_b = [&](const u32x4 q, bf16x8 &k0, bf16x8 &k1) __attribute__((always_inline)) {
            if constexpr (Q4) {
                nib16_to_bf16(q.x, q.y, k0, k1);
            } else {
                q16_to_bf16(q, k0, k1);
            }
        };
        bf16x8 b00, b01, b10, b11;
        if constexpr (Q82) {
            // q8_2f: no block factors, so both tiles accumulate straight into
            // their sums (blocks past the range meet zero activations).
            (void)live;
            q16_to_bf16(q0, b00, b01);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[0][mt] = mfma_bf16(as_bf16x8(a[mt][0]), b00, acc[0][mt]);
                acc[0][mt] = mfma_bf16(as_bf16x8(a[mt][1]), b01, acc[0][mt]);
                acc[0][mt] = mfma_bf16(as_bf16x8(a[mt][2]), b00, acc[0][mt]);
                acc[0][mt] = mfma_bf16(as_bf16x8(a[mt][3]), b01, acc[0][mt]);
            }
            q16_to_bf16(q1, b10, b11);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[1][mt] = mfma_bf16(as_bf16x8(a[mt][0]), b10, acc[1][mt]);
                acc[1][mt] = mfma_bf16(as_bf16x8(a[mt][1]), b11, acc[1][mt]);
                acc[1][mt] = mfma_bf16(as_bf16x8(a[mt][2]), b10, acc[1][mt]);
                acc[1][mt] = mfma_bf16(as_bf16x8(a[mt][3]), b11, acc[1][mt]);
            }
        } else {
        float sl0, sl1;
        if constexpr (Q4) {
            // group scale 2^(base + code step) from the row's 16-byte code window
            const uint32_t bit0 = 5u * (uint32_t)(kb0 + c * KB);
            auto q4_scale = [&](int r, float base, float step) __attribute__((always_inline)) {
                // first code byte of the stage in the row, and the aligned dword the copy started at
                const uint32_t at = (uint32_t)(r_base + r) * (uint32_t)P.code_stride + (bit0 >> 3);
                const uint32_t a4 = at & ~3u;
                uint64_t win;
                if (a4 + 8u <= P.code_bytes) {
                    const uint32_t *cw = reinterpret_cast<const uint32_t *>(wst + C::kWq) + 4 * r;
                    win = (uint64_t)cw[0] | ((uint64_t)cw[1] << 32);
                } else {
                    // the buffer's last bytes: a copied dword that ran past the end
                    // came back as zero, so read the bytes that exist directly
                    win = 0;
                    for (uint32_t k = 0; k < 8u; ++k)
                        if (a4 + k < P.code_bytes) win |= (uint64_t)P.codes[a4 + k] << (8u * k);
                }
                const uint32_t sh = 8u * (at & 3u) + (bit0 & 7u) + 5u * (uint32_t)kbl;
                const uint32_t code = (uint32_t)(win >> sh) & 31u;
                return __builtin_amdgcn_exp2f(fmaf((float)code, step, base));
            };
            sl0 = q4_scale(row0, qb0, qs0);
            sl1 = q4_scale(row1, qb1, qs1);
            // this block's bias (-8 scale) into the group's bias slot: row0 from
            // the lanes of half 0, row1 from half 1
            float *bgw = reinterpret_cast<float *>(lds + C::kBBase + (it & 1) * C::kBGroup);
            bgw[16 * (h ? row1 : row0) + 4 * u + kq] = live ? -8.0f * (h ? sl1 : sl0) : 0.0f;
        } else {
            sl0 = sst[4 * row0 + kbl];
            sl1 = sst[4 * row1 + kbl];
        }
        const float s0 = live ? sl0 : 0.0f;
        to_b(q0, b00, b01);
        // tile 0 chain; previous tile 1 scale step; tile 1 weights converted
        f32x16 t0[MT];
        // the position tiles' chains interleaved: no matrix-core instruction
        // waits on the one just issued
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t0[mt] = mfma_bf16(as_bf16x8(a[mt][0]), b00, zero);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t0[mt] = mfma_bf16(as_bf16x8(a[mt][1]), b01, t0[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t0[mt] = mfma_bf16(as_bf16x8(a[mt][2]), b00, t0[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t0[mt] = mfma_bf16(as_bf16x8(a[mt][3]), b01, t0[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[1][mt][v] = fmaf(s1, t1[mt][v], acc[1][mt][v]);
        to_b(q1, b10, b11);
        // tile 1 chain; tile 0 scale step
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t1[mt] = mfma_bf16(as_bf16x8(a[mt][0]), b10, zero);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t1[mt] = mfma_bf16(as_bf16x8(a[mt][1]), b11, t1[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t1[mt] = mfma_bf16(as_bf16x8(a[mt][2]), b10, t1[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t1[mt] = mfma_bf16(as_bf16x8(a[mt][3]), b11, t1[mt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[0][mt][v] = fmaf(s0, t0[mt][v], acc[0][mt][v]);
        s1 = live ? sl1 : 0.0f;
        }
        // Issue order: LDS reads, tile 0's conversion, then each matrix-core
        // instruction followed by a slice of independent vector work.
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * MT + 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
#pragma unroll
        for (int i = 0; i < 4 * MT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (16 * MT + 24) / (4 * MT), 0);
        }
#pragma unroll
        for (int i = 0; i < 4 * MT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // The weight slot stage c - 1 used, and a share of the next group's
        // biases (their slot was last read a group ago).
        copy_w(c + NW - 1);
#pragma unroll
        for (int k = 0; k < C::kBPer; ++k) copy_b(it + 1, (4 * w + u) * C::kBPer + k);

        if (!Q82 && !Q4 && u == C::kStagesPerGroup - 1 && kq == it % NK) bias_mfma(it);
        // q4tp: the group's biases are complete one barrier after its last stage
        if (Q4 && u == 0 && it > 0 && kq == (it - 1) % NK) bias_mfma(it - 1);

        // Stage c + 1's copies must have landed before the barrier.
        wait_vm<kWaitF>();
        __builtin_amdgcn_s_barrier();
    }

    if (Q4 && nst > 0) {  // the last group's bias term (its biases are complete after the last barrier)
        const int g = (nst - 1) / C::kStagesPerGroup;
        if (kq == g % NK) bias_mfma(g);
    }
    if (!Q82) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[1][mt][v] = fmaf(s1, t1[mt][v], acc[1][mt][v]);
    }

    // ------------------------------------------------------------ epilogue
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the trailing refills
    __builtin_amdgcn_s_barrier();
    // The K waves' partials meet in LDS as 16-byte pieces, and wave kq sums
    // piece v4 == kq of every tile (rt, mt) over the K waves in K order (the
    // same order for every piece).  Piece v4 of tile (rt, mt) from wave
    // k != v4 sits at red4[((j, rh, rt, mt), v4, lane)], j = k - (k > v4).
    // Element v of tile (rt, mt) is position 32 mt + 8 (v / 4) + 4 h + (v %
    // 4), row 64 rh + 32 rt + ml of the panel.
    u32x4 *red4 = lds;
    auto red_at = [&](int k, int rt, int mt, int v4) __attribute__((always_inline)) {
        const int j = k - (k > v4 ? 1 : 0);
        return ((((j * 2 + rh) * 2 + rt) * MT + mt) * 4 + v4) * 64 + lane;
    };
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                if (v4 != kq)
                    red4[red_at(kq, rt, mt, v4)] =
                        u32x4{__float_as_uint(acc[rt][mt][4 * v4]), __float_as_uint(acc[rt][mt][4 * v4 + 1]),
                              __float_as_uint(acc[rt][mt][4 * v4 + 2]), __float_as_uint(acc[rt][mt][4 * v4 + 3])};
    __syncthreads();
    float *tile = reinterpret_cast<float *>(lds + C::kTileBase);  // [m][128]
    const bool direct = P.splits == 1 && P.mode == kDensePlain;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
        if (v4 != kq) continue;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float sum[4];
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    float pk[4];
                    if (k == v4) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk[i] = acc[rt][mt][4 * v4 + i];
                    } else {
                        const u32x4 r = red4[red_at(k, rt, mt, v4)];
                        pk[0] = __uint_as_float(r.x);
                        pk[1] = __uint_as_float(r.y);
                        pk[2] = __uint_as_float(r.z);
                        pk[3] = __uint_as_float(r.w);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) sum[i] = k == 0 ? pk[i] : sum[i] + pk[i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rt][mt][4 * v4 + i] = sum[i];
            }
        if (direct) {
            // Plain, unsplit: straight to the output (bounds by predication).
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int r = r_base + 64 * rh + 32 * rt + ml;
                const float rsc = Q82 ? (float)__builtin_bit_cast(_Float16, P.rs[min(r, P.rows - 1)]) : 1.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 32 * mt + 8 * v4 + 4 * h + i;
                        const float y = apply_act(P.act, Q82 ? acc[rt][mt][4 * v4 + i] * rsc : acc[rt][mt][4 * v4 + i]);
                        if (r < P.rows && m < P.n) P.out[m * P.ldo + r] = y;
                    }
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rl = 64 * rh + 32 * rt + ml;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tile[(32 * mt + 8 * v4 + 4 * h + i) * 128 + rl] = acc[rt][mt][4 * v4 + i];
            }
        }
    }
    if (direct) return;
    dense_finish<MT, NK, NX, NW, FMT>(P, r_base, lds);
}

}  // namespace pg
