// Grouped expert banks of the routed-MoE pass (moe_grouped).
//
// nemotron_prefill.rs, `pb_q8_bank`: one workgroup per (row block, expert); an
// expert that no entry chose returns at once; the expert's weights are read
// once for all of its entries.  For expert e with cnt entries m = 0 .. cnt-1
// (lists[e][m] = entry j, ascending):
//     out[j][r] = act( sum_c (scale[e][r][c/32] * q[e][r][c] + bias[e][r][c/32]) * x[j / src_div][c] )
// regrouped per 32-column block as scale * (sum_c q x) + bias * (sum_c x).
//
// A pass of 64 positions with top-6 over 128 experts gives about three entries
// per expert, so this is a matrix product with a very short side.  It runs on
// the 16 x 16 x 32 bf16 matrix cores (v_mfma_f32_16x16x32_bf16), which pad the
// entries only to 16:
//  - B operand = weights, exact bf16 integers; a step is 16 rows x 2 blocks
//    (1 KB a wave), and a pair of steps comes as two loads of 8 rows x 128
//    bytes (whole lines, non-temporal), from which a step's pieces are
//    gathered to 16 bytes of one row a lane (a half-row rotation, a select);
//  - lanes l and l + 32 trade the upper 8 bytes of those 16
//    (v_permlane32_swap), so that each matrix-core product sees 32 columns of
//    one block and the block scale can multiply its result;
//  - q4tp: a lane's 16 bytes cover one block of a pair of steps, and the four
//    lane groups of a row transpose them (two lane-half swaps, two row swaps)
//    to 8 columns of each block; a nibble n enters as the bf16 bit pattern of
//    128 + n (one and-or for two), which the block term corrects;
//  - A operand = the entries' activations as bf16 hi + lo (two products, exact
//    to about 2^-17), staged once per workgroup in LDS from the f32 rows,
//    together with the f32 block sums that the bias multiplies (the block
//    format's bias term runs once a window of 2 D blocks, block sums times
//    biases on the f32 matrix cores).
// Each wave owns kExpTiles tiles of 16 weight rows over all columns, with
// kExpDepth steps of weights in flight, requested kExpBurst at a time (a
// burst reads 256 contiguous bytes of each of its 16 rows, which HBM serves
// better than the same bytes spread over single steps); the block scales
// and biases arrive a window of steps at a time, spread over the four lanes
// of a row.  When the
// entries' staged rows exceed the LDS budget, the columns are taken in
// chunks, each staged between two barriers.
#include "expert_q8.h"
#include "pg_device.h"
#include "pg_host.h"


namespace pg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// What the scheduler may move across a step boundary (never memory loads,
// which keep their issue order).
constexpr int kExpSched = 0;
constexpr int kExpThreads = 512;
constexpr int kExpWaves = kExpThreads / kWave;
// Threads of a workgroup by format: q4tp's registers leave room for three
// waves a SIMD.
template <int FMT>
constexpr int exp_threads() { return FMT == 2 ? 768 : kExpThreads; }  // 2: kExpQ4
constexpr int kExpDepth = 16;
constexpr int kExpBurst = 4;   // ring slots refilled together
constexpr int kExpTiles = 1;                    // 16-row weight tiles per wave
constexpr int kExpGroup = 16;                // entries per pass over an item
constexpr int kExpLds = (148 * 1024);
constexpr int kExpMaxCnt = 64;
constexpr int kExpMaxExperts = 1024;

// LDS bytes of a chunk of `kp` block pairs for cnt entries in MT tiles of 16:
// hi and lo arrays of cnt + 1 rows (the last all zero) of 64 bytes a block
// plus 48 bytes of padding a row (of the 16-byte multiples tried, the one
// the q4tp bank runs fastest with), and the block sums [block][16 MT] f32.
__host__ __device__ constexpr int exp_chunk_bytes(int kp, int cnt, int mt) {
    return 2 * (cnt + 1) * (128 * kp + 48) + 2 * kp * 16 * mt * 4;
}

// Block pairs per chunk: the most that fit, a multiple of the ring depth D.
__device__ __forceinline__ int exp_chunk_pairs(int cnt, int mt, int d, int np) {
    const int per = 2 * (cnt + 1) * 128 + 2 * 16 * mt * 4;
    int kp = (kExpLds - 2 * 48 * (cnt + 1)) / per;
    kp -= kp % d;
    const int need = (np + d - 1) / d * d;
    return kp < need ? kp : need;
}
// One ring of steps must fit the LDS budget at the largest entry count.
static_assert(exp_chunk_bytes(kExpDepth, kExpGroup, kExpGroup / 16) <= kExpLds, "LDS budget");
static_assert(kExpLds + kExpMaxExperts * 4 + 16 <= 160 * 1024, "LDS of a compute unit");
static_assert(kExpDepth % kExpBurst == 0, "the ring refills in whole bursts");

constexpr int kExpNT = 0;      // q4tp weight loads: normal cache policy
constexpr int kExpNTPair = 2;  // q8 / q8_2f pair loads: non-temporal (each byte is used once)

// Bank formats (template argument FMT): the block format, q8_2f, and q4tp,
// whose nibble n enters the matrix cores as the exact bf16 128 + n while the
// - (128 + 8) rides in the per-block term: group scale times the block's sum
// of the staged activations times -136 (staged with them).
enum ExpFmt { kExpQ8 = 0, kExpQ82 = 1, kExpQ4 = 2 };

// (x & m) | c in one instruction (m a scalar, c a vector register).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
}

// Eight 4-bit codes (one dword, the low half of byte j is column 2j, the high
// half column 2j + 1) as a bf16x8 operand of the exact values 128 + n, in the
// column order 0 4 1 5 2 6 3 7 (dword j = columns j and j + 4).
__device__ __forceinline__ bf16x8 nib8_to_bf16_off(uint32_t w) {
    // 0x4300 | n is the bf16 of 128 + n (n < 128 fits the 7 fraction bits at 2^7)
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = and_or(w >> (4 * j), 0x000F000Fu, 0x43004300u);
    bf16x8 r;
    __builtin_memcpy(&r, p, 16);
    return r;
}

// A buffer resource over `bytes` bytes.  Every load below puts its whole
// offset in the per-lane (vector) offset, which the hardware checks against
// the resource's size (bytes past it read as zero); the scalar offset, which
// it does not check, stays 0.  So a row's last step or window, which may run
// past the row, never reads past the tensor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t exp_rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8 a, const bf16x8 b, const f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, const f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Eight int8 (two dwords, column order) as a bf16x8 operand; integers in
// [-128, 127] are exact in bf16.
__device__ __forceinline__ bf16x8 q8_to_bf16(uint32_t w0, uint32_t w1) {
    const uint32_t in[2] = {w0, w1};
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int v = (int)in[j];
        p[2 * j] = pack_bf16_exact((float)(int8_t)v, (float)(int8_t)(v >> 8));
        p[2 * j + 1] = pack_bf16_exact((float)(int8_t)(v >> 16), (float)(v >> 24));
    }
    bf16x8 r;
    __builtin_memcpy(&r, p, 16);
    return r;
}

// Stage blocks [cb0, cb0 + 2 kp) of the entries' rows (row cnt and blocks
// past the last are zeros).  Item = (row, quarter block of 8 columns); the 4
// quarters of a block sit on adjacent lanes, which add their sums with two
// exchanges into the block sum.  A thread requests kStageBatch items before
// it waits for any of them (the requests queue behind the weight stream).
constexpr int kStageBatch = 6;

// cf: the expert's binary16 column field (q8_2f), multiplied into the staged
// activations; NULL for the block format.
template <int MT, bool NIB, int NTH>
__device__ __forceinline__ void exp_stage(const ExpertBank &P, const int32_t *list, int cnt, int cb0,
                                          int kp, char *lds, const uint16_t *cf) {
    const int nb = P.cols >> 5;
    const int kc = 2 * kp;
    const int pitch = 64 * kc + 48;
    char *lo_base = lds + (cnt + 1) * pitch;
    float *xsum = reinterpret_cast<float *>(lds + 2 * (cnt + 1) * pitch);
    const int total = (cnt + 1) * 4 * kc;
    for (int base = 0; base < total; base += kStageBatch * NTH) {
        float4 xa[kStageBatch][2];
        u32x4 ca[kStageBatch];
#pragma unroll
        for (int k = 0; k < kStageBatch; ++k) {
            const int it = base + k * NTH + threadIdx.x;
            const int r = it / (4 * kc);
            const int qb = it - r * 4 * kc;
            const int blk = cb0 + (qb >> 2);
            xa[k][0] = xa[k][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            ca[k] = u32x4{0u, 0u, 0u, 0u};
            if (it < total && r < cnt && blk < nb) {
                const long long src = list[r] / P.src_div;
                const float4 *xp = reinterpret_cast<const float4 *>(P.x + src * P.ldx + 32 * blk + 8 * (qb & 3));
                xa[k][0] = xp[0];
                xa[k][1] = xp[1];
                if (cf) ca[k] = *reinterpret_cast<const u32x4 *>(cf + 32 * blk + 8 * (qb & 3));
            }
        }
#pragma unroll
        for (int k = 0; k < kStageBatch; ++k) {
            // Every requested item is consumed (stores only for items in range),
            // so no load of the batch is left pending past the staging.
            const int it = base + k * NTH + threadIdx.x;
            const bool in = it < total;
            const int r = it / (4 * kc);
            const int qb = it - r * 4 * kc;
            const int bl = qb >> 2, i = qb & 3;
            float v[8] = {xa[k][0].x, xa[k][0].y, xa[k][0].z, xa[k][0].w,
                          xa[k][1].x, xa[k][1].y, xa[k][1].z, xa[k][1].w};
            if (cf) {
                _Float16 c[8];
                __builtin_memcpy(c, &ca[k], 16);
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] *= (float)c[j];
            }
            if constexpr (NIB) {  // the nibble operand's column order 0 4 1 5 2 6 3 7
                const float t[8] = {v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = t[j];
            }
            __bf16 hi[8], lo[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                hi[j] = to_bf16(v[j]);
                lo[j] = to_bf16(v[j] - (float)hi[j]);
                if constexpr (NIB) v[j] = (float)hi[j] + (float)lo[j];  // the block sum of what the products see
            }
            u32x4 h4, l4;
            __builtin_memcpy(&h4, hi, 16);
            __builtin_memcpy(&l4, lo, 16);
            const int off = r * pitch + 64 * bl + 16 * i;
            if (in) {
                *reinterpret_cast<u32x4 *>(lds + off) = h4;
                *reinterpret_cast<u32x4 *>(lo_base + off) = l4;
            }
            float sum = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
            sum += __shfl_xor(sum, 1, kWave);
            sum += __shfl_xor(sum, 2, kWave);
            if constexpr (NIB) sum *= -136.0f;
            if (in && i == 0 && r < 16 * MT) xsum[bl * 16 * MT + r] = sum;
        }
    }
    // Block sums of the padding rows past the zero row.
    for (int it = threadIdx.x; it < kc * 16 * MT; it += NTH)
        if (it % (16 * MT) > cnt) xsum[it] = 0.0f;
}

// Load-side target: a work item's expert (its weight, scale and bias bases)
// and this lane's offsets in its row.  Past the last item: no memory moves.
struct ExpTgt {
    const int8_t *q;
    const float *s, *b;
    int vq[kExpTiles], vb[kExpTiles], vs[kExpTiles];  // vb: the second slot of a pair (8-bit formats)
    bool live;
    // q4tp: the expert's group codes and parameter words, and this lane's row
    const uint8_t *c;
    const uint32_t *pm;
    int row[kExpTiles];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// q4tp: the raw material of a window's group scales for one lane: the 8-byte
// code window holding the codes of its V blocks (moved back to end inside the
// code buffer), the row's parameter word, and the bit where its first code
// starts; kept as bits in the window registers until the window is taken.
template <int D>
__device__ __forceinline__ void q4_win_load(const ExpertBank &P, const ExpTgt &t, int w, int k, float (&dst)[D / 2]) {
    constexpr int V = D / 2;
    static_assert(5 * V + 7 <= 64 && V >= 5, "a window's codes fit one 8-byte code window");
    const int g = (threadIdx.x & 63) >> 4;
    if (!t.live) {
#pragma unroll
        for (int j = 0; j < V; ++j) dst[j] = 0.0f;
        return;
    }
    const uint32_t fbit = 5u * (uint32_t)(2 * D * w + V * g);
    const uint32_t total = (uint32_t)P.rows * (uint32_t)P.code_stride;
    const uint32_t absb = (uint32_t)t.row[k] * (uint32_t)P.code_stride + (fbit >> 3);
    const uint32_t at = min(absb, total - 8u);
    uint32_t win[2];
    __builtin_memcpy(win, t.c + at, 8);
    dst[0] = __builtin_bit_cast(float, win[0]);
    dst[1] = __builtin_bit_cast(float, win[1]);
    dst[2] = __builtin_bit_cast(float, t.pm[t.row[k]]);
    dst[3] = __builtin_bit_cast(float, 8u * (absb - at) + (fbit & 7u));
    dst[4] = __builtin_bit_cast(float, (uint32_t)(2 * D * w + V * g));  // first block of the share
}

// The group scales of a q4tp window (from q4_win_load's bits) and the block
// biases -8 * scale: scale_j = 2^(base + code_j step) (hardware exp2 of the
// f32 fma, as the q4tp GEMV).
// Blocks past the row's last (nb) get scale 0: their codes are not the row's.
template <int V>
__device__ __forceinline__ void q4_win_take(const float (&raw)[V], int nb, float (&sw)[V], float (&bw)[V]) {
    static_assert(V >= 5, "the window registers hold five words of raw material");
    const uint64_t win = (uint64_t)__builtin_bit_cast(uint32_t, raw[1]) << 32 | __builtin_bit_cast(uint32_t, raw[0]);
    const uint32_t pw = __builtin_bit_cast(uint32_t, raw[2]);
    const uint64_t wv = win >> (__builtin_bit_cast(uint32_t, raw[3]) & 63u);  // the first code at bit 0
    const int fb = (int)__builtin_bit_cast(uint32_t, raw[4]);
    const float base = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw & 0xFFFFu));
    const float step = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw >> 16));
#pragma unroll
    for (int j = 0; j < V; ++j) {
        // a valid block's code ends inside the window (sh + 5 j + 5 <= 64)
        const uint32_t code = (uint32_t)(wv >> (5 * j)) & 31u;
        sw[j] = fb + j < nb ? __builtin_amdgcn_exp2f(fmaf((float)code, step, base)) : 0.0f;
        bw[j] = sw[j];  // the staged block sums carry the -(128 + 8)
    }
}

// One pass over a work item (expert e, weight rows rb * R .., R = 16 rows a
// wave) for its entries m0 .. m0 + cnt - 1 (at most kExpGroup): its column
// chunks (staged when the expert or the entry group changes, or every time
// when the entries take more than one chunk), its steps, and its outputs.
// The weight ring and the scale windows come in holding this pass's first
// steps and leave holding those of the pass after it (target tn).
template <int MT, int D, int AL, int FMT>
__device__ __forceinline__ void exp_item(const ExpertBank &P, int e, int m0, int cnt, int rb, bool fresh,
                                         const ExpTgt &tc, const ExpTgt &tn, u32x4 (&wq)[D][kExpTiles],
                                         float (&sw)[kExpTiles][D / 2], float (&bw)[kExpTiles][D / 2],
                                         float (&swn)[kExpTiles][D / 2], float (&bwn)[kExpTiles][D / 2],
                                         char *lds) {
    constexpr bool Q82 = FMT == kExpQ82, Q4 = FMT == kExpQ4;
    constexpr int T = kExpTiles;
    constexpr int V = D / 2;             // blocks of a window per lane group
    constexpr int LW = AL < V ? AL : V;  // floats per scale / bias load
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g = lane >> 4;
    const int nb = P.cols >> 5;
    const int np = (nb + 1) >> 1;
    const int npp = (np + D - 1) / D * D;
    const int q_bytes = Q4 ? P.rows * (P.cols >> 1) : P.rows * P.cols;
    const int s_bytes = (Q82 || Q4) ? 0 : P.rows * nb * 4;  // q8_2f: no block factors, the windows move nothing
    const int32_t *list = P.lists + (long long)e * P.cap + m0;
    const int kp = exp_chunk_pairs(cnt, MT, D, np);
    const bool chunked = kp < npp;
    const int pitch = 128 * kp + 48;
    const int lo_off = (cnt + 1) * pitch;
    const int xs_off = 2 * (cnt + 1) * pitch;

    // Output rows of this lane's results (entry 16 mt + 4 g + v), requested
    // now so that their wait at the end does not queue behind the next pass.
    int orow[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 16 * mt + 4 * g + v;
            orow[mt][v] = m < cnt ? list[m] : -1;
        }

    // The ring slots of a step pair (p even).  q4tp: one slot, 16 bytes a lane
    // (block 2 p + g of the lane's row).  The 8-bit formats: two slots, each one
    // instruction over 8 rows x 128 bytes (both steps of rows 0-7, then of rows
    // 8-15), the pattern HBM serves best: lane (g, i) reads piece g of row i % 8
    // for step i / 8 in the first, of row 8 + i % 8 for step 1 - i / 8 in the
    // second, so that a step's operand is a lane-wise select of the two.
    auto load = [&](const ExpTgt &t, int p, u32x4 (&wa)[T], u32x4 (&wb)[T]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rq = exp_rsrc(t.q, t.live && p < np ? q_bytes : 0);
#pragma unroll
        for (int k = 0; k < T; ++k) {
            if constexpr (Q4) {
                wa[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, t.vq[k] + 32 * p, 0, kExpNT);
            } else {
                wa[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, t.vq[k] + 64 * p, 0, kExpNTPair);
                wb[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, t.vb[k] + 64 * p, 0, kExpNTPair);
            }
        }
    };
    // Scales and biases come a window of D steps (2D blocks) at a time: lane
    // group g holds blocks V g .. V g + V - 1 of the window for its row; a
    // step takes its two blocks' scales from the group that holds them (a lane
    // permute), so that the four lanes of a row do not each load them, and the
    // biases serve the window's bias term where they lie.
    auto load_win = [&](const ExpTgt &t, int w) __attribute__((always_inline)) {
        if constexpr (Q4) {
#pragma unroll
            for (int k = 0; k < T; ++k) q4_win_load<D>(P, t, w, k, swn[k]);
            return;
        }
        const __amdgpu_buffer_rsrc_t rs = exp_rsrc(t.s, t.live ? s_bytes : 0);
        const __amdgpu_buffer_rsrc_t rbs = exp_rsrc(t.b, t.live ? s_bytes : 0);
        const int off = 8 * D * w;
#pragma unroll
        for (int k = 0; k < T; ++k)
#pragma unroll
            for (int j = 0; j < V; j += LW) {
                if (LW == 4) {
                    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, t.vs[k] + off + 4 * j, 0, 0));
                    const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbs, t.vs[k] + off + 4 * j, 0, 0));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        swn[k][j + i] = a[i];
                        bwn[k][j + i] = b[i];
                    }
                } else if (LW == 2) {
                    const f32x2 a = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, t.vs[k] + off + 4 * j, 0, 0));
                    const f32x2 b = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rbs, t.vs[k] + off + 4 * j, 0, 0));
                    swn[k][j] = a[0];
                    swn[k][j + 1] = a[1];
                    bwn[k][j] = b[0];
                    bwn[k][j + 1] = b[1];
                } else {
                    swn[k][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, t.vs[k] + off + 4 * j, 0, 0));
                    bwn[k][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbs, t.vs[k] + off + 4 * j, 0, 0));
                }
            }
    };

    // acc: the even steps; acc1: the odd steps of the 8-bit formats, whose
    // column n is row n ^ 8.
    f32x4 acc[T][MT], acc1[T][MT];
#pragma unroll
    for (int k = 0; k < T; ++k)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[k][mt] = acc1[k][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // A operand of lane (i16, g): entry 16 mt + i16 (the zero row past cnt),
    // columns 16 (g & 1) + 8 (g >> 1) .. + 7 of the block, matching the
    // weight columns this lane group holds after the exchange.
    const int a_col = Q4 ? 16 * g : 2 * (16 * (g & 1) + 8 * (g >> 1));
    int a_row[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + i16;
        a_row[mt] = (m < cnt ? m : cnt) * pitch + a_col;
    }

    // Step u of a window: blocks 2u, 2u + 1 sit in lane group 2u / V at
    // entries 2u % V and 2u % V + 1.
    auto compute = [&](auto uc, int p, int cb0, u32x4 (&w)[T], const u32x4 (&w2)[T]) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr int gs = 2 * u / V, ev = 2 * u % V;
        constexpr bool ODD = !Q4 && (u & 1);  // this step's column n holds row n ^ 8
        const int src = ((ODD ? i16 ^ 8 : i16) + 16 * gs) * 4;
        const int bl = 2 * p - cb0;
        f32x2 s[T];
        bf16x8 b0[T], b1[T];
#pragma unroll
        for (int k = 0; k < T; ++k) {
            s[k].x = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sw[k][ev])));
            s[k].y = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sw[k][ev + 1])));
            // Lanes 0-31 hold block 2p, lanes 32-63 block 2p + 1; after the
            // exchange operand 0 carries block 2p on every lane, operand 1 block 2p + 1.
            if constexpr (Q4) {
                // The slot of a step pair holds block 4P + g in lane group g
                // (dword j: its columns 8 j .. 8 j + 7); the even step
                // transposes it in place (lane-half swaps, then row swaps) to
                // dword j = block 4P + j, columns 8 g .. 8 g + 7.
                if constexpr (u % 2 == 0) {
                    const auto h0 = __builtin_amdgcn_permlane32_swap(w[k].x, w[k].z, false, false);
                    const auto h1 = __builtin_amdgcn_permlane32_swap(w[k].y, w[k].w, false, false);
                    const auto r0 = __builtin_amdgcn_permlane16_swap(h0[0], h1[0], false, false);
                    const auto r1 = __builtin_amdgcn_permlane16_swap(h0[1], h1[1], false, false);
                    w[k] = u32x4{r0[0], r0[1], r1[0], r1[1]};
                }
                b0[k] = nib8_to_bf16_off(u % 2 ? w[k].z : w[k].x);
                b1[k] = nib8_to_bf16_off(u % 2 ? w[k].w : w[k].y);
            } else {
                // The pair's slots: w holds rows 0-7 (lane (g, i): piece g of row
                // i % 8 for step i / 8), w2 rows 8-15 the other way round (step
                // 1 - i / 8).  Step 0 takes w's first half-rows and w2's second
                // (column n = row n); step 1 w2's first and w's second (column
                // n = row n ^ 8).
                auto pick = [&](uint32_t a, uint32_t b) __attribute__((always_inline)) {
                    return (i16 < 8) != ODD ? a : b;
                };
                const u32x4 q{pick(w[k].x, w2[k].x), pick(w[k].y, w2[k].y), pick(w[k].z, w2[k].z), pick(w[k].w, w2[k].w)};
                const auto e0 = __builtin_amdgcn_permlane32_swap(q.x, q.z, false, false);
                const auto e1 = __builtin_amdgcn_permlane32_swap(q.y, q.w, false, false);
                b0[k] = q8_to_bf16(e0[0], e1[0]);
                b1[k] = q8_to_bf16(e0[1], e1[1]);
            }
        }
        const f32x4 z{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const char *a = lds + a_row[mt] + 64 * bl;
            const bf16x8 ah0 = as_bf16x8(*reinterpret_cast<const u32x4 *>(a));
            const bf16x8 ah1 = as_bf16x8(*reinterpret_cast<const u32x4 *>(a + 64));
            const bf16x8 al0 = as_bf16x8(*reinterpret_cast<const u32x4 *>(a + lo_off));
            const bf16x8 al1 = as_bf16x8(*reinterpret_cast<const u32x4 *>(a + lo_off + 64));
            const float *xs = reinterpret_cast<const float *>(lds + xs_off) + bl * 16 * MT + 16 * mt + 4 * g;
            const f32x4 xs0 = *reinterpret_cast<const f32x4 *>(xs);
            const f32x4 xs1 = *reinterpret_cast<const f32x4 *>(xs + 16 * MT);
#pragma unroll
            for (int k = 0; k < T; ++k) {
                if constexpr (Q82) {  // no block factors: one chain through the accumulator
                    f32x4 &A = ODD ? acc1[k][mt] : acc[k][mt];
                    A = mfma16(ah0, b0[k], A);
                    A = mfma16(al0, b0[k], A);
                    A = mfma16(ah1, b1[k], A);
                    A = mfma16(al1, b1[k], A);
                    continue;
                }
                // q4tp: the chains start from the staged block sums (times -136)
                f32x4 d0 = mfma16(ah0, b0[k], Q4 ? xs0 : z);
                d0 = mfma16(al0, b0[k], d0);
                f32x4 d1 = mfma16(ah1, b1[k], Q4 ? xs1 : z);
                d1 = mfma16(al1, b1[k], d1);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float x = ODD ? acc1[k][mt][v] : acc[k][mt][v];
                    x = fmaf(s[k].x, d0[v], x);
                    x = fmaf(s[k].y, d1[v], x);
                    if constexpr (ODD) acc1[k][mt][v] = x;
                    else acc[k][mt][v] = x;
                }
            }
        }
    };

    // Every window issues the same loads in the same order (window w + 1 at
    // the start of window w, then one weight step per step), so the wait for
    // a step's data is always the same count.  The last window of the pass
    // requests the next pass's first window and steps.
    for (int c0 = 0; c0 < npp; c0 += kp) {
        if (c0 > 0 || chunked || fresh) {
            __syncthreads();
            exp_stage<MT, Q4, exp_threads<FMT>()>(P, list, cnt, 2 * c0, kp, lds, Q82 ? P.cf + (long long)e * P.cf_stride : nullptr);
            __syncthreads();
        }
        const int c1 = min(npp, c0 + kp);
        for (int p0 = c0; p0 < c1; p0 += D) {
#pragma unroll
            for (int k = 0; k < T; ++k) {
                if constexpr (Q4) {
                    q4_win_take<V>(swn[k], nb, sw[k], bw[k]);
                } else {
#pragma unroll
                    for (int j = 0; j < V; ++j) {
                        sw[k][j] = swn[k][j];
                        bw[k][j] = bwn[k][j];
                    }
                }
            }
            if constexpr (!Q4 && !Q82) {
                // The window's bias term, sum over its 2 D blocks of bias x block
                // sum, on the f32 matrix cores: lane group g holds the biases of
                // blocks V g .. V g + V - 1 of its row (the B operand as loaded)
                // and reads the matching block sums of entry 16 mt + i16.
                const float *xw = reinterpret_cast<const float *>(lds + xs_off) + (2 * (p0 - c0) + V * g) * 16 * MT + i16;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    float a[V];
#pragma unroll
                    for (int j = 0; j < V; ++j) a[j] = xw[j * 16 * MT + 16 * mt];
#pragma unroll
                    for (int k = 0; k < T; ++k)
#pragma unroll
                        for (int j = 0; j < V; ++j) acc[k][mt] = mfma16_f32(a[j], bw[k][j], acc[k][mt]);
                }
            }
            const bool last = p0 + D >= npp;
            const ExpTgt &tl = last ? tn : tc;
            const int pl = last ? p0 + D - npp : p0 + D;
            load_win(tl, pl / D);
            __builtin_amdgcn_sched_barrier(kExpSched);
            static_for<D>([&](auto uc) __attribute__((always_inline)) {
                constexpr int u = decltype(uc)::value;
                const int p = p0 + u;
                if (p < np) compute(uc, p, 2 * c0, wq[u & ~1], wq[(u & ~1) + (Q4 ? 0 : 1)]);
                // after the last step of a burst, its slots are refilled together
                if constexpr (u % kExpBurst == kExpBurst - 1) {
#pragma unroll
                    for (int j = u + 1 - kExpBurst; j <= u; j += 2) load(tl, pl + j, wq[j], wq[j + 1]);
                }
                __builtin_amdgcn_sched_barrier(kExpSched);
            });
        }
    }

    if constexpr (!Q4) {  // the odd steps' sums: column n held row n ^ 8 (all lanes take part)
#pragma unroll
        for (int k = 0; k < T; ++k)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float o = acc1[k][mt][v];  // a copy: bit_cast of a vector element read element 0
                    acc[k][mt][v] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, o), 0x128, 0xF, 0xF, false));
                }
    }
    // Output element v of tile (k, mt): entry 16 mt + 4 g + v, weight row
    // rb * R + (wave T + k) * 16 + i16.
#pragma unroll
    for (int k = 0; k < T; ++k) {
        const int r = rb * (exp_threads<FMT>() / 4) + (wave * T + k) * 16 + i16;
        if (r >= P.rows) continue;
        // q8_2f: the row scale multiplies the finished sum.
        const float rsc = Q82 ? (float)__builtin_bit_cast(_Float16, P.rs[(long long)e * P.rs_stride + r]) : 1.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (orow[mt][v] >= 0)
                    P.out[(long long)orow[mt][v] * P.ldo + r] = apply_act(P.act, Q82 ? acc[k][mt][v] * rsc : acc[k][mt][v]);
    }
}

// Persistent workgroups, one per compute unit (8 waves; 12 for q4tp).  The
// work items are (active expert, block of 16 rows a wave), experts in
// ascending order; each workgroup takes one contiguous share, so that it
// stages an expert's entries once for all of that expert's items in its
// share, and its weight stream runs from one item into the next without
// draining.  An expert with more than kExpGroup entries takes one pass per
// group of kExpGroup over each item.
// Ring depth of a format (the same for all: q4tp's scale window reads the
// codes of its 2 D blocks from one 8-byte window).
template <int FMT>
constexpr int exp_depth() { return kExpDepth; }

template <int AL, int FMT>
__global__ __launch_bounds__(exp_threads<FMT>(), 1) void expert_bank_kernel(ExpertBank P) {
    constexpr bool Q82 = FMT == kExpQ82, Q4 = FMT == kExpQ4;
    extern __shared__ u32x4 exp_lds[];
    __shared__ int act[kExpMaxExperts];
    __shared__ int nact_s;
    constexpr int D = exp_depth<FMT>(), T = kExpTiles, V = D / 2;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g = lane >> 4;
    char *lds = reinterpret_cast<char *>(exp_lds);

    // Active experts (at least one entry), ascending.
    if (wave == 0) {
        int base = 0;
        for (int e0 = 0; e0 < P.experts; e0 += 64) {
            const int e = e0 + lane;
            const bool on = e < P.experts && P.counts[e] > 0;
            const unsigned long long m = __ballot(on);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (on) act[base + below] = e;
            base += __popcll(m);
        }
        if (lane == 0) nact_s = base;
    }
    __syncthreads();
    constexpr int kRows = exp_threads<FMT>() / 4 * kExpTiles;  // weight rows of one work item
    const int RB = (P.rows + kRows - 1) / kRows;
    const long long N = (long long)nact_s * RB;
    const int i0 = (int)(N * blockIdx.x / gridDim.x);
    const int i1 = (int)(N * (blockIdx.x + 1) / gridDim.x);
    if (i0 >= i1) return;

    const int nb = P.cols >> 5;
    auto target = [&](int item) __attribute__((always_inline)) {
        ExpTgt t;
        t.live = item < i1;
        const int it = t.live ? item : i1 - 1;
        const int e = __builtin_amdgcn_readfirstlane(act[it / RB]);
        const int rb = it % RB;
        if (Q4) {
            t.q = reinterpret_cast<const int8_t *>(P.nib + (long long)e * P.rows * (P.cols >> 1));
            t.c = P.codes + (long long)e * P.rows * P.code_stride;
            t.pm = P.params + (long long)e * P.rows;
        } else {
            t.q = P.q + (long long)e * P.q_stride;
        }
        t.s = P.scale + (long long)e * P.s_stride;
        t.b = P.bias + (long long)e * P.s_stride;
#pragma unroll
        for (int k = 0; k < T; ++k) {
            const int r = min(rb * kRows + (wave * T + k) * 16 + i16, P.rows - 1);
            const int r8 = rb * kRows + (wave * T + k) * 16 + (i16 & 7);
            t.vq[k] = Q4 ? r * (P.cols >> 1) + 16 * g : min(r8, P.rows - 1) * P.cols + 64 * (i16 >> 3) + 16 * g;
            t.vb[k] = Q4 ? 0 : min(r8 + 8, P.rows - 1) * P.cols + 64 * (1 - (i16 >> 3)) + 16 * g;
            t.vs[k] = (r * nb + V * g) * 4;
            t.row[k] = r;
        }
        return t;
    };
    auto count = [&](int e) __attribute__((always_inline)) { return min(P.counts[e], min(P.cap, kExpMaxCnt)); };

    // The ring and the windows start out holding the first item's window 0
    // and steps 0 .. D - 1 (loaded in step order).
    u32x4 wq[D][T];
    float sw[T][V], bw[T][V], swn[T][V], bwn[T][V];
    {
        const ExpTgt t0 = target(i0);
        if constexpr (Q4) {
#pragma unroll
            for (int k = 0; k < T; ++k) {
                q4_win_load<D>(P, t0, 0, k, swn[k]);
#pragma unroll
                for (int j = 0; j < V; ++j) bwn[k][j] = 0.0f;
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs = exp_rsrc(t0.s, Q82 ? 0 : P.rows * nb * 4);
            const __amdgpu_buffer_rsrc_t rbs = exp_rsrc(t0.b, Q82 ? 0 : P.rows * nb * 4);
#pragma unroll
            for (int k = 0; k < T; ++k)
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    swn[k][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, t0.vs[k] + 4 * j, 0, 0));
                    bwn[k][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbs, t0.vs[k] + 4 * j, 0, 0));
                }
        }
        __builtin_amdgcn_sched_barrier(kExpSched);
        const int np = (nb + 1) >> 1;
        static_for<D>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
#pragma unroll
            for (int k = 0; k < T; ++k) {
                if constexpr (Q4) {
                    if constexpr (u % 2 == 0) {
                        const __amdgpu_buffer_rsrc_t r = exp_rsrc(t0.q, u < np ? P.rows * (P.cols >> 1) : 0);
                        wq[u][k] = __builtin_amdgcn_raw_buffer_load_b128(r, t0.vq[k] + 32 * u, 0, kExpNT);
                    }
                } else if constexpr (u % 2 == 0) {
                    const __amdgpu_buffer_rsrc_t r = exp_rsrc(t0.q, u < np ? P.rows * P.cols : 0);
                    wq[u][k] = __builtin_amdgcn_raw_buffer_load_b128(r, t0.vq[k] + 64 * u, 0, kExpNTPair);
                    wq[u + 1][k] = __builtin_amdgcn_raw_buffer_load_b128(r, t0.vb[k] + 64 * u, 0, kExpNTPair);
                }
            }
            __builtin_amdgcn_sched_barrier(kExpSched);
        });
    }

    int prev = -1;
    for (int item = i0; item < i1; ++item) {
        const int e = __builtin_amdgcn_readfirstlane(act[item / RB]);
        const int rb = item % RB;
        const int cnt = count(e);
        const ExpTgt tc = target(item), tn = target(item + 1);
        const int groups = (cnt + kExpGroup - 1) / kExpGroup;
        for (int gi = 0; gi < groups; ++gi) {
            const int m0 = gi * kExpGroup;
            const int cg = min(kExpGroup, cnt - m0);
            const bool fresh = e != prev || groups > 1;
            const ExpTgt &nx = gi + 1 < groups ? tc : tn;
            if (kExpGroup <= 16 || cg <= 16)
                exp_item<1, D, AL, FMT>(P, e, m0, cg, rb, fresh, tc, nx, wq, sw, bw, swn, bwn, lds);
            else
                exp_item<2, D, AL, FMT>(P, e, m0, cg, rb, fresh, tc, nx, wq, sw, bw, swn, bwn, lds);
        }
        prev = e;
    }
}

static int exp_grid() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

template <int AL, int FMT = kExpQ8>
static int launch_bank(const ExpertBank &P, hipStream_t s) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(expert_bank_kernel<AL, FMT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kExpLds);
    if (attr != hipSuccess) return PG_ELAUNCH;
    hipLaunchKernelGGL((expert_bank_kernel<AL, FMT>), dim3(exp_grid()), dim3(exp_threads<FMT>()), kExpLds, s, P);
    return launch_status();
}

int launch_expert_bank(const ExpertBank &P, hipStream_t s) {
    if (P.rows < 1 || P.cols < 32 || P.cols % 32 || P.cap > kExpMaxCnt) return PG_EUNSUPPORTED;
    if (P.experts < 1 || P.experts > kExpMaxExperts) return PG_EUNSUPPORTED;
    if ((long long)P.rows * P.cols >= (1ll << 31)) return PG_EUNSUPPORTED;  // 32-bit buffer offsets
    const int nb = P.cols / 32;
    if (P.nib) {  // q4tp: code windows instead of scale loads
        if (!P.params || !P.codes || (long long)P.rows * P.code_stride < 8) return PG_EINVAL;
        return launch_bank<1, kExpQ4>(P, s);
    }
    if (P.rs) {  // q8_2f: the (empty) window loads take the widest form the block count allows
        if (!P.cf) return PG_EINVAL;
        return nb % 4 == 0 ? launch_bank<4, kExpQ82>(P, s) : nb % 2 == 0 ? launch_bank<2, kExpQ82>(P, s)
                                                                          : launch_bank<1, kExpQ82>(P, s);
    }
    // Widest scale / bias loads: a row's blocks must start on that boundary.
    const uintptr_t a = (uintptr_t)P.scale | (uintptr_t)P.bias;
    if (nb % 4 == 0 && (a & 15) == 0) return launch_bank<4>(P, s);
    if (nb % 2 == 0 && (a & 7) == 0) return launch_bank<2>(P, s);
    if ((a & 3) == 0) return launch_bank<1>(P, s);
    return PG_EINVAL;
}

}  // namespace pg

using namespace pg;

// The q8_2f expert bank over a pass (nemotron_prefill.rs, the q8_2f bank
// payload: int8 body, f16 row scales, f16 column field per expert).
extern "C" int expert_bank_q82(const int8_t *q, const uint16_t *row_scale, const uint16_t *col_field, int32_t E,
                               int32_t rows, int32_t cols, const float *x, int64_t ldx, int32_t src_div,
                               const int32_t *counts, const int32_t *lists, int32_t cap, float *out, int64_t ldo,
                               int32_t act, pg_stream_t stream) {
    if (!q || !row_scale || !col_field || !x || !counts || !lists || !out) return PG_EINVAL;
    if (E <= 0 || rows <= 0 || cols <= 0 || cap <= 0 || src_div <= 0 || ldx < cols || ldo < rows) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (!aligned16(q) || !aligned16(x) || !aligned16(col_field) || ldx % 4 || ((uintptr_t)row_scale & 1))
        return PG_EINVAL;
    ExpertBank P{};
    P.q = q;
    P.rows = rows;
    P.cols = cols;
    P.q_stride = (long long)rows * cols;
    P.x = x;
    P.ldx = ldx;
    P.src_div = src_div;
    P.counts = counts;
    P.lists = lists;
    P.cap = cap;
    P.experts = E;
    P.out = out;
    P.ldo = ldo;
    P.act = act;
    P.rs = row_scale;
    P.cf = col_field;
    P.rs_stride = rows;
    P.cf_stride = cols;
    return launch_expert_bank(P, as_stream(stream));
}

// The q4tp expert bank over a pass (nemotron_prefill.rs, `pb_q4_bank` and its
// nibble and code readers: 4-bit codes, a binary16 base and step per row, a
// 5-bit code per 32-column group; w = 2^(base + code step) (nib - 8)), each
// selected expert's weights streamed once for all of its entries.
extern "C" int expert_bank_q4tp(const uint8_t *nib, const uint32_t *params, const uint8_t *codes, int32_t E,
                                int32_t rows, int32_t cols, const float *x, int64_t ldx, int32_t src_div,
                                const int32_t *counts, const int32_t *lists, int32_t cap, float *out, int64_t ldo,
                                int32_t act, pg_stream_t stream) {
    if (!nib || !params || !codes || !x || !counts || !lists || !out) return PG_EINVAL;
    if (E <= 0 || rows <= 0 || cols <= 0 || cap <= 0 || src_div <= 0 || ldx < cols || ldo < rows) return PG_EINVAL;
    if (act != 0 && act != 1) return PG_EINVAL;
    if (cols % 32) return PG_EUNSUPPORTED;
    if (!aligned16(nib) || !aligned16(x) || ldx % 4 || ((uintptr_t)params & 3)) return PG_EINVAL;
    ExpertBank P{};
    P.rows = rows;
    P.cols = cols;
    P.x = x;
    P.ldx = ldx;
    P.src_div = src_div;
    P.counts = counts;
    P.lists = lists;
    P.cap = cap;
    P.experts = E;
    P.out = out;
    P.ldo = ldo;
    P.act = act;
    P.nib = nib;
    P.params = params;
    P.codes = codes;
    P.code_stride = (5 * (cols / 32) + 7) / 8;
    if ((long long)rows * P.code_stride < 8) return PG_EUNSUPPORTED;  // 8-byte code windows
    return launch_expert_bank(P, as_stream(stream));
}
