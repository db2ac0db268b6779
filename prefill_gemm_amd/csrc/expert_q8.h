// Grouped expert bank launcher (defined in expert_q8.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pg {

// One bank of q8 experts [E][rows][cols] applied to the entries each expert
// was chosen for: out[j][r] for j in lists[e][0 .. counts[e]), reading the
// activation row x[j / src_div] (ldx floats apart).  Rows of `out` are ldo
// floats apart; act = 1 applies relu^2.
struct ExpertBank {
    const int8_t *q;
    const float *scale;
    const float *bias;
    int rows, cols;
    long long q_stride;  // int8 elements from one expert to the next
    long long s_stride;  // scale / bias elements from one expert to the next
    const float *x;
    long long ldx;
    int src_div;
    const int32_t *counts;
    const int32_t *lists;  // [E][cap]
    int cap;               // at most 64
    int experts;
    float *out;
    long long ldo;
    int act;
    // q8_2f banks (scale / bias unused): binary16 row scales [E][rows] and
    // column fields [E][cols], rs_stride / cf_stride elements apart; NULL: q8 block.
    const uint16_t *rs;
    const uint16_t *cf;
    long long rs_stride, cf_stride;
    // q4tp banks (q, scale, bias unused): nibbles [E][rows][cols/2], parameter
    // words [E][rows] (binary16 base low, step high), 5-bit group codes
    // [E][rows][code_stride]; NULL nib: not q4tp.
    const uint8_t *nib;
    const uint32_t *params;
    const uint8_t *codes;
    int code_stride;
};

// Experts [0, experts); those with no entries are skipped.
int launch_expert_bank(const ExpertBank &P, hipStream_t s);

}  // namespace pg
