// Host-side helpers shared by the libpg entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pg.h"

namespace pg {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline hipStream_t as_stream(pg_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the launch just issued.
inline int launch_status() { return hipGetLastError() == hipSuccess ? PG_OK : PG_ELAUNCH; }

constexpr size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Byte sizes of the matrix-core staging of `rows` activation rows of `cols`
// columns (plus one all-zero padding row); see mma_q8.h for the layout.
inline size_t stage_x_bytes(int rows, int cols) { return (size_t)(rows + 1) * (size_t)cols * 4; }
inline size_t stage_s_bytes(int rows, int cols) {
    const int nb = cols / 32, ng = (nb + 15) / 16;
    return (size_t)(rows + 1) * (size_t)ng * 64;
}

// Launch helpers (defined in mma_q8.hip): stage rows of X for the matrix cores.
int launch_stage_x(const float *X, int rows, int cols, void *xp, void *xs, hipStream_t s);

}  // namespace pg
