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

// Whether the byte ranges [a, a + an) and [b, b + bn) share a byte (null: no).
inline bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!a || !b) return false;
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x < y + bn && y < x + an;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Whether any two of the ranges (pointer, bytes) share a byte.
struct Span {
    const void *p;
    size_t bytes;
};
template <size_t N>
inline bool any_overlap(const Span (&sp)[N]) {
    for (size_t i = 0; i < N; ++i)
        for (size_t j = i + 1; j < N; ++j)
            if (overlaps(sp[i].p, sp[i].bytes, sp[j].p, sp[j].bytes)) return true;
    return false;
}

// Number of K splits the dense pass uses for a rows x cols weight (mma_q8.hip).
int dense_splits(int rows, int cols);

}  // namespace pg
