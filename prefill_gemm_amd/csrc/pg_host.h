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

// Number of K splits the dense pass uses for a rows x cols weight (mma_q8.hip).
int dense_splits(int rows, int cols);

}  // namespace pg
