// Host launchers of the matrix-core kernels (defined in mma_q8.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "mma_q8.h"

namespace pg {

// Grouped expert bank over experts [0, experts): grid (panels, experts).
int launch_expert_bank(const MmaPanel &P, int experts, const int32_t *counts,
                       const int32_t *lists, int cap, hipStream_t s);

// Number of K splits the dense pass uses for a rows x cols weight.
int dense_splits(int rows, int cols);

}  // namespace pg
