#pragma once

#include <hip/hip_runtime.h>

#include "nets.hpp"

namespace rl {

// Repack the caller's [out, in] fp32 weights into `block` (packed_offsets()
// layout).  Enqueued on `st`; the sources must stay valid until it runs.
hipError_t pack_weights(const float* const actor[6], const float* const critic[12],
                        const float* const cur[4], float* block, hipStream_t st);

}  // namespace rl
