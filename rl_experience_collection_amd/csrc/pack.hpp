#pragma once

#include <hip/hip_runtime.h>

#include "nets.hpp"

namespace rl {

// Repack the caller's [out, in] fp32 weights into `block` (packed_offsets()
// layout).  Enqueued on `st`; the sources must stay valid until it runs.
hipError_t pack_weights(const float* const actor[6], const float* const critic[12],
                        const float* const cur[4], float* block, hipStream_t st);

// Repack the DQN collection's networks into `block` (dqn_packed_offsets()
// layout): online[12] and target[12] = trunk 1, trunk 2, value 1, value 2,
// advantage 1, advantage 2 (weight [out, in], then bias); cur[4] as for
// pack_weights.  A NULL online, target or cur keeps that part of the block.
// `scratch` holds dqn_pack_scratch_floats() floats of device memory for the
// assembled head layers; it must stay allocated until the packing has run.
size_t dqn_pack_scratch_floats();
hipError_t pack_dqn_weights(const float* const online[12], const float* const target[12],
                            const float* const cur[4], float* block, float* scratch,
                            hipStream_t st);

}  // namespace rl
