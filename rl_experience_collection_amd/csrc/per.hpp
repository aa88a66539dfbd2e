// Host-side interface of the prioritized-replay kernels (see per.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace rl {

constexpr int kPerBlock = 2048;  // priorities per block of the two-level prefix sums

inline int64_t per_blocks(int64_t n) { return (n + kPerBlock - 1) / kPerBlock; }

struct PerGatherArgs {
  const int32_t* indices;
  int32_t batch;
  int64_t n;
  const float* states;       // [n][54] or null
  const float* next_states;  // [n][54] or null
  const int32_t* actions;    // [n] or null
  const float* rewards;      // [n] or null
  const uint8_t* dones;      // [n] or null
  float* out_states;         // [batch][54]
  float* out_next_states;    // [batch][54]
  int32_t* out_actions;      // [batch]
  float* out_rewards;        // [batch]
  uint8_t* out_dones;        // [batch]
};

// Scratch: block_prefix per_blocks(n) doubles, lane_prefix 64 * per_blocks(n)
// doubles, raw_weights batch doubles.
hipError_t per_sample_launch(const float* priorities, int64_t n, int32_t batch, uint64_t seed,
                             float beta, int32_t* indices, float* weights, double* block_prefix,
                             double* lane_prefix, double* raw_weights, hipStream_t st);
hipError_t per_gather_launch(const PerGatherArgs& a, hipStream_t st);
hipError_t per_update_launch(float* priorities, int64_t n, const int32_t* indices, const float* td,
                             int32_t batch, float alpha, float eps, float pmax, hipStream_t st);

}  // namespace rl
