// Arguments and launchers of the two collection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nets.hpp"

namespace rl {

// Sequential part: state assembly, actor, draw, portfolio / barrier /
// diversity, partial reward (everything a later step depends on).
struct RolloutArgs {
  const float* weights;   // packed block (packed_offsets layout)
  const float* features;  // [n_bars][51]
  const float* prices;    // [n_bars]
  int64_t n_bars;
  const int32_t* starts;  // [N]
  uint64_t seed;
  int32_t N, L;
  EnvParams ep;
  int32_t* start_used;    // [N] clamped starts (read back by the value kernel)
  float* states;          // [L][N][54]
  int32_t* actions;       // [L][N]
  float* log_probs;       // [L][N]
  float* rewards;         // [L][N] partial: pnl (1 + scale hit) + diversity
  uint8_t* dones;         // [L][N]
  uint8_t* barrier;       // [L][N]
  float* logits;          // [L][N][45] or null
  uint32_t* counters;     // [2] or null
  int bf16;               // bf16 weights and layer inputs, fp32 accumulation
  int32_t* bars;          // [L][N] bar of every step, or null: non-null selects recycling
  int32_t t_begin, t_end; // the steps of this launch: [0, L) for the whole rollout
  int32_t* carry;         // [N][kCarryWords] episode state between launches, or null
  // [blocks * kSplit][kStampWords] per-wave cycle totals (instrumented
  // kernel), or null: the plain kernel
  uint64_t* stamps;
  // [L][N][kActorOut1] first-layer feature part of every step (written by
  // launch_feature_table; never with recycling), or null: computed in the
  // step
  const float* ftable;
};

// Cycle totals of one wave of the instrumented step kernel: kStampPhases
// phases of every step, then the steps counted and the whole loop's cycles.
constexpr int kStampWords = 16;
constexpr int kStampPhases = 11;

// Episode state a launch that ends before step L leaves for the next one:
// bar (2 words), V, exposure held, entry price, armed, side, open step,
// the three window counts, pushes, slot, window ring (2 words).
constexpr int kCarryWords = 16;

// Batched part: critic value and curiosity bonus of every stored (t, n),
// which no later step reads, then the final reward.
struct ValueArgs {
  const float* weights;
  const float* features;
  const float* states;
  const int32_t* actions;
  const int32_t* start_used;
  const int32_t* bars;    // [L][N] bar of every step (recycling), or null: start_used + t
  int32_t N, L;
  EnvParams ep;
  float* values;
  float* rewards;  // in: partial reward, out: full reward
  uint32_t* counters;
  unsigned long long* sched;  // [1] work counter of the persistent grid (zeroed per launch)
  int bf16;
  int32_t t_off;  // global step of row 0 (a launch over the steps from t_off on)
  int32_t max_grid;  // > 0: at most this many workgroups
  int32_t lds_pad;   // extra LDS bytes reserved per workgroup (placement only)
};

// DQN collection: every step of every episode in one sequential kernel.
struct DqnArgs {
  const float* weights;   // packed block (dqn_packed_offsets layout)
  const float* features;  // [n_bars][51]
  const float* prices;    // [n_bars]
  int64_t n_bars;
  const int32_t* starts;  // [N]
  uint64_t seed;
  int32_t N, L;
  EnvParams ep;
  float epsilon, gamma, alpha;
  int recycle;            // restart an ended episode at a fresh random bar
  float* states;          // [L][N][54]
  float* next_states;     // [L][N][54] or null
  float* q_values;        // [L][N][45] or null
  int32_t* actions;       // [L][N]
  uint8_t* explored;      // [L][N] or null
  float* q_taken;         // [L][N]
  float* q_next_max;      // [L][N]
  float* rewards;         // [L][N]
  uint8_t* dones;         // [L][N]
  uint8_t* barrier;       // [L][N]
  float* td;              // [L][N]
  float* priority;        // [L][N]
  uint32_t* counters;     // [2] or null
};

hipError_t launch_actor_rollout(const RolloutArgs& a, hipStream_t st);
// Rows [row0, row1) of the feature table of RolloutArgs::ftable for the
// packed weights' actor, episodes starting at the clamped `starts` (at most
// `grid` workgroups, each reserving lds_pad bytes of LDS it does not use).
hipError_t launch_feature_table(const float* weights, const float* features, const int32_t* starts,
                                int64_t n_bars, int32_t N, int32_t L, bool bf16, float* table,
                                int64_t row0, int64_t row1, int grid, int lds_pad,
                                hipStream_t st);
int feature_table_lds_bytes(bool bf16);
hipError_t launch_dqn(const DqnArgs& a, hipStream_t st);
hipError_t launch_value(const ValueArgs& a, hipStream_t st);
// Static LDS bytes of a workgroup of the rollout / value kernel (-1 on error).
int actor_lds_bytes(bool bf16, bool recycle);
int value_lds_bytes(bool bf16);

}  // namespace rl
