// Host-side interface of the GAE scan kernel (see gae.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rl {

// Two shapes: rollouts of at most 512 steps use columns of 32 episodes and
// 16-step slots (two per wave), longer ones columns of 64 episodes and
// 32-step slots (one per wave) with super-chunks chained by a look-back.
// Both have 16-wave workgroups and 512-step super-chunks; each thread holds
// one slot in registers (3 words per step).
constexpr int kGaeWaves = 16;
constexpr int gae_chunk(int cols) { return cols == 32 ? 16 : 32; }
constexpr int gae_slots(int cols) { return kGaeWaves * 64 / cols; }
constexpr int gae_super(int cols) { return gae_slots(cols) * gae_chunk(cols); }
inline int32_t cdiv_i(int32_t a, int32_t b) { return (a + b - 1) / b; }

struct GaeArgs {
  const float* rewards;
  const float* values;
  const uint8_t* dones;
  const float* last_values;  // nullable
  int32_t L, N;
  float gamma, lambda;
  float* advantages;
  float* returns;
  // nullable: incremented once per look-back that gave up waiting (never
  // expected; the carry of that super-chunk is NaN, so the advantages and
  // returns of its column from there back to step 0 are NaN)
  uint32_t* status;
  // polls of a look-back before it gives up (kGaeSpinLimit unless the host
  // sets another, e.g. to exercise the give-up path)
  uint32_t spin_limit;
};

constexpr uint32_t kGaeSpinLimit = 1u << 24;

struct GaeShape {
  int32_t cols;    // episodes per column (32 or 64)
  int32_t nc, nk;  // columns and super-chunks
  int64_t tiles() const { return (int64_t)nc * nk; }  // workgroups of a launch
};

// Device view of the carry scratch of one stream/collector.
struct GaeScratchView {
  uint64_t* words;     // [nk * N]: value | (epoch << 3 | has_done << 2 | status) << 32
  uint32_t* ticket;    // monotonically increasing ticket counter
  uint32_t ticket_base;
  uint32_t epoch;      // < 2^29
};

inline size_t gae_words_bytes(int32_t nk, int32_t N) {
  return ((size_t)nk * N * 8 + 255) / 256 * 256;
}
inline size_t gae_scratch_bytes(int32_t nk, int32_t N) { return 256 + gae_words_bytes(nk, N); }

GaeShape gae_shape(int32_t L, int32_t N);
// Zero `words` 32-bit words at p, stream-ordered, with a kernel (a memset node
// is avoided so that the launch sequence can be captured into a graph).
hipError_t zero_words(uint32_t* p, size_t words, hipStream_t stream);
hipError_t gae_launch(const GaeArgs& a, const GaeShape& shape, const GaeScratchView& sc,
                      hipStream_t stream);

}  // namespace rl
