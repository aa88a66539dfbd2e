// Host-side interface of the GAE scan kernel (see gae.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rl {

constexpr int kGaeChunk = 16;  // steps per tile (registers: 16 x EPT x 3 words)

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
};

struct GaeShape {
  int ept;  // episodes per thread (vector width of the loads)
  int tc;   // steps per tile
  int32_t nc, nk;  // tile columns and chunks
  int64_t tiles() const { return (int64_t)nc * nk; }
};

// Device view of the carry scratch of one stream/collector.
struct GaeScratchView {
  uint32_t* flags;     // [nk * nc], (epoch << 2) | status
  uint64_t* agg;       // [nk * N] packed (alpha, beta)
  float* incl;         // [nk * N]
  uint32_t* ticket;    // monotonically increasing ticket counter
  uint32_t* error;     // spin-limit events (never expected)
  uint32_t ticket_base;
  uint32_t epoch;
};

inline size_t gae_scratch_bytes(int32_t nk, int32_t nc, int32_t N) {
  const size_t flags = (size_t)nk * nc * 4;
  const size_t agg = (size_t)nk * N * 8;
  const size_t incl = (size_t)nk * N * 4;
  return 256 + ((flags + 255) / 256) * 256 + ((agg + 255) / 256) * 256 + ((incl + 255) / 256) * 256;
}

GaeShape gae_shape(int32_t L, int32_t N, bool aligned16, bool aligned8);
hipError_t gae_launch(const GaeArgs& a, const GaeShape& shape, const GaeScratchView& sc,
                      hipStream_t stream);

}  // namespace rl
