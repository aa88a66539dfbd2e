// Episode-row helpers shared by the sequential collection kernels: after a
// layer, wave q of a 16-episode workgroup owns episodes 4q .. 4q+3, one row
// of 16 lanes each, for the per-episode work (draws, environment, stores).
#pragma once

#include "nets.hpp"

namespace rl {

// Cross-lane steps within a row of 16 lanes (DPP).  Sums use xor-pattern
// partners (quad_perm 1,0,3,2 and 2,3,0,1, then row_half_mirror i^7 and
// row_mirror i^15), so every lane of the row ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
__device__ __forceinline__ float row_sum(float x) {
  x = x + dpp_f<kXor1>(x);
  x = x + dpp_f<kXor2>(x);
  x = x + dpp_f<kHalfMirror>(x);
  return x + dpp_f<kMirror>(x);
}
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_f<kXor1>(x));
  x = fmaxf(x, dpp_f<kXor2>(x));
  x = fmaxf(x, dpp_f<kHalfMirror>(x));
  return fmaxf(x, dpp_f<kMirror>(x));
}
__device__ __forceinline__ int row_min_i(int x) {
  x = min(x, dpp_i<kXor1>(x));
  x = min(x, dpp_i<kXor2>(x));
  x = min(x, dpp_i<kHalfMirror>(x));
  return min(x, dpp_i<kMirror>(x));
}
__device__ __forceinline__ int row_max_i(int x) {
  x = max(x, dpp_i<kXor1>(x));
  x = max(x, dpp_i<kXor2>(x));
  x = max(x, dpp_i<kHalfMirror>(x));
  return max(x, dpp_i<kMirror>(x));
}
// The value lane `src` (uniform, 0..15) of this lane's row holds.
__device__ __forceinline__ uint32_t row_pick_u32(uint32_t x, int src, int lane) {
  const uint32_t r0 = __builtin_amdgcn_readlane(x, src);
  const uint32_t r1 = __builtin_amdgcn_readlane(x, 16 + src);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 32 + src);
  const uint32_t r3 = __builtin_amdgcn_readlane(x, 48 + src);
  const int row = lane >> 4;
  return row == 0 ? r0 : (row == 1 ? r1 : (row == 2 ? r2 : r3));
}

// Counter-based draws of one episode row, 16 steps at a time: at every 16th
// step of a launch (t - t_begin = 0 mod 16) lane j evaluates the generator
// for step t + j, and each step takes its draw from lane (t - t_begin) % 16.
// One evaluation per lane per 16 steps instead of one per step: Philox's 40
// 32-bit multiplies per evaluation are quarter-rate instructions.
struct RowDraws {
  uint32_t pool = 0;
  __device__ __forceinline__ uint32_t take(int src, int lane) const {
    return row_pick_u32(pool, src, lane);
  }
};

// inclusive prefix sum over the row (lanes below the shift read 0)
__device__ __forceinline__ float row_scan(float x) {
  x = x + dpp_f<0x111>(x);  // row_shr:1
  x = x + dpp_f<0x112>(x);  // row_shr:2
  x = x + dpp_f<0x114>(x);  // row_shr:4
  return x + dpp_f<0x118>(x);  // row_shr:8
}

// Position of state element k of episode e in the first-layer operand
// buffer (natural order k = 4 s + g for fp32, k = 32 s + 8 g + j for bf16):
// fp32 as a float index (slot s of lane e + 16 g), bf16 as a 16-bit index.
template <bool BF16>
__device__ __forceinline__ int state_slot(int e, int k) {
  if constexpr (BF16) {
    return ((k >> 5) * 64 + e + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
  } else {
    const int s = k >> 2, g = k & 3;
    return ((s >> 2) * 64 + e + 16 * g) * 4 + (s & 3);
  }
}
template <bool BF16>
__device__ __forceinline__ void put_state(f32x4* sbuf, int e, int k, float v) {
  if constexpr (BF16)
    reinterpret_cast<uint16_t*>(sbuf)[state_slot<true>(e, k)] = (uint16_t)bf16_bits(v);
  else
    reinterpret_cast<float*>(sbuf)[state_slot<false>(e, k)] = v;
}

// The 4 features k = j + 16 h (h = 0..3, k < 51) of a bar that lane j of an
// episode row handles; unconditional loads (clamped), masked after.
__device__ __forceinline__ void load_features(const float* __restrict__ F, int64_t bar, int j,
                                              float (&f)[4]) {
  const float* row = F + bar * kFeatures;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int k = j + 16 * h;
    const float v = row[k < kFeatures ? k : kFeatures - 1];
    f[h] = k < kFeatures ? v : 0.0f;
  }
}

// Restart bar of an episode that ends at step t < L-1 (dynamic episode
// recycling, "GPU Pipeline Phase 2b", Future Phase 3 Optimization): with
// R = L - t - 1 steps left, floor(x range / 2^32) over range = n_bars - R
// valid starts, x the first Philox word of counter (episode, t, 5, 0).
__device__ __forceinline__ int64_t recycle_bar(uint64_t seed, uint32_t n, int32_t t, int32_t L,
                                               int64_t n_bars) {
  const uint4 r = philox10(make_uint4(n, (uint32_t)t, 5u, 0u), (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t range = (uint64_t)(n_bars - ((int64_t)L - t - 1));
  return (int64_t)(((uint64_t)r.x * range) >> 32);
}

}  // namespace rl
