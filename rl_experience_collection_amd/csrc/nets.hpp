// Packed network weights, environment constants and the MFMA layer
// evaluator shared by the actor-rollout and value kernels.
#pragma once

#include "device.hpp"

namespace rl {

// ---------------------------------------------------------------------------
// Packed weight block.  One device allocation holds every layer in the MFMA
// operand order described in device.hpp; offsets are in floats and 64-float
// aligned.  First layers (state input) use S = 16 k-steps, the 54 inputs
// spread 14 per lane group with the last two steps zero.
// ---------------------------------------------------------------------------
struct LayerDesc {
  int in, out, steps, first;  // first: state-input k order, else chained order
};

// Actor: 54 -> 128 -> 64 -> 45 (PPO CUDA Pipeline Design, Weight Layout).
constexpr LayerDesc kActor[3] = {{54, 128, 16, 1}, {128, 64, 32, 0}, {64, 45, 16, 0}};
// Critic: 54 -> 512 -> 384 -> 256 -> 128 -> 64 (-> 1 handled on the VALU).
constexpr LayerDesc kCritic[5] = {
    {54, 512, 16, 1}, {512, 384, 128, 0}, {384, 256, 96, 0}, {256, 128, 64, 0}, {128, 64, 32, 0}};
// Curiosity forward model: 54 dense inputs (+45 one-hot, gathered) -> 128 -> 51.
constexpr LayerDesc kCur[2] = {{54, 128, 16, 1}, {128, 51, 32, 0}};

struct PackedOffsets {
  // actor block (contiguous, staged into LDS by the rollout kernel)
  int64_t actor_w[3], actor_b[3], actor_end;
  int64_t critic_w[5], critic_b[5], critic_w6, critic_b6;
  int64_t cur_w[2], cur_b[2], cur_onehot;
  int64_t total;
};

__host__ __device__ constexpr int64_t align64(int64_t x) { return (x + 63) / 64 * 64; }

__host__ __device__ constexpr PackedOffsets packed_offsets() {
  PackedOffsets p{};
  int64_t off = 0;
  for (int l = 0; l < 3; ++l) {
    p.actor_w[l] = off;
    off = align64(off + packed_floats(kActor[l].steps, kActor[l].out));
  }
  for (int l = 0; l < 3; ++l) {
    p.actor_b[l] = off;
    off = align64(off + 16 * out_tiles(kActor[l].out));
  }
  p.actor_end = off;
  for (int l = 0; l < 5; ++l) {
    p.critic_w[l] = off;
    off = align64(off + packed_floats(kCritic[l].steps, kCritic[l].out));
  }
  for (int l = 0; l < 5; ++l) {
    p.critic_b[l] = off;
    off = align64(off + 16 * out_tiles(kCritic[l].out));
  }
  p.critic_w6 = off;
  off = align64(off + 64);
  p.critic_b6 = off;
  off = align64(off + 1);
  for (int l = 0; l < 2; ++l) {
    p.cur_w[l] = off;
    off = align64(off + packed_floats(kCur[l].steps, kCur[l].out));
  }
  for (int l = 0; l < 2; ++l) {
    p.cur_b[l] = off;
    off = align64(off + 16 * out_tiles(kCur[l].out));
  }
  p.cur_onehot = off;
  off = align64(off + 45 * 128);
  p.total = off;
  return p;
}

// Scalar constants of the environment step, computed once on the host.
struct EnvParams {
  float ex0, ex1, ex2, ex3, ex4;   // exposure of a/9
  float cost0, cost1, cost2;       // cost rate of (a%9)/3
  float urgency_mult;
  float up_pt, dn_sl, dn_pt, up_sl;  // 1 +/- profit_take, 1 +/- stop_loss (fp32)
  int32_t max_hold;
  int32_t div_window;
  float div_threshold, div_penalty;
  float barrier_scale, spread, risk_coef, curiosity_coef;
};

__device__ __forceinline__ float exposure_of(const EnvParams& p, int x) {
  return x == 0 ? p.ex0 : (x == 1 ? p.ex1 : (x == 2 ? p.ex2 : (x == 3 ? p.ex3 : p.ex4)));
}
__device__ __forceinline__ float cost_of(const EnvParams& p, int o) {
  return o == 0 ? p.cost0 : (o == 1 ? p.cost1 : p.cost2);
}

// ---------------------------------------------------------------------------
// One MFMA layer for the 16 rows of a wave: acc[ot] = bias + W x, where the
// lane's B operands for k-steps 4*kt .. 4*kt+3 sit in its own LDS slot
// act[kt*64 + lane] (a float4).  Those slots are written by the same lane
// (its D registers of the previous layer, or its state inputs), so the
// buffer is lane-private and needs no barrier.  Weights are read with one
// 16-byte load per 4 MFMAs and prefetched one k-step ahead.
// ---------------------------------------------------------------------------
template <int S, int OT>
__device__ __forceinline__ void mfma_layer(const f32x4* __restrict__ pk, const float* __restrict__ pb,
                                           const f32x4* act, f32x4 (&acc)[OT], int lane) {
  constexpr int OG = (OT + 3) / 4;
  constexpr int KT = (S + 3) / 4;
  const int g = lane >> 4;
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) acc[ot] = *reinterpret_cast<const f32x4*>(pb + 16 * ot + 4 * g);
  const f32x4* w = pk + lane;
  f32x4 a_cur[OG], a_nxt[OG];
#pragma unroll
  for (int og = 0; og < OG; ++og) a_cur[og] = w[og * 64];
#pragma unroll 1
  for (int kt = 0; kt < KT; ++kt) {
    const f32x4 b = act[kt * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 4 * kt + r;
      const int sn = (s + 1 < S) ? s + 1 : s;
#pragma unroll
      for (int og = 0; og < OG; ++og) a_nxt[og] = w[(sn * OG + og) * 64];
#pragma unroll
      for (int og = 0; og < OG; ++og) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * og + c < OT) acc[4 * og + c] = mfma4(a_cur[og][c], b[r], acc[4 * og + c]);
      }
#pragma unroll
      for (int og = 0; og < OG; ++og) a_cur[og] = a_nxt[og];
    }
  }
}

// ReLU the accumulators into the lane's LDS slots (next layer's B operands).
template <int OT>
__device__ __forceinline__ void relu_store(const f32x4 (&acc)[OT], f32x4* act, int lane) {
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    f32x4 v = acc[ot];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = fmaxf(v[r], 0.0f);
    act[ot * 64 + lane] = v;
  }
}

}  // namespace rl
