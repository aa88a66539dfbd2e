// Batched part of PPO experience collection: the critic value (PPO CUDA
// Pipeline Design, Kernel Phases, Phase A step 5) and the curiosity bonus
// (step 9, the forward model of GPU Pipeline Phase 2b, Kernel Components 2)
// of every stored step, then the final reward (step 10).
//
// Neither output feeds a later step, so the L*N stored states are evaluated
// as one batch: each wave takes 16 consecutive (t, n) rows of the [L][N]
// layout through
//   critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (fp32 MFMA, ReLU) -> 1 (VALU),
//   curiosity [state, one-hot(a)] -> 128 (ReLU) -> 51, MSE against the next
//   bar's 51 features, bonus = coef * MSE,
// keeping activations in a lane-private LDS slot between layers and
// streaming the packed weights (1.46 MB critic, L2-resident) through
// registers, one 16-byte load per 4 MFMAs.  The one-hot half of the
// curiosity input is a column gather, not a dense product.
#include "collect.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
constexpr int kWavesPerBlock = 4;
constexpr int kActF4PerWave = 32 * 64;  // widest activation: 512 = 32 tiles

__device__ __forceinline__ void store_state_operands(const float* __restrict__ srow, int g,
                                                     f32x4* act, int lane) {
  float B[16];
#pragma unroll
  for (int s = 0; s < kFirstSteps; ++s) B[s] = (kFirstSteps * g + s < kState) ? srow[s] : 0.0f;
  B[14] = 0.0f;
  B[15] = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 v;
    v[0] = B[4 * q]; v[1] = B[4 * q + 1]; v[2] = B[4 * q + 2]; v[3] = B[4 * q + 3];
    act[q * 64 + lane] = v;
  }
}

__global__ __launch_bounds__(64 * kWavesPerBlock, 1) void value_kernel(ValueArgs a) {
  __shared__ f32x4 s_act[kWavesPerBlock][kActF4PerWave];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int64_t rows = (int64_t)a.L * a.N;
  const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave;
  if (row0 >= rows) return;  // whole wave past the end (no barriers below)
  const int64_t row_raw = row0 + (lane & 15);
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;
  const int32_t t = (int32_t)(row / a.N);
  const int32_t n = (int32_t)(row % a.N);
  int act_a = a.actions[row];
  act_a = act_a < 0 ? 0 : (act_a >= kActions ? kActions - 1 : act_a);
  const int64_t bar = (int64_t)a.start_used[n] + t;
  const float* W = a.weights;
  const float* srow = a.states + row * kState + kFirstSteps * g;
  f32x4* act = s_act[wave];

  // ---- critic -----------------------------------------------------------
  store_state_operands(srow, g, act, lane);
  {
    f32x4 h[32];
    mfma_layer<16, 32>(reinterpret_cast<const f32x4*>(W + kP.critic_w[0]), W + kP.critic_b[0], act, h,
                       lane);
    relu_store<32>(h, act, lane);
  }
  {
    f32x4 h[24];
    mfma_layer<128, 24>(reinterpret_cast<const f32x4*>(W + kP.critic_w[1]), W + kP.critic_b[1], act,
                        h, lane);
    relu_store<24>(h, act, lane);
  }
  {
    f32x4 h[16];
    mfma_layer<96, 16>(reinterpret_cast<const f32x4*>(W + kP.critic_w[2]), W + kP.critic_b[2], act, h,
                       lane);
    relu_store<16>(h, act, lane);
  }
  {
    f32x4 h[8];
    mfma_layer<64, 8>(reinterpret_cast<const f32x4*>(W + kP.critic_w[3]), W + kP.critic_b[3], act, h,
                      lane);
    relu_store<8>(h, act, lane);
  }
  float value;
  {
    f32x4 h[4];
    mfma_layer<32, 4>(reinterpret_cast<const f32x4*>(W + kP.critic_w[4]), W + kP.critic_b[4], act, h,
                      lane);
    // 64 -> 1 on the VALU: lane partial over its 16 hidden units, then the
    // 4 lanes of the row combine pairwise (identical in every lane)
    const float* w6 = W + kP.critic_w6;
    float part = 0.0f;
#pragma unroll
    for (int ot = 0; ot < 4; ++ot)
#pragma unroll
      for (int r = 0; r < 4; ++r) part += w6[16 * ot + 4 * g + r] * fmaxf(h[ot][r], 0.0f);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    value = W[kP.critic_b6] + part;
  }

  // ---- curiosity --------------------------------------------------------
  store_state_operands(srow, g, act, lane);
  {
    f32x4 c[8];
    mfma_layer<16, 8>(reinterpret_cast<const f32x4*>(W + kP.cur_w[0]), W + kP.cur_b[0], act, c, lane);
    const float* oh = W + kP.cur_onehot + act_a * 128 + 4 * g;
#pragma unroll
    for (int ot = 0; ot < 8; ++ot) c[ot] += *reinterpret_cast<const f32x4*>(oh + 16 * ot);
    relu_store<8>(c, act, lane);
  }
  float bonus;
  {
    f32x4 pr[4];
    mfma_layer<32, 4>(reinterpret_cast<const f32x4*>(W + kP.cur_w[1]), W + kP.cur_b[1], act, pr, lane);
    const float* fn = a.features + (bar + 1) * kFeatures;
    float se = 0.0f;
#pragma unroll
    for (int ot = 0; ot < 4; ++ot)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * ot + 4 * g + r;
        if (j < kFeatures) {
          const float d = pr[ot][r] - fn[j];
          se += d * d;
        }
      }
    se += __shfl_xor(se, 16);
    se += __shfl_xor(se, 32);
    bonus = a.ep.curiosity_coef * (se / (float)kFeatures);
  }

  // ---- step 10: reward = partial + curiosity - risk ----------------------
  if (valid && g == 0) {
    const float ex = exposure_of(a.ep, act_a / 9);
    const float reward = (a.rewards[row] + bonus) - a.ep.risk_coef * fabsf(ex);
    a.values[row] = value;
    a.rewards[row] = reward;
    if (a.counters && (!isfinite(value) || !isfinite(reward))) atomicAdd(a.counters, 1u);
  }
}

}  // namespace

hipError_t launch_value(const ValueArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.L * a.N;
  if (rows <= 0) return hipSuccess;
  const int64_t per_block = kWavesPerBlock * kRowsPerWave;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  hipLaunchKernelGGL(value_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace rl
