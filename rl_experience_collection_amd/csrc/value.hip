// Batched part of PPO experience collection: the critic value (PPO CUDA
// Pipeline Design, Kernel Phases, Phase A step 5) and the curiosity bonus
// (step 9, the forward model of GPU Pipeline Phase 2b, Kernel Components 2)
// of every stored step, then the final reward (step 10).
//
// Neither output feeds a later step, so the L*N stored states are evaluated
// as one batch.  A workgroup holds kRowGroups groups of 16 consecutive (t, n)
// rows of the [L][N] layout; the kSplit = 4 waves of a group share its rows
// and each computes a quarter of every layer's outputs:
//   critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (fp32 MFMA, ReLU) -> 1 (VALU),
//   curiosity [state, one-hot(a)] -> 128 (ReLU) -> 51, MSE against the next
//   bar's 51 features, bonus = coef * MSE.
// Activations of a group live in one LDS buffer (a layer's input is read by
// all four waves, its output written back after a barrier), so a CU holds
// several workgroups and four waves per SIMD hide the weight-load latency.
// The packed weights (1.46 MB critic) stay L2-resident; the waves of the row
// groups read the same weight addresses in step (barriers keep them
// together), so L1 serves the repeats.  The one-hot half of the curiosity
// input is a column gather, not a dense product.
#include "collect.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
#ifndef RL_VALUE_ROW_GROUPS
#define RL_VALUE_ROW_GROUPS 2
#endif
constexpr int kRowGroups = RL_VALUE_ROW_GROUPS;
constexpr int kThreads = 64 * kSplit * kRowGroups;
constexpr int kBufF4 = 32 * 64;  // widest activation: 512 = 32 tiles of 16

template <int S, int OT>
__device__ __forceinline__ void layer(const float* W, int64_t w_off, int64_t b_off, f32x4* buf,
                                      int q, int lane) {
  constexpr int OTW = OT / kSplit;
  f32x4 acc[OTW];
  mfma_layer<S, OTW>(W + w_off, W + b_off, buf, acc, q, lane);
  __syncthreads();  // every wave has read the input
  relu_store<OTW>(acc, buf, q, lane);
  __syncthreads();  // the output is complete
}

__global__ __launch_bounds__(kThreads) void value_kernel(ValueArgs a) {
  __shared__ f32x4 s_buf[kRowGroups][kBufF4];
  __shared__ f32x4 s_state[kRowGroups][4 * 64];
  __shared__ float s_part[kRowGroups][kSplit][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / kSplit;
  const int q = wave % kSplit;
  const int g = lane >> 4;
  const int64_t rows = (int64_t)a.L * a.N;
  const int64_t row_raw = ((int64_t)blockIdx.x * kRowGroups + rg) * kRowsPerWave + (lane & 15);
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;  // tail rows recompute the last row
  const float* W = a.weights;
  f32x4* buf = s_buf[rg];

  // ---- state operands (first-layer k order: 14 per lane group) ------------
  if (q == 0) {
    const float* srow = a.states + row * kState + kFirstSteps * g;
    float B[16];
#pragma unroll
    for (int s = 0; s < kFirstSteps; ++s) B[s] = (kFirstSteps * g + s < kState) ? srow[s] : 0.0f;
    B[14] = 0.0f;
    B[15] = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      f32x4 v;
      v[0] = B[4 * k4]; v[1] = B[4 * k4 + 1]; v[2] = B[4 * k4 + 2]; v[3] = B[4 * k4 + 3];
      s_state[rg][k4 * 64 + lane] = v;
      buf[k4 * 64 + lane] = v;
    }
  }
  __syncthreads();

  // ---- critic -----------------------------------------------------------
  layer<16, 32>(W, kP.critic_w[0], kP.critic_b[0], buf, q, lane);
  layer<128, 24>(W, kP.critic_w[1], kP.critic_b[1], buf, q, lane);
  layer<96, 16>(W, kP.critic_w[2], kP.critic_b[2], buf, q, lane);
  layer<64, 8>(W, kP.critic_w[3], kP.critic_b[3], buf, q, lane);
  {
    // 64 -> 1 on the VALU: this wave holds hidden units 16q .. 16q+15
    f32x4 h[1];
    mfma_layer<32, 1>(W + kP.critic_w[4], W + kP.critic_b[4], buf, h, q, lane);
    const float* w6 = W + kP.critic_w6 + 16 * q + 4 * g;
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) part += w6[r] * fmaxf(h[0][r], 0.0f);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0) s_part[rg][q][lane] = part;
  }
  __syncthreads();  // critic input no longer needed; partial sums visible
  float value = 0.0f;
  if (q == 0)
    value = W[kP.critic_b6] + ((s_part[rg][0][lane & 15] + s_part[rg][1][lane & 15]) +
                               (s_part[rg][2][lane & 15] + s_part[rg][3][lane & 15]));

  // ---- curiosity --------------------------------------------------------
  int act_a = a.actions[row];
  act_a = act_a < 0 ? 0 : (act_a >= kActions ? kActions - 1 : act_a);
  {
    f32x4 c[2];
    mfma_layer<16, 2>(W + kP.cur_w[0], W + kP.cur_b[0], s_state[rg], c, q, lane);
    const float* oh = W + kP.cur_onehot + act_a * 128 + 4 * g;
#pragma unroll
    for (int i = 0; i < 2; ++i) c[i] += *reinterpret_cast<const f32x4*>(oh + 16 * (2 * q + i));
    relu_store<2>(c, buf, q, lane);  // buf was released by the barrier above
  }
  __syncthreads();
  float bonus = 0.0f;
  {
    f32x4 pr[1];
    mfma_layer<32, 1>(W + kP.cur_w[1], W + kP.cur_b[1], buf, pr, q, lane);
    const int32_t t = (int32_t)(row / a.N);
    const int32_t n = (int32_t)(row % a.N);
    const int64_t bar = (int64_t)a.start_used[n] + t;
    const float* fn = a.features + (bar + 1) * kFeatures;
    float se = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * q + 4 * g + r;
      if (j < kFeatures) {
        const float d = pr[0][r] - fn[j];
        se += d * d;
      }
    }
    se += __shfl_xor(se, 16);
    se += __shfl_xor(se, 32);
    __syncthreads();  // value partials read by wave 0 before they are reused
    if (g == 0) s_part[rg][q][lane] = se;
    __syncthreads();
    if (q == 0) {
      const float sum = (s_part[rg][0][lane & 15] + s_part[rg][1][lane & 15]) +
                        (s_part[rg][2][lane & 15] + s_part[rg][3][lane & 15]);
      bonus = a.ep.curiosity_coef * (sum / (float)kFeatures);
    }
  }

  // ---- step 10: reward = partial + curiosity - risk ----------------------
  if (q == 0 && valid && g == 0) {
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
  const int64_t per_block = kRowGroups * kRowsPerWave;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  hipLaunchKernelGGL(value_kernel, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rl
