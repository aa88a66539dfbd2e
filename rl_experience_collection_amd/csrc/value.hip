// Batched part of PPO experience collection: the critic value (PPO CUDA
// Pipeline Design, Kernel Phases, Phase A step 5) and the curiosity bonus
// (step 9, the forward model of GPU Pipeline Phase 2b, Kernel Components 2)
// of every stored step, then the final reward (step 10).
//
// Neither output feeds a later step, so the L*N stored states are evaluated
// as one batch.  A workgroup holds kRowGroups groups of 16 consecutive (t, n)
// rows of the [L][N] layout; the kSplit = 4 waves of a group share its rows
// and each computes a quarter of every layer's outputs:
//   critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (MFMA, ReLU) -> 1 (VALU),
//   curiosity [state, one-hot(a)] -> 128 (ReLU) -> 51, MSE against the next
//   bar's 51 features, bonus = coef * MSE.
// Activations of a group live in one LDS buffer (a layer's input is read by
// all four waves, its output written back after a barrier), so a CU holds
// several workgroups and four waves per SIMD hide the weight-load latency.
// The packed weights (1.46 MB critic) stay L2-resident; the waves of the row
// groups read the same weight addresses in step (barriers keep them
// together), so L1 serves the repeats.  The one-hot half of the curiosity
// input is a column gather, not a dense product.
// Precision: fp32 (v_mfma_f32_16x16x4_f32) or bf16 weights and layer inputs
// with fp32 accumulation (v_mfma_f32_16x16x32_bf16); biases, the last-layer
// outputs, the MSE and the reward stay fp32 in both.
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

// One layer of this wave: MFMA share, barrier, ReLU store, barrier.
template <bool BF16, int S32, int SB, int OT>
__device__ __forceinline__ void layer(const float* W, int64_t w32, int64_t wb, int64_t b_off,
                                      void* buf, int q, int lane) {
  constexpr int OTW = OT / kSplit;
  f32x4 acc[OTW];
  if constexpr (BF16)
    mfma_layer_bf16<SB, OTW>(reinterpret_cast<const uint4*>(W + wb), W + b_off,
                             reinterpret_cast<const uint4*>(buf), acc, q, lane);
  else
    mfma_layer<S32, OTW>(W + w32, W + b_off, reinterpret_cast<const f32x4*>(buf), acc, q, lane);
  lds_barrier();  // every wave has read the input
  if constexpr (BF16)
    relu_store_bf16<OTW>(acc, reinterpret_cast<uint4*>(buf), q, lane);
  else
    relu_store<OTW>(acc, reinterpret_cast<f32x4*>(buf), q, lane);
  lds_barrier();  // the output is complete
}

// This wave's share of a layer whose output is not stored (accumulators).
template <bool BF16, int S32, int SB, int OT>
__device__ __forceinline__ void last_layer(const float* W, int64_t w32, int64_t wb, int64_t b_off,
                                           const void* buf, f32x4 (&acc)[OT / kSplit], int q,
                                           int lane) {
  constexpr int OTW = OT / kSplit;
  if constexpr (BF16)
    mfma_layer_bf16<SB, OTW>(reinterpret_cast<const uint4*>(W + wb), W + b_off,
                             reinterpret_cast<const uint4*>(buf), acc, q, lane);
  else
    mfma_layer<S32, OTW>(W + w32, W + b_off, reinterpret_cast<const f32x4*>(buf), acc, q, lane);
}

template <bool BF16>
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
  void* buf = s_buf[rg];

  // ---- state operands ----------------------------------------------------
  if (q == 0) {
    const float* srow = a.states + row * kState;
    float B[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int k = state_k<BF16>(g, s);
      B[s] = k < kState ? srow[k] : 0.0f;
    }
    store_state_operands<BF16>(B, s_state[rg], lane);
    store_state_operands<BF16>(B, buf, lane);
  }
  lds_barrier();

  // ---- critic -----------------------------------------------------------
  layer<BF16, 16, 2, 32>(W, kP.critic_w[0], kP.bcritic_w[0], kP.critic_b[0], buf, q, lane);
  layer<BF16, 128, 16, 24>(W, kP.critic_w[1], kP.bcritic_w[1], kP.critic_b[1], buf, q, lane);
  layer<BF16, 96, 12, 16>(W, kP.critic_w[2], kP.bcritic_w[2], kP.critic_b[2], buf, q, lane);
  layer<BF16, 64, 8, 8>(W, kP.critic_w[3], kP.bcritic_w[3], kP.critic_b[3], buf, q, lane);
  {
    // 64 -> 1 on the VALU: this wave holds hidden units 16q .. 16q+15
    f32x4 h[1];
    last_layer<BF16, 32, 4, 4>(W, kP.critic_w[4], kP.bcritic_w[4], kP.critic_b[4], buf, h, q, lane);
    const float* w6 = W + (BF16 ? kP.bcritic_w6 : kP.critic_w6) + 16 * q + 4 * g;
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = fmaxf(h[0][r], 0.0f);
      part += w6[r] * (BF16 ? bf16_round(x) : x);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0) s_part[rg][q][lane] = part;
  }
  lds_barrier();  // critic input no longer needed; partial sums visible
  float value = 0.0f;
  if (q == 0)
    value = W[kP.critic_b6] + ((s_part[rg][0][lane & 15] + s_part[rg][1][lane & 15]) +
                               (s_part[rg][2][lane & 15] + s_part[rg][3][lane & 15]));

  // ---- curiosity --------------------------------------------------------
  int act_a = a.actions[row];
  act_a = act_a < 0 ? 0 : (act_a >= kActions ? kActions - 1 : act_a);
  {
    f32x4 c[2];
    last_layer<BF16, 16, 2, 8>(W, kP.cur_w[0], kP.bcur_w[0], kP.cur_b[0], s_state[rg], c, q, lane);
    const float* oh = W + (BF16 ? kP.bcur_onehot : kP.cur_onehot) + act_a * 128 + 4 * g;
#pragma unroll
    for (int i = 0; i < 2; ++i) c[i] += *reinterpret_cast<const f32x4*>(oh + 16 * (2 * q + i));
    // buf was released by the barrier above
    if constexpr (BF16)
      relu_store_bf16<2>(c, reinterpret_cast<uint4*>(buf), q, lane);
    else
      relu_store<2>(c, reinterpret_cast<f32x4*>(buf), q, lane);
  }
  lds_barrier();
  float bonus = 0.0f;
  {
    f32x4 pr[1];
    last_layer<BF16, 32, 4, 4>(W, kP.cur_w[1], kP.bcur_w[1], kP.cur_b[1], buf, pr, q, lane);
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
    lds_barrier();  // value partials read by wave 0 before they are reused
    if (g == 0) s_part[rg][q][lane] = se;
    lds_barrier();
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
  if (a.bf16)
    hipLaunchKernelGGL(value_kernel<true>, dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(value_kernel<false>, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rl
