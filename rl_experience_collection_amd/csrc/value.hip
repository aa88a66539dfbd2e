// Batched part of PPO experience collection: the critic value (PPO CUDA
// Pipeline Design, Kernel Phases, Phase A step 5) and the curiosity bonus
// (step 9, the forward model of GPU Pipeline Phase 2b, Kernel Components 2)
// of every stored step, then the final reward (step 10).
//
// Neither output feeds a later step, so the L*N stored states are evaluated
// as one batch.  A workgroup holds RT row tiles of 16 consecutive (t, n)
// rows of the [L][N] layout; its kSplit = 4 waves share all RT tiles and
// each computes a quarter of every layer's outputs for all of them:
//   critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (MFMA, ReLU) -> 1 (VALU),
//   curiosity [state, one-hot(a)] -> 128 (ReLU) -> 51, MSE against the next
//   bar's 51 features, bonus = coef * MSE.
// Every weight operand a wave loads feeds RT MFMAs (one per row tile), and
// the next layer's first weight steps are loaded before the barriers that
// end the current layer.  Activations live in LDS (a layer's input is read
// by all four waves, its output written back after a barrier).  The packed
// weights (1.46 MB fp32, 0.73 MB bf16) stay resident in every XCD's L2.
// The one-hot half of the curiosity input is a column gather, not a dense
// product.
// Precision: fp32 (v_mfma_f32_16x16x4_f32) or bf16 weights and layer inputs
// with fp32 accumulation (v_mfma_f32_16x16x32_bf16); biases, the last-layer
// outputs, the MSE and the reward stay fp32 in both.
#include "collect.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
#ifndef RL_VALUE_RT_F32
#define RL_VALUE_RT_F32 2
#endif
#ifndef RL_VALUE_RT_BF16
#define RL_VALUE_RT_BF16 4
#endif
constexpr int kThreads = 64 * kSplit;

template <bool BF16>
struct ValueShape {
  static constexpr int RT = BF16 ? RL_VALUE_RT_BF16 : RL_VALUE_RT_F32;
  // 16-byte LDS operands per row tile: the widest activation (512) and the
  // first-layer state operands
  static constexpr int kTile = BF16 ? 16 * 64 : 32 * 64;
  static constexpr int kStateTile = BF16 ? 2 * 64 : 4 * 64;
  static_assert(RT >= 1 && RT <= kSplit, "one wave loads each row tile's states");
};

template <bool BF16, int OTW>
__device__ __forceinline__ void begin(WeightStream<BF16, OTW>& st, const float* W, int64_t w32,
                                      int64_t wb, int64_t b_off, int q, int lane) {
  stream_begin<BF16, OTW>(st, W + (BF16 ? wb : w32), W + b_off, q, lane);
}

template <bool BF16, int S, int OTW, int RT>
__device__ __forceinline__ void run(WeightStream<BF16, OTW>& st, const float* W, int64_t w32,
                                    int64_t wb, const f32x4* buf, int tile_stride,
                                    f32x4 (&acc)[RT][OTW], int q, int lane) {
  if constexpr (BF16)
    stream_layer<S, OTW, RT>(st, W + wb, reinterpret_cast<const uint4*>(buf), tile_stride, acc, q,
                             lane);
  else
    stream_layer<S, OTW, RT>(st, W + w32, buf, tile_stride, acc, q, lane);
}

template <bool BF16, int OTW, int RT>
__device__ __forceinline__ void store(const f32x4 (&acc)[RT][OTW], f32x4* buf, int tile_stride,
                                      int q, int lane) {
  if constexpr (BF16)
    relu_store_tiles_bf16<OTW, RT>(acc, reinterpret_cast<uint4*>(buf), tile_stride, q, lane);
  else
    relu_store_tiles<OTW, RT>(acc, buf, tile_stride, q, lane);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void value_kernel(ValueArgs a) {
  using Sh = ValueShape<BF16>;
  constexpr int RT = Sh::RT;
  constexpr int TS = Sh::kTile;
  constexpr int SS = Sh::kStateTile;
  // layer k-steps (fp32 / bf16 forms differ) and per-wave output tiles
  constexpr int S1 = BF16 ? kCriticB[0].steps : kCritic[0].steps;
  constexpr int S2 = BF16 ? kCriticB[1].steps : kCritic[1].steps;
  constexpr int S3 = BF16 ? kCriticB[2].steps : kCritic[2].steps;
  constexpr int S4 = BF16 ? kCriticB[3].steps : kCritic[3].steps;
  constexpr int S5 = BF16 ? kCriticB[4].steps : kCritic[4].steps;
  constexpr int SC1 = BF16 ? kCurB[0].steps : kCur[0].steps;
  constexpr int SC2 = BF16 ? kCurB[1].steps : kCur[1].steps;
  __shared__ f32x4 s_buf[RT * TS];
  __shared__ f32x4 s_state[RT * SS];
  __shared__ float s_part[2][RT][kSplit][16];

  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int64_t rows = (int64_t)a.L * a.N;
  const int64_t tile0 = (int64_t)blockIdx.x * RT;
  const float* W = a.weights;

  WeightStream<BF16, 8> w1;
  begin(w1, W, kP.critic_w[0], kP.bcritic_w[0], kP.critic_b[0], q, lane);

  // ---- state operands: wave q < RT loads row tile q ----------------------
  const int64_t my_raw = (tile0 + q) * kRowsPerWave + (lane & 15);
  const int64_t my_row = my_raw < rows ? my_raw : rows - 1;  // tail rows recompute the last row
  if (q < RT) {
    const float* srow = a.states + my_row * kState;
    float B[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int k = state_k<BF16>(g, s);
      B[s] = k < kState ? srow[k] : 0.0f;
    }
    store_state_operands<BF16>(B, s_state + q * SS, lane);
    store_state_operands<BF16>(B, s_buf + q * TS, lane);
  }
  lds_barrier();

  // ---- critic -----------------------------------------------------------
  f32x4 h1[RT][8];
  run<BF16, S1, 8, RT>(w1, W, kP.critic_w[0], kP.bcritic_w[0], s_buf, TS, h1, q, lane);
  WeightStream<BF16, 6> w2;
  begin(w2, W, kP.critic_w[1], kP.bcritic_w[1], kP.critic_b[1], q, lane);
  lds_barrier();  // every wave has read the input
  store<BF16, 8, RT>(h1, s_buf, TS, q, lane);
  lds_barrier();  // the output is complete

  f32x4 h2[RT][6];
  run<BF16, S2, 6, RT>(w2, W, kP.critic_w[1], kP.bcritic_w[1], s_buf, TS, h2, q, lane);
  WeightStream<BF16, 4> w3;
  begin(w3, W, kP.critic_w[2], kP.bcritic_w[2], kP.critic_b[2], q, lane);
  lds_barrier();
  store<BF16, 6, RT>(h2, s_buf, TS, q, lane);
  lds_barrier();

  f32x4 h3[RT][4];
  run<BF16, S3, 4, RT>(w3, W, kP.critic_w[2], kP.bcritic_w[2], s_buf, TS, h3, q, lane);
  WeightStream<BF16, 2> w4;
  begin(w4, W, kP.critic_w[3], kP.bcritic_w[3], kP.critic_b[3], q, lane);
  lds_barrier();
  store<BF16, 4, RT>(h3, s_buf, TS, q, lane);
  lds_barrier();

  f32x4 h4[RT][2];
  run<BF16, S4, 2, RT>(w4, W, kP.critic_w[3], kP.bcritic_w[3], s_buf, TS, h4, q, lane);
  WeightStream<BF16, 1> w5;
  begin(w5, W, kP.critic_w[4], kP.bcritic_w[4], kP.critic_b[4], q, lane);
  lds_barrier();
  store<BF16, 2, RT>(h4, s_buf, TS, q, lane);
  lds_barrier();

  f32x4 h5[RT][1];
  run<BF16, S5, 1, RT>(w5, W, kP.critic_w[4], kP.bcritic_w[4], s_buf, TS, h5, q, lane);
  WeightStream<BF16, 2> c1;
  begin(c1, W, kP.cur_w[0], kP.bcur_w[0], kP.cur_b[0], q, lane);
  {
    // 64 -> 1 on the VALU: this wave holds hidden units 16q .. 16q+15
    const float* w6 = W + (BF16 ? kP.bcritic_w6 : kP.critic_w6) + 16 * q + 4 * g;
    const f32x4 w6v = *reinterpret_cast<const f32x4*>(w6);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = fmaxf(h5[rt][0][r], 0.0f);
        part += w6v[r] * (BF16 ? bf16_round(x) : x);
      }
      part += lane_xor16f(part, lane);
      part += lane_xor32f(part, lane);
      if (g == 0) s_part[0][rt][q][lane] = part;
    }
  }

  // ---- curiosity layer 1 (reads the state operands, not s_buf) ----------
  int act[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t raw = (tile0 + rt) * kRowsPerWave + (lane & 15);
    int v = a.actions[raw < rows ? raw : rows - 1];
    act[rt] = v < 0 ? 0 : (v >= kActions ? kActions - 1 : v);
  }
  f32x4 c[RT][2];
  run<BF16, SC1, 2, RT>(c1, W, kP.cur_w[0], kP.bcur_w[0], s_state, SS, c, q, lane);
  WeightStream<BF16, 1> c2;
  begin(c2, W, kP.cur_w[1], kP.bcur_w[1], kP.cur_b[1], q, lane);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float* oh = W + (BF16 ? kP.bcur_onehot : kP.cur_onehot) + act[rt] * 128 + 4 * g;
#pragma unroll
    for (int i = 0; i < 2; ++i) c[rt][i] += *reinterpret_cast<const f32x4*>(oh + 16 * (2 * q + i));
  }
  lds_barrier();  // critic input no longer read; value partials visible
  float value = 0.0f;
  if (q < RT)
    value = W[kP.critic_b6] + ((s_part[0][q][0][lane & 15] + s_part[0][q][1][lane & 15]) +
                               (s_part[0][q][2][lane & 15] + s_part[0][q][3][lane & 15]));
  store<BF16, 2, RT>(c, s_buf, TS, q, lane);
  lds_barrier();

  // ---- curiosity layer 2, MSE against the next bar's features -------------
  f32x4 pr[RT][1];
  run<BF16, SC2, 1, RT>(c2, W, kP.cur_w[1], kP.bcur_w[1], s_buf, TS, pr, q, lane);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t raw = (tile0 + rt) * kRowsPerWave + (lane & 15);
    const int64_t row = raw < rows ? raw : rows - 1;
    const int32_t t = (int32_t)(row / a.N);
    const int32_t n = (int32_t)(row % a.N);
    const int64_t bar = (int64_t)a.start_used[n] + t;
    const float* fn = a.features + (bar + 1) * kFeatures;
    float se = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * q + 4 * g + r;
      if (j < kFeatures) {
        const float d = pr[rt][0][r] - fn[j];
        se += d * d;
      }
    }
    se += lane_xor16f(se, lane);
    se += lane_xor32f(se, lane);
    if (g == 0) s_part[1][rt][q][lane] = se;
  }
  lds_barrier();

  // ---- step 10: reward = partial + curiosity - risk (wave q: row tile q) ---
  if (q < RT && g == 0 && my_raw < rows) {
    const float sum = (s_part[1][q][0][lane] + s_part[1][q][1][lane]) +
                      (s_part[1][q][2][lane] + s_part[1][q][3][lane]);
    const float bonus = a.ep.curiosity_coef * (sum / (float)kFeatures);
    int my_act = a.actions[my_row];
    my_act = my_act < 0 ? 0 : (my_act >= kActions ? kActions - 1 : my_act);
    const float ex = exposure_of(a.ep, my_act / 9);
    const float reward = (a.rewards[my_row] + bonus) - a.ep.risk_coef * fabsf(ex);
    a.values[my_row] = value;
    a.rewards[my_row] = reward;
    if (a.counters && (!isfinite(value) || !isfinite(reward))) atomicAdd(a.counters, 1u);
  }
}

}  // namespace

hipError_t launch_value(const ValueArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.L * a.N;
  if (rows <= 0) return hipSuccess;
  const int64_t tiles = (rows + kRowsPerWave - 1) / kRowsPerWave;
  if (a.bf16) {
    constexpr int RT = ValueShape<true>::RT;
    hipLaunchKernelGGL(value_kernel<true>, dim3((unsigned)((tiles + RT - 1) / RT)), dim3(kThreads),
                       0, st, a);
  } else {
    constexpr int RT = ValueShape<false>::RT;
    hipLaunchKernelGGL(value_kernel<false>, dim3((unsigned)((tiles + RT - 1) / RT)), dim3(kThreads),
                       0, st, a);
  }
  return hipGetLastError();
}

}  // namespace rl
