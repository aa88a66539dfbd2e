// Sequential part of PPO experience collection (PPO CUDA Pipeline Design,
// Kernel Phases, Phase A): the chain that each step's state depends on.
//
// Four waves own 16 episodes for all L steps, each computing a quarter of
// every actor layer's outputs (activations shared through LDS).  Per step
//   - assembles the 54-wide state (51 features of the bar, V/V0 - 1, the
//     exposure held, the spread) and stores it (steps 1-2, 11),
//   - runs the actor 54 -> 128 -> 64 -> 45 on MFMA (fp32, or bf16 weights and
//     layer inputs with fp32 accumulation) with the packed actor resident in
//     LDS for the whole kernel (step 3),
//   - takes a max-shifted softmax, its CDF and the inverse-CDF draw
//     a = min{k : u < CDF_k} with u from the counter-based generator, and
//     log p(a) = (l_a - max) - ln S (step 4),
//   - steps the portfolio, the triple barrier and the diversity window,
//     kept in registers, and forms the part of the reward that needs them
//     (steps 6-8, 10), then resets the episode when a barrier fired (12).
// The critic value (step 5) and the curiosity bonus (step 9) are not read
// by any later step, so they are evaluated afterwards by the value kernel
// in one batched pass over every stored state.
//
// The layers use the MFMA layout (lane l computes rows l % 16).  The draw
// and the environment use another: wave q owns episodes 4q .. 4q+3 of the
// row group, one 16-lane row each; lane j of a row holds logits j, j + 16
// and j + 32 (read from LDS), so the softmax sums and the CDF are DPP
// reductions and scans within the row, and every lane of the row holds the
// episode's portfolio state.  Each wave writes its own episodes' state
// operands, state rows and outputs.
#include "collect.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
constexpr int64_t kActorF32 = kP.actor_end;                  // fp32 actor block (floats)
constexpr int64_t kActorBF16 = kP.bact_end - kP.bact_begin;  // bf16 actor block (floats)
constexpr int kActorF4 = (int)((kActorF32 > kActorBF16 ? kActorF32 : kActorBF16) / 4);
constexpr int kBufA = 8 * 64;  // first-layer output (128 = 8 tiles), then the logits
constexpr int kBufB = 4 * 64;  // second-layer output (64 = 4 tiles)

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
// inclusive prefix sum over the row (lanes below the shift read 0)
__device__ __forceinline__ float row_scan(float x) {
  x = x + dpp_f<0x111>(x);  // row_shr:1
  x = x + dpp_f<0x112>(x);  // row_shr:2
  x = x + dpp_f<0x114>(x);  // row_shr:4
  return x + dpp_f<0x118>(x);  // row_shr:8
}

// Position of state element k of row-group episode e in the first-layer
// operand buffer: fp32 as a float index (k = 14 g + s, slot s of lane
// e + 16 g), bf16 as a 16-bit index (k = 32 s' + 8 g + j).
template <bool BF16>
__device__ __forceinline__ int state_slot(int e, int k) {
  if constexpr (BF16) {
    return ((k >> 5) * 64 + e + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
  } else {
    const int g = k / kFirstSteps, s = k - kFirstSteps * g;
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

template <int RG, bool BF16>
__global__ __launch_bounds__(64 * kSplit * RG) void actor_rollout_kernel(RolloutArgs a) {
  __shared__ f32x4 s_w[kActorF4];
  __shared__ f32x4 s_bufA[RG][kBufA];
  __shared__ f32x4 s_bufB[RG][kBufB];
  __shared__ f32x4 s_state[RG][4 * 64];
  __shared__ float s_ln[33];  // ln k for window counts k = 0..32 (ln 0 unused: times 0)
  __shared__ float s_env[kEnvTable];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / kSplit;
  const int q = wave % kSplit;

  if (threadIdx.x <= 32) s_ln[threadIdx.x] = threadIdx.x == 0 ? 0.0f : logf((float)threadIdx.x);
  fill_env_table(a.ep, s_env, (int)threadIdx.x);
  {  // stage the packed actor (fp32 or bf16 block) into LDS
    const int64_t begin = BF16 ? kP.bact_begin : 0;
    const int n4 = (int)((BF16 ? kActorBF16 : kActorF32) / 4);
    const f32x4* src = reinterpret_cast<const f32x4*>(a.weights + begin);
    for (int i = threadIdx.x; i < n4; i += 64 * kSplit * RG) s_w[i] = src[i];
  }
  // state operands start at zero: the padding slots stay zero
  for (int i = threadIdx.x; i < RG * 4 * 64; i += 64 * kSplit * RG)
    (&s_state[0][0])[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Draw and environment layout: wave q owns episodes 4q .. 4q+3 of its
  // row group, one row of 16 lanes (j = lane % 16) per episode; a row holds
  // the episode's portfolio state identically in all 16 lanes.
  const int e = 4 * q + (lane >> 4);  // episode within the row group
  const int j = lane & 15;
  const int32_t n_raw = (blockIdx.x * RG + rg) * kRowsPerWave + e;
  const bool valid = n_raw < a.N;
  const int32_t n = valid ? n_raw : a.N - 1;
  const EnvParams& ep = a.ep;

  // clamp the start so every read stays inside the market buffers
  const int64_t hi = a.n_bars - (int64_t)a.L - 1;
  int64_t st = a.starts[n];
  const bool clamped = st < 0 || st > hi;
  st = st < 0 ? 0 : (st > hi ? hi : st);
  if (valid && j == 0) {
    a.start_used[n] = (int32_t)st;
    if (clamped && a.counters) atomicAdd(a.counters + 1, 1u);
  }

  const float* sw = reinterpret_cast<const float*>(s_w);
  f32x4* bufA = s_bufA[rg];
  f32x4* bufB = s_bufB[rg];
  f32x4* sbuf = s_state[rg];

  float fcur[4];
  load_features(a.features, st, j, fcur);
  float p0 = a.prices[st], p1 = a.prices[st + 1];

  // episode state (PPO CUDA Pipeline Design, Phase A steps 6-8, 12)
  float V = 1.0f, e_prev = 0.0f, entry = 0.0f;
  int armed = 0, side = 0, t_open = 0;
  int cnt0 = 0, cnt1 = 0, cnt2 = 0, pushed = 0, pos = 0;
  uint64_t ring = 0;  // 2 bits per window slot
  const float V0 = 1.0f;
  lds_barrier();  // weights staged, operand buffer cleared
  if (j == 2) put_state<BF16>(sbuf, e, 53, ep.spread);  // constant element

  for (int32_t t = 0; t < a.L; ++t) {
    const int64_t bar = st + t;
    const int64_t o = (int64_t)t * a.N + n;

    // prefetch the next bar (independent of this step's outcome), issued
    // before this step's stores so that no wait in the step covers them; on
    // the last step the bar is still inside the buffers and goes unused
    float fnext[4];
    load_features(a.features, bar + 1, j, fnext);
    const float p2 = a.prices[bar + 2 < a.n_bars ? bar + 2 : a.n_bars - 1];

    // ---- steps 1-2: state = 51 features, V/V0 - 1, exposure held, spread --
    const float vn = V / V0 - 1.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (j + 16 * h < kFeatures) put_state<BF16>(sbuf, e, j + 16 * h, fcur[h]);
    if (j == 0) put_state<BF16>(sbuf, e, 51, vn);
    if (j == 1) put_state<BF16>(sbuf, e, 52, e_prev);
    if (valid) {
      float* srow = a.states + o * kState;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (j + 16 * h < kFeatures) srow[j + 16 * h] = fcur[h];
      if (j < 3) srow[kFeatures + j] = j == 0 ? vn : (j == 1 ? e_prev : ep.spread);
    }
    lds_barrier();  // state operands written; last step's logits read

    // the step's draw depends only on (seed, episode, step)
    const float u = draw_uniform(a.seed, (uint32_t)n, (uint32_t)t, 0u);

    // ---- step 3: actor, a quarter of each layer per wave ------------------
    // (MFMA layout: lane l computes rows l % 16 of the row group)
    {
      f32x4 h[2];
      if constexpr (BF16) {
        mfma_layer_bf16<2, 2>(reinterpret_cast<const uint4*>(sw + kP.bact_w[0] - kP.bact_begin),
                              sw + kP.bact_b[0] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(sbuf), h, q, lane);
        relu_store_bf16<2>(h, reinterpret_cast<uint4*>(bufA), q, lane);
      } else {
        mfma_layer<16, 2>(sw + kP.actor_w[0], sw + kP.actor_b[0], sbuf, h, q, lane);
        relu_store<2>(h, bufA, q, lane);
      }
    }
    lds_barrier();
    {
      f32x4 h[1];
      if constexpr (BF16) {
        mfma_layer_bf16<4, 1>(reinterpret_cast<const uint4*>(sw + kP.bact_w[1] - kP.bact_begin),
                              sw + kP.bact_b[1] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(bufA), h, q, lane);
        relu_store_bf16<1>(h, reinterpret_cast<uint4*>(bufB), q, lane);
      } else {
        mfma_layer<32, 1>(sw + kP.actor_w[1], sw + kP.actor_b[1], bufA, h, q, lane);
        relu_store<1>(h, bufB, q, lane);
      }
    }
    lds_barrier();
    {
      f32x4 h[1];
      if constexpr (BF16)
        mfma_layer_bf16<2, 1>(reinterpret_cast<const uint4*>(sw + kP.bact_w[2] - kP.bact_begin),
                              sw + kP.bact_b[2] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(bufB), h, q, lane);
      else
        mfma_layer<16, 1>(sw + kP.actor_w[2], sw + kP.actor_b[2], bufB, h, q, lane);
      // raw logits, fp32 (tile 3 is padding), over the first-layer output,
      // which every wave finished reading before the previous barrier:
      // logit k of row e at bufA[(k / 16) * 64 + e + 16 * (k % 16 / 4)][k % 4]
      bufA[q * 64 + lane] = h[0];
    }
    lds_barrier();

    // ---- step 4: softmax, CDF, inverse-CDF draw, log-prob -----------------
    // lane j of the episode's row holds logits k = j + 16 h, h = 0..2
    const float* lg = reinterpret_cast<const float*>(bufA);
    float l[3], ex[3];
    bool ok[3];
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      ok[h] = j + 16 * h < kActions;
      l[h] = lg[(h * 64 + e + 16 * (j >> 2)) * 4 + (j & 3)];
    }
    int bad = 0;
    float m = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (ok[h]) {
        bad |= !isfinite(l[h]);
        m = fmaxf(m, l[h]);
      }
    m = row_max(m);
#pragma unroll
    for (int h = 0; h < 3; ++h) ex[h] = ok[h] ? expf(l[h] - m) : 0.0f;
    // CDF_k = (totals of the earlier blocks h) + (prefix within block h)
    float T[3], run[3];
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      T[h] = row_sum(ex[h]);
      run[h] = row_scan(ex[h]);
    }
    run[1] = T[0] + run[1];
    run[2] = (T[0] + T[1]) + run[2];
    const float S = (T[0] + T[1]) + T[2];
    // first k with u < CDF_k, as u * S < (sum of e up to k)
    const float uS = u * S;
    int cand = 64;
#pragma unroll
    for (int h = 2; h >= 0; --h)
      if (ok[h] && uS < run[h]) cand = j + 16 * h;
    int act_a = row_min_i(cand);
    if (act_a == 64) {  // rounding left u >= CDF_44: last action with weight
      int lastk = -1;
#pragma unroll
      for (int h = 0; h < 3; ++h)
        if (ok[h] && ex[h] > 0.0f) lastk = j + 16 * h;
      lastk = row_max_i(lastk);
      act_a = lastk >= 0 ? lastk : kActions - 1;
    }
    float la = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (j + 16 * h == act_a) la = l[h];
    la = row_max(la);
    const float logp = (la - m) - logf(S);
    bad = row_max_i(bad);

    // ---- step 6: portfolio (exposure fraction of equity, turnover cost) ---
    const int xi = act_a / 9;
    const int oi = (act_a % 9) / 3;
    const int ui = act_a % 3;
    const float exq = s_env[xi];
    const float cost = s_env[5 + oi] * (1.0f + ep.urgency_mult * (float)ui);
    const float ret = p1 / p0 - 1.0f;
    const float pnl = exq * ret - cost * fabsf(exq - e_prev);
    V = V * (1.0f + pnl);

    // ---- step 7: triple barrier on raw prices ------------------------------
    if (exq != 0.0f) {
      const int sd = exq > 0.0f ? 1 : -1;
      const int prev = e_prev > 0.0f ? 1 : (e_prev < 0.0f ? -1 : 0);
      if (prev == 0 || prev != sd) {
        armed = 1;
        side = sd;
        entry = p0;
        t_open = t;
      }
    } else {
      armed = 0;
    }
    int hit = 0, code = 0;
    if (armed) {
      if (side > 0) {
        if (p1 >= entry * ep.up_pt) { hit = 1; code = 1; }
        else if (p1 <= entry * ep.dn_sl) { hit = -1; code = 2; }
      } else {
        if (p1 <= entry * ep.dn_pt) { hit = 1; code = 1; }
        else if (p1 >= entry * ep.up_sl) { hit = -1; code = 2; }
      }
      if (code == 0 && t + 1 - t_open >= ep.max_hold) code = 3;
    }

    // ---- step 8: diversity window, 3-class entropy in nats -----------------
    // H = ln n - (sum_c n_c ln n_c) / n, compared as n ln n - sum n_c ln n_c
    // < threshold * n; ln of the counts 0..32 comes from an LDS table
    const int cat = xi <= 1 ? 0 : (xi == 2 ? 1 : 2);
    if (pushed >= ep.div_window) {
      const int old = (int)((ring >> (2 * pos)) & 3u);
      cnt0 -= old == 0; cnt1 -= old == 1; cnt2 -= old == 2;
    }
    ring = (ring & ~(3ull << (2 * pos))) | ((uint64_t)cat << (2 * pos));
    cnt0 += cat == 0; cnt1 += cat == 1; cnt2 += cat == 2;
    ++pushed;
    pos = pos + 1 == ep.div_window ? 0 : pos + 1;
    const int nn = cnt0 + cnt1 + cnt2;
    const float hn = (float)nn * s_ln[nn] -
                     (((float)cnt0 * s_ln[cnt0] + (float)cnt1 * s_ln[cnt1]) + (float)cnt2 * s_ln[cnt2]);
    const float div = hn < ep.div_threshold * (float)nn ? ep.div_penalty : 0.0f;

    // ---- steps 10-11: partial reward and stores (lane 0 of the row) -------
    const float partial = pnl * (1.0f + ep.barrier_scale * (float)hit) + div;
    const int done = code != 0;
    if (valid) {
      if (j == 0) {
        a.actions[o] = act_a;
        a.log_probs[o] = logp;
        a.rewards[o] = partial;
        a.dones[o] = (uint8_t)done;
        a.barrier[o] = (uint8_t)code;
        if (bad && a.counters) atomicAdd(a.counters, 1u);
      }
      if (a.logits) {
        float* lrow = a.logits + o * kActions;
#pragma unroll
        for (int h = 0; h < 3; ++h)
          if (ok[h]) lrow[j + 16 * h] = l[h];
      }
    }

    // ---- step 12: reset on done; the bar pointer keeps advancing ------------
    e_prev = exq;
    if (done) {
      V = 1.0f;
      e_prev = 0.0f;
      armed = 0;
      cnt0 = cnt1 = cnt2 = 0;
      pushed = 0;
      pos = 0;
      ring = 0;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) fcur[h] = fnext[h];
    p0 = p1;
    p1 = p2;
  }
}

}  // namespace

hipError_t launch_actor_rollout(const RolloutArgs& a, hipStream_t st) {
  if (a.N <= 0 || a.L <= 0) return hipSuccess;
  // two 16-episode groups per workgroup once there are enough episodes to
  // fill every CU with one workgroup; otherwise one group, spread wider
  const bool two = a.N >= 2 * 16 * 256;
  const unsigned blocks = (unsigned)(two ? (a.N + 31) / 32 : (a.N + 15) / 16);
  const dim3 block(64 * kSplit * (two ? 2 : 1));
  if (two && a.bf16)
    hipLaunchKernelGGL((actor_rollout_kernel<2, true>), dim3(blocks), block, 0, st, a);
  else if (two)
    hipLaunchKernelGGL((actor_rollout_kernel<2, false>), dim3(blocks), block, 0, st, a);
  else if (a.bf16)
    hipLaunchKernelGGL((actor_rollout_kernel<1, true>), dim3(blocks), block, 0, st, a);
  else
    hipLaunchKernelGGL((actor_rollout_kernel<1, false>), dim3(blocks), block, 0, st, a);
  return hipGetLastError();
}

}  // namespace rl
