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
// MFMA output layout: lane l holds logits 16*ot + 4*(l/16) + r of episode
// l%16, so each episode's 45 logits sit in the 4 lanes l%16 + 16*g once the
// three logit tiles are gathered from LDS.  All per-episode scalars (draw,
// portfolio, barrier, window) are computed redundantly by those 4 lanes in
// each of the 4 waves, so no broadcast is needed; wave 0 stores.
#include "collect.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
constexpr int64_t kActorF32 = kP.actor_end;                  // fp32 actor block (floats)
constexpr int64_t kActorBF16 = kP.bact_end - kP.bact_begin;  // bf16 actor block (floats)
constexpr int kActorF4 = (int)((kActorF32 > kActorBF16 ? kActorF32 : kActorBF16) / 4);
constexpr int kBufF4 = 8 * 64;  // widest actor activation: 128 = 8 tiles

// The features a lane feeds to the first layer (its 16 state slots).
template <bool BF16>
__device__ __forceinline__ void load_features(const float* __restrict__ F, int64_t bar, int g,
                                              float (&f)[16]) {
  const float* row = F + bar * kFeatures;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int k = state_k<BF16>(g, s);
    f[s] = k < kFeatures ? row[k] : 0.0f;
  }
}

template <int RG, bool BF16>
__global__ __launch_bounds__(64 * kSplit * RG) void actor_rollout_kernel(RolloutArgs a) {
  __shared__ f32x4 s_w[kActorF4];
  __shared__ f32x4 s_buf[RG][kBufF4];
  __shared__ f32x4 s_state[RG][4 * 64];
  __shared__ float s_ln[33];  // ln k for window counts k = 0..32 (ln 0 unused: times 0)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / kSplit;
  const int q = wave % kSplit;
  const int g = lane >> 4;

  if (threadIdx.x <= 32) s_ln[threadIdx.x] = threadIdx.x == 0 ? 0.0f : logf((float)threadIdx.x);
  {  // stage the packed actor (fp32 or bf16 block) into LDS
    const int64_t begin = BF16 ? kP.bact_begin : 0;
    const int n4 = (int)((BF16 ? kActorBF16 : kActorF32) / 4);
    const f32x4* src = reinterpret_cast<const f32x4*>(a.weights + begin);
    for (int i = threadIdx.x; i < n4; i += 64 * kSplit * RG) s_w[i] = src[i];
  }

  const int32_t n_raw = (blockIdx.x * RG + rg) * kRowsPerWave + (lane & 15);
  const bool valid = n_raw < a.N;
  const int32_t n = valid ? n_raw : a.N - 1;
  const bool writer = valid && q == 0;
  const EnvParams& ep = a.ep;

  // clamp the start so every read stays inside the market buffers
  const int64_t hi = a.n_bars - (int64_t)a.L - 1;
  int64_t st = a.starts[n];
  const bool clamped = st < 0 || st > hi;
  st = st < 0 ? 0 : (st > hi ? hi : st);
  if (writer && g == 0) {
    a.start_used[n] = (int32_t)st;
    if (clamped && a.counters) atomicAdd(a.counters + 1, 1u);
  }

  const float* sw = reinterpret_cast<const float*>(s_w);
  f32x4* buf = s_buf[rg];
  f32x4* sbuf = s_state[rg];

  float fcur[16];
  load_features<BF16>(a.features, st, g, fcur);
  float p0 = a.prices[st], p1 = a.prices[st + 1];

  // episode state (PPO CUDA Pipeline Design, Phase A steps 6-8, 12), held
  // identically by the 4 lanes of the episode in each of the 4 waves
  float V = 1.0f, e_prev = 0.0f, entry = 0.0f;
  int armed = 0, side = 0, t_open = 0;
  int cnt0 = 0, cnt1 = 0, cnt2 = 0, pushed = 0, pos = 0;
  uint64_t ring = 0;  // 2 bits per window slot
  const float V0 = 1.0f;
  lds_barrier();  // weights staged

  for (int32_t t = 0; t < a.L; ++t) {
    const int64_t bar = st + t;
    const int64_t o = (int64_t)t * a.N + n;

    // ---- steps 1-2: state, as this lane's 16 first-layer slots -----------
    // features k < 51, then V/V0 - 1, the exposure held and the spread
    const float vn = V / V0 - 1.0f;
    float B[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int k = state_k<BF16>(g, s);
      B[s] = k < kFeatures ? fcur[s]
                           : (k == 51 ? vn : (k == 52 ? e_prev : (k == 53 ? ep.spread : 0.0f)));
    }
    if (q == 0) {
      store_state_operands<BF16>(B, sbuf, lane);
      if (valid) {
        float* srow = a.states + o * kState;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int k = state_k<BF16>(g, s);
          if (k < kState) srow[k] = B[s];
        }
      }
    }

    // prefetch the next bar (independent of this step's outcome)
    float fnext[16];
    float p2 = p1;
    if (t + 1 < a.L) {
      load_features<BF16>(a.features, bar + 1, g, fnext);
      p2 = a.prices[bar + 2];
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) fnext[s] = fcur[s];
    }
    lds_barrier();  // state operands written

    // the step's draw depends only on (seed, episode, step)
    const float u = draw_uniform(a.seed, (uint32_t)n, (uint32_t)t, 0u);

    // ---- step 3: actor, a quarter of each layer per wave ------------------
    {
      f32x4 h[2];
      if constexpr (BF16) {
        mfma_layer_bf16<2, 2>(reinterpret_cast<const uint4*>(sw + kP.bact_w[0] - kP.bact_begin),
                              sw + kP.bact_b[0] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(sbuf), h, q, lane);
        relu_store_bf16<2>(h, reinterpret_cast<uint4*>(buf), q, lane);
      } else {
        mfma_layer<16, 2>(sw + kP.actor_w[0], sw + kP.actor_b[0], sbuf, h, q, lane);
        relu_store<2>(h, buf, q, lane);  // buf is free: last read before the previous barrier
      }
    }
    lds_barrier();
    {
      f32x4 h[1];
      if constexpr (BF16) {
        mfma_layer_bf16<4, 1>(reinterpret_cast<const uint4*>(sw + kP.bact_w[1] - kP.bact_begin),
                              sw + kP.bact_b[1] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(buf), h, q, lane);
        lds_barrier();
        relu_store_bf16<1>(h, reinterpret_cast<uint4*>(buf), q, lane);
      } else {
        mfma_layer<32, 1>(sw + kP.actor_w[1], sw + kP.actor_b[1], buf, h, q, lane);
        lds_barrier();
        relu_store<1>(h, buf, q, lane);
      }
    }
    lds_barrier();
    {
      f32x4 h[1];
      if constexpr (BF16)
        mfma_layer_bf16<2, 1>(reinterpret_cast<const uint4*>(sw + kP.bact_w[2] - kP.bact_begin),
                              sw + kP.bact_b[2] - kP.bact_begin,
                              reinterpret_cast<const uint4*>(buf), h, q, lane);
      else
        mfma_layer<16, 1>(sw + kP.actor_w[2], sw + kP.actor_b[2], buf, h, q, lane);
      lds_barrier();
      buf[q * 64 + lane] = h[0];  // raw logits, fp32 (tile 3 is padding)
    }
    lds_barrier();

    // ---- step 4: softmax, CDF, inverse-CDF draw, log-prob (every wave) ----
    // The 4 lanes of an episode hold logit tiles ot = 0..2 as groups g:
    // index k = 16 ot + 4 g + r.  Cross-lane steps use lane swaps; sums over
    // the 4 lanes are butterflies (b_g + b_g^1) + (b_g^2 + b_g^3), the same
    // bits in every lane.
    float l[12], e[12];
    bool ok[12];
    int bad = 0;
#pragma unroll
    for (int ot = 0; ot < 3; ++ot) {
      const f32x4 lv = buf[ot * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * ot + r;
        ok[i] = 16 * ot + 4 * g + r < kActions;
        l[i] = lv[r];
        if (ok[i] && !isfinite(l[i])) bad = 1;
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 12; ++i)
      if (ok[i]) m = fmaxf(m, l[i]);
    m = fmaxf(m, lane_xor16f(m, lane));
    m = fmaxf(m, lane_xor32f(m, lane));
#pragma unroll
    for (int i = 0; i < 12; ++i) e[i] = ok[i] ? expf(l[i] - m) : 0.0f;
    // block sums of the 4 groups of each tile, by absolute group index
    float T[3], pre[3];
#pragma unroll
    for (int ot = 0; ot < 3; ++ot) {
      const float bs = ((e[4 * ot] + e[4 * ot + 1]) + e[4 * ot + 2]) + e[4 * ot + 3];
      const float p16 = lane_xor16f(bs, lane);  // group g ^ 1
      const float p32 = lane_xor32f(bs, lane);  // group g ^ 2
      const float p48 = lane_xor16f(p32, lane); // group g ^ 3
      T[ot] = (bs + p16) + (p32 + p48);
      const float b0 = g == 0 ? bs : (g == 1 ? p16 : (g == 2 ? p32 : p48));
      const float b1 = g == 1 ? bs : (g == 0 ? p16 : (g == 3 ? p32 : p48));
      const float b2 = g == 2 ? bs : (g == 3 ? p16 : (g == 0 ? p32 : p48));
      pre[ot] = g == 0 ? 0.0f : (g == 1 ? b0 : (g == 2 ? b0 + b1 : (b0 + b1) + b2));
    }
    const float S = (T[0] + T[1]) + T[2];
    // first k with u < CDF_k, as u * S < (sum of e up to k)
    const float uS = u * S;
    int first = 64;
    float before = 0.0f;
#pragma unroll
    for (int ot = 0; ot < 3; ++ot) {
      float run = before + pre[ot];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        run += e[4 * ot + r];
        const int k = 16 * ot + 4 * g + r;
        if (ok[4 * ot + r] && first == 64 && uS < run) first = k;
      }
      before += T[ot];
    }
    int act_a = min(first, (int)lane_xor16((uint32_t)first, lane));
    act_a = min(act_a, (int)lane_xor32((uint32_t)act_a, lane));
    if (act_a == 64) {  // rounding left u >= CDF_44: last action with weight
      int lastk = -1;
#pragma unroll
      for (int ot = 0; ot < 3; ++ot)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ok[4 * ot + r] && e[4 * ot + r] > 0.0f) lastk = max(lastk, 16 * ot + 4 * g + r);
      lastk = max(lastk, (int)lane_xor16((uint32_t)lastk, lane));
      lastk = max(lastk, (int)lane_xor32((uint32_t)lastk, lane));
      act_a = lastk >= 0 ? lastk : kActions - 1;
    }
    float la = -INFINITY;
#pragma unroll
    for (int ot = 0; ot < 3; ++ot)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * ot + 4 * g + r == act_a) la = l[4 * ot + r];
    la = fmaxf(la, lane_xor16f(la, lane));
    la = fmaxf(la, lane_xor32f(la, lane));
    const float logp = (la - m) - logf(S);
    bad |= (int)lane_xor16((uint32_t)bad, lane);
    bad |= (int)lane_xor32((uint32_t)bad, lane);

    // ---- step 6: portfolio (exposure fraction of equity, turnover cost) ---
    const int xi = act_a / 9;
    const int oi = (act_a % 9) / 3;
    const int ui = act_a % 3;
    const float ex = exposure_of(ep, xi);
    const float cost = cost_of(ep, oi) * (1.0f + ep.urgency_mult * (float)ui);
    const float ret = p1 / p0 - 1.0f;
    const float pnl = ex * ret - cost * fabsf(ex - e_prev);
    V = V * (1.0f + pnl);

    // ---- step 7: triple barrier on raw prices ------------------------------
    if (ex != 0.0f) {
      const int sd = ex > 0.0f ? 1 : -1;
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

    // ---- steps 10-11: partial reward and stores ----------------------------
    const float partial = pnl * (1.0f + ep.barrier_scale * (float)hit) + div;
    const int done = code != 0;
    if (writer) {
      if (g == 0) {
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
        for (int ot = 0; ot < 3; ++ot)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (ok[4 * ot + r]) lrow[16 * ot + 4 * g + r] = l[4 * ot + r];
      }
    }

    // ---- step 12: reset on done; the bar pointer keeps advancing ------------
    e_prev = ex;
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
    for (int s = 0; s < 16; ++s) fcur[s] = fnext[s];
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
