// DQN experience collection ("GPU Pipeline Phase 2b: Zero-Roundtrip CUDA
// Experience Collection", Data Flow steps 1-15 and Kernel Components 1-8):
// N independent episodes advance L steps in one launch.  Per step and
// episode:
//   - the 54-wide state (51 features of the bar, V/V0 - 1, the exposure
//     held, the spread), stored (steps 1-3);
//   - the online dueling Q-network on it (step 4): trunk 54 -> 256 -> 128,
//     value head 128 -> 64 -> 1, advantage head 128 -> 64 -> 45,
//     Q = V + (A - mean A);
//   - epsilon-greedy (step 5): a counter-based draw (stream 1) below epsilon
//     takes a uniformly random action floor(45 u) from a second draw
//     (stream 2), else the greedy action (lowest index among equal maxima);
//   - portfolio, triple barrier, diversity window and curiosity bonus, and
//     the reward, exactly as in the PPO collection (steps 6-9, 13);
//   - the next state (bar + 1, the portfolio after the trade, before any
//     reset), the target network's Q on it and
//     TD = r + gamma (1 - done) max Q_target - Q_online(s, a), with
//     priority |TD|^alpha (steps 10-12, "GPU-Resident Prioritized
//     Experience Replay", Sampling Kernels, priority update);
//   - the stores and the reset on done (steps 14-15); with recycling the
//     episode then restarts at a fresh random bar (Future Phase 3
//     Optimization) instead of running on.
//
// Mapping: a workgroup of four waves owns 16 episodes for all L steps.  The
// layers run on MFMA (v_mfma_f32_16x16x4_f32, lane l computes rows l % 16);
// each wave computes a quarter of every layer's output tiles, streaming its
// weights from L2 through buffer loads (the ten layers' 0.66 MB do not fit
// in LDS), with activations shared through LDS.  The per-episode work uses
// rows of 16 lanes: wave q owns episodes 4q .. 4q+3, lane j of a row holds
// outputs j, j + 16, j + 32, so the dueling mean, the argmax and the MSE are
// DPP reductions within the row, and every lane of a row holds the
// episode's environment state.
#include "collect.hpp"
#include "rows.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr DqnOffsets kD = dqn_packed_offsets();
constexpr int kOpnd = 4 * 64;   // first-layer operands: 4 groups of 4 k-steps x 64 lanes
constexpr int kBufA = 16 * 64;  // widest layer output: 256 = 16 tiles
constexpr int kBufB = 8 * 64;   // 128 = 8 tiles
constexpr int kBufC = 4 * 64;   // curiosity prediction: 64 = 4 tiles

// One streamed layer of 16 rows: this wave's OTW output tiles, bias
// included, B operands from the LDS operand layout.  With four workgroups
// per CU the weight ring needs fewer steps in flight than the value
// kernel's: 4 steps for 4 tiles per wave, 8 otherwise.
template <int S, int OTW, int SK = S>
__device__ __forceinline__ void dense(const GlobalWeights& gw, uint32_t pk_b, const float* pb,
                                      const f32x4* in, f32x4 (&acc)[1][OTW], int q, int lane) {
  constexpr int D = OTW >= 4 ? 4 : 8;
  WeightStream<false, OTW, D> st;
  stream_begin<S>(st, gw, pk_b, pb, q, lane);
  stream_layer<S, OTW, D, 1, SK>(st, gw, pk_b, LdsOperands{in, 0}, acc, q, lane);
}

// Dueling Q-network `net` (0 online, 1 target) on the state operands `in`:
// the head layer's raw outputs (advantages 0..44, value 45) end in bufB.
// Entry: `in` complete, bufA and bufB free; exit: before any barrier.  Each
// layer's weight stream starts before the store and barrier that end the
// previous layer, so its first loads are in flight while the waves meet.
// The head layer skips its zero blocks: output tiles 0-1 (advantages 0..31)
// read only inputs 64..127 (k-steps 16..31), tile 2 (advantages 32..44 and
// the value) reads all, and tile 3 holds only padding.
__device__ __forceinline__ void q_network(const GlobalWeights& gw, const float* W, int net,
                                          const f32x4* in, f32x4* bufA, f32x4* bufB, int q,
                                          int lane) {
  constexpr uint32_t kHeadStepB = kSplit * 64 * 4;  // bytes per k-step, one tile per wave
  const uint32_t w0 = 4u * (uint32_t)kD.w[net][0], w1 = 4u * (uint32_t)kD.w[net][1];
  const uint32_t w2 = 4u * (uint32_t)kD.w[net][2], w3 = 4u * (uint32_t)kD.w[net][3];
  WeightStream<false, 4, 4> s0;
  stream_begin<16>(s0, gw, w0, W + kD.b[net][0], q, lane);
  f32x4 h0[1][4];
  stream_layer<16, 4, 4, 1, 14>(s0, gw, w0, LdsOperands{in, 0}, h0, q, lane);  // 2 padding steps
  WeightStream<false, 2, 8> s1;
  stream_begin<64>(s1, gw, w1, W + kD.b[net][1], q, lane);
  relu_store_tiles<4, 1>(h0, bufA, 0, q, lane);
  lds_barrier();
  f32x4 h1[1][2];
  stream_layer<64, 2, 8, 1>(s1, gw, w1, LdsOperands{bufA, 0}, h1, q, lane);
  WeightStream<false, 2, 8> s2;
  stream_begin<32>(s2, gw, w2, W + kD.b[net][2], q, lane);
  relu_store_tiles<2, 1>(h1, bufB, 0, q, lane);
  lds_barrier();
  f32x4 h2[1][2];
  stream_layer<32, 2, 8, 1>(s2, gw, w2, LdsOperands{bufB, 0}, h2, q, lane);
  WeightStream<false, 1, 8> s3;
  // (wave-uniform: as an SGPR it is the loads' scalar offset, not a per-lane
  // value the compiler would loop over)
  const uint32_t w3q = __builtin_amdgcn_readfirstlane(q < 2 ? w3 + 16u * kHeadStepB : w3);
  stream_begin<16>(s3, gw, w3q, W + kD.b[net][3], q, lane);
  relu_store_tiles<2, 1>(h2, bufA, 0, q, lane);
  lds_barrier();
  f32x4 h3[1][1];
  if (q < 2) {
    stream_layer<16, 1, 8, 1>(s3, gw, w3q, LdsOperands{bufA + 4 * 64, 0}, h3, q, lane);
    bufB[q * 64 + lane] = h3[0][0];
  } else if (q == 2) {
    stream_layer<32, 1, 8, 1>(s3, gw, w3, LdsOperands{bufA, 0}, h3, q, lane);
    bufB[q * 64 + lane] = h3[0][0];  // raw: no ReLU on the head outputs
  }
}

// Output k of episode row e of a layer stored in the MFMA layout.
__device__ __forceinline__ float row_output(const f32x4* buf, int e, int k) {
  return reinterpret_cast<const float*>(buf)[((k >> 4) * 64 + e + 16 * ((k & 15) >> 2)) * 4 + (k & 3)];
}

// Q-values of episode row e from the head outputs: lane j holds actions
// j + 16 h (h = 0..2, valid when < 45); Q = V + (A - mean A), the mean a
// row sum over the 45 advantages divided by 45.
__device__ __forceinline__ void dueling_q(const f32x4* buf, int e, int j, float (&Q)[3],
                                          bool (&ok)[3]) {
  float A[3];
#pragma unroll
  for (int h = 0; h < 3; ++h) {
    ok[h] = j + 16 * h < kActions;
    A[h] = ok[h] ? row_output(buf, e, j + 16 * h) : 0.0f;
  }
  const float V = row_output(buf, e, kQValueRow);
  const float mean = row_sum((A[0] + A[1]) + A[2]) / (float)kActions;
#pragma unroll
  for (int h = 0; h < 3; ++h) Q[h] = V + (A[h] - mean);
}

template <bool RECYCLE>
__global__ __launch_bounds__(64 * kSplit) __attribute__((amdgpu_waves_per_eu(4))) void dqn_collect_kernel(DqnArgs a) {
  __shared__ f32x4 s_opnd[kOpnd];  // state of the step
  __shared__ f32x4 s_next[kOpnd];  // next state (target network input)
  __shared__ f32x4 s_bufA[kBufA];
  __shared__ f32x4 s_bufB[kBufB];
  __shared__ f32x4 s_bufC[kBufC];
  __shared__ float s_ln[33];  // ln k for window counts k = 0..32
  __shared__ int s_act[kRowsPerWave];

  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;

  if (threadIdx.x <= 32) s_ln[threadIdx.x] = threadIdx.x == 0 ? 0.0f : logf((float)threadIdx.x);
  // operands start at zero: the padding slots (k >= 54) stay zero
  s_opnd[threadIdx.x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  s_next[threadIdx.x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // episode rows: wave q owns episodes 4q .. 4q+3, 16 lanes each
  const int e = 4 * q + (lane >> 4);
  const int j = lane & 15;
  const int32_t n_raw = blockIdx.x * kRowsPerWave + e;
  const bool valid = n_raw < a.N;
  const int32_t n = valid ? n_raw : a.N - 1;
  const EnvParams& ep = a.ep;

  // clamp the start so every read stays inside the market buffers
  const int64_t hi = a.n_bars - (int64_t)a.L - 1;
  int64_t st = a.starts[n];
  const bool clamped = st < 0 || st > hi;
  st = st < 0 ? 0 : (st > hi ? hi : st);
  if (valid && j == 0 && clamped && a.counters) atomicAdd(a.counters + 1, 1u);

  float f0[4], f1[4];
  load_features(a.features, st, j, f0);
  load_features(a.features, st + 1, j, f1);
  float p0 = a.prices[st], p1 = a.prices[st + 1];

  // episode state ("GPU Pipeline Phase 2b", Kernel Components 3-5)
  float V = 1.0f, e_prev = 0.0f, entry = 0.0f;
  int armed = 0, side = 0, t_open = 0;
  int cnt0 = 0, cnt1 = 0, cnt2 = 0, pushed = 0, pos = 0;
  uint64_t ring = 0;  // 2 bits per window slot
  const float V0 = 1.0f;

  lds_barrier();  // operand buffers cleared
  if (j == 2) {
    put_state<false>(s_opnd, e, 53, ep.spread);
    put_state<false>(s_next, e, 53, ep.spread);
  }
#pragma unroll
  for (int h = 0; h < 4; ++h)
    if (j + 16 * h < kFeatures) put_state<false>(s_opnd, e, j + 16 * h, f0[h]);
  if (j == 0) put_state<false>(s_opnd, e, 51, 0.0f);
  if (j == 1) put_state<false>(s_opnd, e, 52, 0.0f);

  int64_t bar = st;
  // the step's two draws (and, recycling, its restart bar), 16 steps at a
  // time per episode row
  RowDraws ue_pool, ua_pool, rb_pool;
#pragma unroll 1
  for (int32_t t = 0; t < a.L; ++t) {
    const int64_t o = (int64_t)t * a.N + n;
    const int slot16 = t & 15;
    if (slot16 == 0) {
      const int32_t tj = t + (int)(threadIdx.x & 15);
      ue_pool.pool = __float_as_uint(draw_uniform(a.seed, (uint32_t)n, (uint32_t)tj, 1u));
      ua_pool.pool = __float_as_uint(draw_uniform(a.seed, (uint32_t)n, (uint32_t)tj, 2u));
      if constexpr (RECYCLE)
        rb_pool.pool = tj + 1 < a.L ? (uint32_t)recycle_bar(a.seed, (uint32_t)n, tj, a.L, a.n_bars) : 0u;
    }

    // the weights are the same every step: an opaque zero offset keeps the
    // compiler from hoisting their loads (and registers) out of the loop
    int32_t opaque0 = 0;
    asm volatile("" : "+s"(opaque0));
    const float* W = a.weights + opaque0;
    const GlobalWeights gw{weights_rsrc(W, (uint32_t)(4 * kD.total))};
    // an opaque copy of the thread index: the LDS and weight addresses of
    // the layers are recomputed each step instead of held in registers
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int q = tid >> 6;
    const int e = 4 * q + (lane >> 4);
    const int j = lane & 15;


    // ---- steps 1-3: the state (its operands were written last step) -------
    if (valid) {
      float* srow = a.states + o * kState;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (j + 16 * h < kFeatures) srow[j + 16 * h] = f0[h];
      if (j < 3) srow[kFeatures + j] = j == 0 ? V / V0 - 1.0f : (j == 1 ? e_prev : ep.spread);
    }
    lds_barrier();  // state operands complete

    // ---- step 4: online Q --------------------------------------------------
    q_network(gw, W, 0, s_opnd, s_bufA, s_bufB, q, lane);
    lds_barrier();

    // Market rows loaded here, where the row work below (no weight loads)
    // covers their latency before the target network's first weight wait
    // (the memory counter is in order; at the top of the step the online
    // network's weight waits waited for them): the bar two ahead
    // (independent of the outcomes) and, with recycling, the restart bar
    // this step would take if the episode ended, and its first two bars.
    float f2[4];
    load_features(a.features, bar + 2 < a.n_bars ? bar + 2 : a.n_bars - 1, j, f2);
    const float p2 = a.prices[bar + 2 < a.n_bars ? bar + 2 : a.n_bars - 1];
    int64_t rbar = 0;
    float fr0[4], fr1[4], pr0 = 0.0f, pr1 = 0.0f;
    if constexpr (RECYCLE) {
      rbar = t + 1 < a.L ? (int64_t)rb_pool.take(slot16, lane) : bar;
      load_features(a.features, rbar, j, fr0);
      load_features(a.features, rbar + 1, j, fr1);
      pr0 = a.prices[rbar];
      pr1 = a.prices[rbar + 1];
    }

    // The row work (epsilon-greedy and the environment here, the TD and the
    // stores below) runs at a raised wave priority and the networks at the
    // base one: where the four workgroups of a CU meet, the one doing its
    // short row work issues first and returns to its weight stream sooner.
    __builtin_amdgcn_s_setprio(2);
    // ---- step 5: epsilon-greedy on the episode rows -------------------------
    float Q[3];
    bool ok[3];
    dueling_q(s_bufB, e, j, Q, ok);
    int bad = 0;
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (ok[h]) {
        bad |= !isfinite(Q[h]);
        mx = fmaxf(mx, Q[h]);
      }
    mx = row_max(mx);
    int greedy = 64;
#pragma unroll
    for (int h = 2; h >= 0; --h)
      if (ok[h] && Q[h] == mx) greedy = j + 16 * h;
    greedy = row_min_i(greedy);
    if (greedy >= kActions) greedy = 0;  // every Q non-finite (counted below)
    const float u_explore = __uint_as_float(ue_pool.take(slot16, lane));
    const float u_action = __uint_as_float(ua_pool.take(slot16, lane));
    const bool explore = u_explore < a.epsilon;
    // u = m 2^-24 with m < 2^24: floor(45 u) = (45 m) >> 24, exactly
    const int random_a = (int)(((uint32_t)(u_action * 16777216.0f) * (uint32_t)kActions) >> 24);
    const int act = explore ? random_a : greedy;
    float qa = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (j + 16 * h == act) qa = Q[h];
    const float q_taken = row_max(qa);
    if (valid && a.q_values) {
      float* qrow = a.q_values + o * kActions;
#pragma unroll
      for (int h = 0; h < 3; ++h)
        if (ok[h]) qrow[j + 16 * h] = Q[h];
    }

    // ---- step 6: portfolio (exposure fraction of equity, turnover cost) ---
    const int xi = act / 9;
    const int oi = (act % 9) / 3;
    const int ui = act % 3;
    // the exposure and cost-rate tables by selects on the kernel arguments
    float exq = ep.ex0, rate = ep.cost0;
    exq = xi == 1 ? ep.ex1 : exq;
    exq = xi == 2 ? ep.ex2 : exq;
    exq = xi == 3 ? ep.ex3 : exq;
    exq = xi == 4 ? ep.ex4 : exq;
    rate = oi == 1 ? ep.cost1 : rate;
    rate = oi == 2 ? ep.cost2 : rate;
    const float cost = rate * (1.0f + ep.urgency_mult * (float)ui);
    const float ret = p1 / p0 - 1.0f;
    const float pnl = exq * ret - cost * fabsf(exq - e_prev);
    V = V * (1.0f + pnl);

    // ---- step 7: triple barrier on raw prices (selects, no branches) -------
    {
      const int sd = exq > 0.0f ? 1 : -1;
      const int prev = e_prev > 0.0f ? 1 : (e_prev < 0.0f ? -1 : 0);
      // a position opens, or flips side: the barriers are set at this bar
      const bool open = exq != 0.0f && (prev == 0 || prev != sd);
      armed = exq != 0.0f ? (open ? 1 : armed) : 0;
      side = open ? sd : side;
      entry = open ? p0 : entry;
      t_open = open ? t : t_open;
    }
    const bool lng = side > 0;
    const float take_px = entry * (lng ? ep.up_pt : ep.dn_pt);
    const float stop_px = entry * (lng ? ep.dn_sl : ep.up_sl);
    const bool take = lng ? p1 >= take_px : p1 <= take_px;
    const bool stop = lng ? p1 <= stop_px : p1 >= stop_px;
    const bool expire = t + 1 - t_open >= ep.max_hold;
    const int hit = armed ? (take ? 1 : (stop ? -1 : 0)) : 0;
    const int code = armed ? (take ? 1 : (stop ? 2 : (expire ? 3 : 0))) : 0;
    const int done = code != 0;

    // ---- step 8: diversity window, 3-class entropy in nats -----------------
    // H = ln n - (sum_c n_c ln n_c) / n, compared as n ln n - sum n_c ln n_c
    // < threshold * n
    const int cat = xi <= 1 ? 0 : (xi == 2 ? 1 : 2);
    {
      // a full window drops its oldest entry, the one this slot holds
      const bool full = pushed >= ep.div_window;
      const int old = (int)((ring >> (2 * pos)) & 3u);
      cnt0 += (cat == 0) - (full && old == 0);
      cnt1 += (cat == 1) - (full && old == 1);
      cnt2 += (cat == 2) - (full && old == 2);
    }
    ring = (ring & ~(3ull << (2 * pos))) | ((uint64_t)cat << (2 * pos));
    ++pushed;
    pos = pos + 1 == ep.div_window ? 0 : pos + 1;
    const int nn = cnt0 + cnt1 + cnt2;
    const float hn = (float)nn * s_ln[nn] -
                     (((float)cnt0 * s_ln[cnt0] + (float)cnt1 * s_ln[cnt1]) + (float)cnt2 * s_ln[cnt2]);
    const float div = hn < ep.div_threshold * (float)nn ? ep.div_penalty : 0.0f;
    e_prev = exq;

    // ---- step 10: the next state, before any reset ---------------------------
    const float vn_next = V / V0 - 1.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (j + 16 * h < kFeatures) put_state<false>(s_next, e, j + 16 * h, f1[h]);
    if (j == 0) put_state<false>(s_next, e, 51, vn_next);
    if (j == 1) put_state<false>(s_next, e, 52, exq);
    if (valid && a.next_states) {
      float* nrow = a.next_states + o * kState;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (j + 16 * h < kFeatures) nrow[j + 16 * h] = f1[h];
      if (j < 3) nrow[kFeatures + j] = j == 0 ? vn_next : (j == 1 ? exq : ep.spread);
    }
    if (j == 0) s_act[e] = act;
    lds_barrier();

    __builtin_amdgcn_s_setprio(0);
    // ---- step 11: target Q of the next state --------------------------------
    q_network(gw, W, 1, s_next, s_bufA, s_bufB, q, lane);
    lds_barrier();  // every wave is done reading bufA

    // ---- step 9: curiosity on [state, one-hot(action)] ----------------------
    {
      f32x4 h[1][2];
      dense<16, 2, 14>(gw, 4u * (uint32_t)kD.cw[0], W + kD.cb[0], s_opnd, h, q, lane);
      // the one-hot half of the input is a column gather: + W[:, 54 + a]
      const int ra = s_act[lane & 15];
      const float* oh = W + kD.c_onehot + ra * 128 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        h[0][i] += *reinterpret_cast<const f32x4*>(oh + 16 * (q * 2 + i));
      relu_store_tiles<2, 1>(h, s_bufA, 0, q, lane);
    }
    lds_barrier();
    {
      f32x4 h[1][1];
      dense<32, 1>(gw, 4u * (uint32_t)kD.cw[1], W + kD.cb[1], s_bufA, h, q, lane);
      s_bufC[q * 64 + lane] = h[0][0];
    }
    lds_barrier();

    __builtin_amdgcn_s_setprio(2);
    // ---- steps 12-14: target max, curiosity bonus, reward, TD, stores ------
    float Qt[3];
    bool okt[3];
    dueling_q(s_bufB, e, j, Qt, okt);
    float qmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (okt[h]) qmax = fmaxf(qmax, Qt[h]);
    qmax = row_max(qmax);
    float se = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int k = j + 16 * h;
      const float d = k < kFeatures ? row_output(s_bufC, e, k) - f1[h] : 0.0f;
      se = se + d * d;
    }
    se = row_sum(se);
    const float bonus = ep.curiosity_coef * (se / (float)kFeatures);
    const float reward = ((pnl * (1.0f + ep.barrier_scale * (float)hit) + div) + bonus) -
                         ep.risk_coef * fabsf(exq);
    const float td = (reward + (a.gamma * qmax) * (float)(1 - done)) - q_taken;
    bad = row_max_i(bad | !isfinite(reward) | !isfinite(td));
    if (valid && j == 0) {
      a.actions[o] = act;
      a.q_taken[o] = q_taken;
      a.q_next_max[o] = qmax;
      a.rewards[o] = reward;
      a.dones[o] = (uint8_t)done;
      a.barrier[o] = (uint8_t)code;
      a.td[o] = td;
      a.priority[o] = powf(fabsf(td), a.alpha);
      if (a.explored) a.explored[o] = (uint8_t)explore;
      if (bad && a.counters) atomicAdd(a.counters, 1u);
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- step 15: reset on done; the bar pointer keeps advancing ------------
    if (done) {
      V = 1.0f;
      e_prev = 0.0f;
      armed = 0;
      cnt0 = cnt1 = cnt2 = 0;
      pushed = 0;
      pos = 0;
      ring = 0;
    }
    // the bars of the next step: the following ones, or the restart bar
    const bool restart = RECYCLE && done && t + 1 < a.L;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f0[h] = restart ? fr0[h] : f1[h];
      f1[h] = restart ? fr1[h] : f2[h];
    }
    p0 = restart ? pr0 : p1;
    p1 = restart ? pr1 : p2;
    bar = restart ? rbar : bar + 1;
    // the next step's state operands (the curiosity layer read these before
    // the last barrier)
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (j + 16 * h < kFeatures) put_state<false>(s_opnd, e, j + 16 * h, f0[h]);
    if (j == 0) put_state<false>(s_opnd, e, 51, V / V0 - 1.0f);
    if (j == 1) put_state<false>(s_opnd, e, 52, e_prev);
  }
}

}  // namespace

hipError_t launch_dqn(const DqnArgs& a, hipStream_t st) {
  if (a.N <= 0 || a.L <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.N + kRowsPerWave - 1) / kRowsPerWave);
  if (a.recycle)
    hipLaunchKernelGGL(dqn_collect_kernel<true>, dim3(blocks), dim3(64 * kSplit), 0, st, a);
  else
    hipLaunchKernelGGL(dqn_collect_kernel<false>, dim3(blocks), dim3(64 * kSplit), 0, st, a);
  return hipGetLastError();
}

}  // namespace rl
