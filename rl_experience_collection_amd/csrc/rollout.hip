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
//     (steps 6-8, 10), then resets the episode when a barrier fired (12);
//     with recycling ("GPU Pipeline Phase 2b", Future Phase 3 Optimization)
//     the episode also restarts at a drawn bar instead of running on.
// The critic value (step 5) and the curiosity bonus (step 9) are not read
// by any later step, so they are evaluated afterwards by the value kernel
// in one batched pass over every stored state.
//
// The layers use the MFMA layout (lane l computes rows l % 16).  The draw
// and the environment use another: wave q owns episodes 4q .. 4q+3 of the
// row group, one 16-lane row each; lane j of a row holds logits 3j .. 3j+2
// (read from LDS), so the softmax sum and the CDF are one DPP reduction and
// one scan within the row, and every lane of the row holds the episode's
// portfolio state.  Each wave writes its own episodes' state
// operands, state rows and outputs.
#include "collect.hpp"
#include "rows.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();
constexpr int kBufA = 8 * 64;  // first-layer output (128 = 8 tiles), then the logits
constexpr int kBufB = 4 * 64;  // second-layer output (64 = 4 tiles)

// Wave q's share of an actor layer, held in registers for the whole kernel:
// the A operands of its OTW output tiles for k-steps 0..S-1, and its bias.
template <bool BF16, int S, int OTW>
struct RegLayer {
  using Op = typename std::conditional<BF16, uint4, float>::type;
  Op a[S][OTW];
  f32x4 bias[OTW];
};

template <bool BF16, int S, int OTW>
__device__ __forceinline__ void load_reg_layer(RegLayer<BF16, S, OTW>& L, const float* pk,
                                               const float* pb, int q, int lane) {
  constexpr int kStep = kSplit * 64 * OTW;  // packed operands per k-step
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < OTW; ++i)
    L.bias[i] = *reinterpret_cast<const f32x4*>(pb + 16 * (q * OTW + i) + 4 * g);
  const int lane_off = (q * 64 + lane) * OTW;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < OTW; ++i) L.a[s][i] = reinterpret_cast<const uint4*>(pk)[s * kStep + lane_off + i];
    } else {
      load_operands<OTW>(pk + s * kStep + lane_off, L.a[s]);
    }
  }
}

// acc += sum over k-steps [S0, S1) of A_s B_s, B from the LDS operand layout
// (fp32: one f32x4 per group of 4 steps; bf16: one uint4 per step), all
// B reads issued before the first MFMA.
template <int S0, int S1, bool BF16, int S, int OTW>
__device__ __forceinline__ void reg_mfma(const RegLayer<BF16, S, OTW>& L, const f32x4* buf,
                                         f32x4 (&acc)[OTW], int lane) {
  if constexpr (BF16) {
    const uint4* bb = reinterpret_cast<const uint4*>(buf);
    uint4 b[S1 - S0];
#pragma unroll
    for (int s = S0; s < S1; ++s) b[s - S0] = bb[s * 64 + lane];
#pragma unroll
    for (int s = S0; s < S1; ++s)
#pragma unroll
      for (int i = 0; i < OTW; ++i) acc[i] = mfma_bf16(L.a[s][i], b[s - S0], acc[i]);
  } else {
    constexpr int G0 = S0 / 4, G1 = (S1 + 3) / 4;
    f32x4 b[G1 - G0];
#pragma unroll
    for (int gr = G0; gr < G1; ++gr) b[gr - G0] = buf[gr * 64 + lane];
#pragma unroll
    for (int s = S0; s < S1; ++s)
#pragma unroll
      for (int i = 0; i < OTW; ++i) acc[i] = mfma4(L.a[s][i], b[s / 4 - G0][s % 4], acc[i]);
  }
}

// The first-layer feature part, one k-step at a time: step<p>() issues the
// MFMAs of k-step p (the whole part for bf16, where it is one k-step) with
// scheduling fences on both sides, so callers can place them between
// independent VALU work.  The B operands are read once, at construction.
// With ACTIVE false (the part comes from the feature table instead) it
// reads and issues nothing.
template <bool BF16, int S, int TAIL, bool ACTIVE>
struct PreStepper {
  const RegLayer<BF16, S, 2>& L;
  typename std::conditional<BF16, uint4, f32x4>::type b[BF16 ? TAIL : (TAIL + 3) / 4];
  __device__ __forceinline__ PreStepper(const RegLayer<BF16, S, 2>& layer, const f32x4* buf, int lane)
      : L(layer) {
#pragma unroll
    for (int i = 0; i < (BF16 ? TAIL : (TAIL + 3) / 4); ++i) {
      if constexpr (!ACTIVE)
        ;
      else if constexpr (BF16)
        b[i] = reinterpret_cast<const uint4*>(buf)[i * 64 + lane];
      else
        b[i] = buf[i * 64 + lane];
    }
  }
  template <int P>
  __device__ __forceinline__ void step(f32x4 (&acc)[2]) const {
    if constexpr (ACTIVE && P < TAIL) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (BF16)
          acc[i] = mfma_bf16(L.a[P][i], b[P], acc[i]);
        else
          acc[i] = mfma4(L.a[P][i], b[P / 4][P % 4], acc[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// The actor's first-layer feature part: the first kTail k-steps of the first
// layer (k < 48 in fp32, k < 32 in bf16) read only the bar's market features
// (the portfolio inputs come after them), so bias + that part is known for
// every step of an episode that is not recycled (its bar is start + t)
// before the rollout runs.  The feature table holds it for every (t, n),
// [L][N][128] fp32 at output o = 16 * tile + 4 * g + c (the accumulator
// layout: lane e + 16 g of the wave that owns `tile` holds outputs
// 4g .. 4g+3 of row e).
template <bool BF16>
constexpr int feature_tail() { return BF16 ? 1 : 12; }

__device__ __forceinline__ void load_table_part(const float* __restrict__ table, int64_t row, int q,
                                                int lane, f32x4 (&pre)[2]) {
  const float* p = table + row * kActorOut1 + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 2; ++i) pre[i] = *reinterpret_cast<const f32x4*>(p + 16 * (2 * q + i));
}

// Persistent workgroups over groups of 16 consecutive (t, n) rows, the
// first layer's feature k-steps held in registers throughout: the same
// operands, MFMA instructions and order as the step kernel's in-place
// computation, so the table holds the same bits.
template <bool BF16>
__global__ __launch_bounds__(64 * kSplit) void feature_table_kernel(
    const float* __restrict__ weights, const float* __restrict__ features,
    const int32_t* __restrict__ starts, int64_t n_bars, int32_t N, int32_t L, int64_t row0,
    int64_t row1, float* __restrict__ table) {
  constexpr int kTail = feature_tail<BF16>();
  constexpr int kIn = BF16 ? 32 * kTail : 4 * kTail;  // inputs of the part
  __shared__ f32x4 s_state[4 * 64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  RegLayer<BF16, kTail, 2> w1;
  load_reg_layer(w1, weights + (BF16 ? kP.bact_w[0] : kP.actor_w[0]),
                 weights + (BF16 ? kP.bact_b[0] : kP.actor_b[0]), q, lane);
  s_state[threadIdx.x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // rows [row0, row1) of the [L][N] table, in groups of 16
  const int64_t groups = (row1 - row0 + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t hi = n_bars - (int64_t)L - 1;  // the step kernel's start clamp
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    __syncthreads();  // the previous group's operands are read
    for (int x = threadIdx.x; x < kRowsPerWave * kIn; x += 64 * kSplit) {
      const int e = x / kIn, k = x % kIn;
      int64_t r = row0 + grp * kRowsPerWave + e;
      r = r < row1 ? r : row1 - 1;
      const int32_t t = (int32_t)(r / N), n = (int32_t)(r % N);
      int64_t st = starts[n];
      st = st < 0 ? 0 : (st > hi ? hi : st);
      put_state<BF16>(s_state, e, k, features[(st + t) * kFeatures + k]);
    }
    __syncthreads();
    f32x4 pre[2] = {w1.bias[0], w1.bias[1]};
    reg_mfma<0, kTail>(w1, s_state, pre, lane);
    const int64_t r = row0 + grp * kRowsPerWave + (lane & 15);
    if (r < row1) {
      float* p = table + r * kActorOut1 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 2; ++i) *reinterpret_cast<f32x4*>(p + 16 * (2 * q + i)) = pre[i];
    }
  }
}

// TABLE (never with RECYCLE): the first-layer feature part comes from the
// feature table (a.ftable), loaded a step ahead, instead of being computed
// in the step.
template <bool BF16, bool RECYCLE, bool STAMPS, bool TABLE>
__global__ __launch_bounds__(64 * kSplit) void actor_rollout_kernel(RolloutArgs a) {
  __shared__ int s_restart[2];  // recycling: an episode of the workgroup restarted in step t (t % 2)
  __shared__ f32x4 s_bufA[kBufA];
  __shared__ f32x4 s_bufB[kBufB];
  __shared__ f32x4 s_state[4 * 64];
  __shared__ float s_ln[33];  // ln k for window counts k = 0..32 (ln 0 unused: times 0)

  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;

  if (threadIdx.x <= 32) s_ln[threadIdx.x] = threadIdx.x == 0 ? 0.0f : logf((float)threadIdx.x);
  if (threadIdx.x < 2) s_restart[threadIdx.x] = 0;
  // state operands start at zero: the padding slots stay zero
  s_state[threadIdx.x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // this wave's output tiles of the three layers, in registers throughout
  // (fp32 first layer: k-steps 14 and 15 only carry zero padding)
  constexpr int kS1 = BF16 ? kActorB[0].steps : 14;
  constexpr int kS2 = BF16 ? kActorB[1].steps : kActor[1].steps;
  constexpr int kS3 = BF16 ? kActorB[2].steps : kActor[2].steps;
  // first k-step holding a portfolio input (k = 48 .. 53): the steps before
  // it depend only on market features, known a step ahead
  constexpr int kTail = feature_tail<BF16>();
  RegLayer<BF16, kS1, 2> w1;
  RegLayer<BF16, kS2, 1> w2;
  RegLayer<BF16, kS3, 1> w3;
  load_reg_layer(w1, a.weights + (BF16 ? kP.bact_w[0] : kP.actor_w[0]),
                 a.weights + (BF16 ? kP.bact_b[0] : kP.actor_b[0]), q, lane);
  load_reg_layer(w2, a.weights + (BF16 ? kP.bact_w[1] : kP.actor_w[1]),
                 a.weights + (BF16 ? kP.bact_b[1] : kP.actor_b[1]), q, lane);
  load_reg_layer(w3, a.weights + (BF16 ? kP.bact_w[2] : kP.actor_w[2]),
                 a.weights + (BF16 ? kP.bact_b[2] : kP.actor_b[2]), q, lane);

  // Draw and environment layout: wave q owns episodes 4q .. 4q+3 of the
  // workgroup's 16, one row of 16 lanes (j = lane % 16) per episode; a row
  // holds the episode's portfolio state identically in all 16 lanes.
  const int e = 4 * q + (lane >> 4);
  const int j = lane & 15;
  const int32_t n_raw = blockIdx.x * kRowsPerWave + e;
  const bool valid = n_raw < a.N;
  const int32_t n = valid ? n_raw : a.N - 1;
  const EnvParams& ep = a.ep;

  // episode state (PPO CUDA Pipeline Design, Phase A steps 6-8, 12)
  float V = 1.0f, e_prev = 0.0f, entry = 0.0f;
  int armed = 0, side = 0, t_open = 0;
  int cnt0 = 0, cnt1 = 0, cnt2 = 0, pushed = 0, pos = 0;
  uint64_t ring = 0;  // 2 bits per window slot
  const float V0 = 1.0f;
  int64_t bar;  // the bar of step t
  if (a.t_begin == 0) {
    // clamp the start so every read stays inside the market buffers
    const int64_t hi = a.n_bars - (int64_t)a.L - 1;
    int64_t st = a.starts[n];
    const bool clamped = st < 0 || st > hi;
    st = st < 0 ? 0 : (st > hi ? hi : st);
    if (valid && j == 0) {
      a.start_used[n] = (int32_t)st;
      if (clamped && a.counters) atomicAdd(a.counters + 1, 1u);
    }
    bar = st;
  } else {
    // a later launch of a rollout split over several: the episode's state
    // as the previous launch left it (every lane of the row reads it)
    const int32_t* c = a.carry + (int64_t)n * kCarryWords;
    bar = (int64_t)(uint32_t)c[0] | ((int64_t)c[1] << 32);
    V = __int_as_float(c[2]);
    e_prev = __int_as_float(c[3]);
    entry = __int_as_float(c[4]);
    armed = c[5]; side = c[6]; t_open = c[7];
    cnt0 = c[8]; cnt1 = c[9]; cnt2 = c[10]; pushed = c[11]; pos = c[12];
    ring = (uint64_t)(uint32_t)c[13] | ((uint64_t)(uint32_t)c[14] << 32);
  }

  f32x4* bufA = s_bufA;
  f32x4* bufB = s_bufB;
  f32x4* sbuf = s_state;
  uint32_t n_bad = 0;  // this row's steps with a non-finite logit (lane j = 0)

  // features and prices of the first step's bar and the one after
  float f0[4], f1[4];
  load_features(a.features, bar, j, f0);
  load_features(a.features, bar + 1, j, f1);
  float p0 = a.prices[bar], p1 = a.prices[bar + 1];
  lds_barrier();  // operand buffer cleared
  if (j == 2) put_state<BF16>(sbuf, e, 53, ep.spread);  // constant element
#pragma unroll
  for (int h = 0; h < 4; ++h)
    if (j + 16 * h < kFeatures) put_state<BF16>(sbuf, e, j + 16 * h, f0[h]);
  lds_barrier();
  // first-layer feature part of the first step; with the table, that of
  // this lane's MFMA row (episode lane % 16)
  static_assert(!(TABLE && RECYCLE), "the table assumes the bar of step t is start + t");
  f32x4 pre[2];
  int32_t n_m = blockIdx.x * kRowsPerWave + (lane & 15);
  n_m = n_m < a.N ? n_m : a.N - 1;
  if constexpr (TABLE) {
    load_table_part(a.ftable, (int64_t)a.t_begin * a.N + n_m, q, lane, pre);
  } else {
    pre[0] = w1.bias[0];
    pre[1] = w1.bias[1];
    reg_mfma<0, kTail>(w1, sbuf, pre, lane);
  }

  // instrumented build: the clock at each phase boundary of a step, added
  // up per phase (the same value in every lane of the wave)
  uint64_t ph[kStampPhases];
  uint64_t t_prev = 0, t_loop = 0;
  if constexpr (STAMPS) {
#pragma unroll
    for (int k = 0; k < kStampPhases; ++k) ph[k] = 0;
    t_loop = __builtin_amdgcn_s_memtime();
  }
  auto stamp = [&](int k) {
    if constexpr (STAMPS) {
      const uint64_t now = __builtin_amdgcn_s_memtime();
      ph[k] += now - t_prev;
      t_prev = now;
    }
  };

  // the step's draw (and, recycling, its restart bar), 16 steps at a time
  RowDraws u_pool, rb_pool;
  for (int32_t t = a.t_begin; t < a.t_end; ++t) {
    if constexpr (STAMPS) t_prev = __builtin_amdgcn_s_memtime();
    const int64_t o = (int64_t)t * a.N + n;
    const int slot16 = (t - a.t_begin) & 15;
    if (slot16 == 0) {
      const int32_t tj = t + j;
      u_pool.pool = __float_as_uint(draw_uniform(a.seed, (uint32_t)n, (uint32_t)tj, 0u));
      if constexpr (RECYCLE)
        rb_pool.pool = tj + 1 < a.L ? (uint32_t)recycle_bar(a.seed, (uint32_t)n, tj, a.L, a.n_bars) : 0u;
    }

    // prefetch two bars ahead (independent of the outcomes), issued before
    // this step's stores so that no wait in the step covers them
    float f2[4];
    load_features(a.features, bar + 2 < a.n_bars ? bar + 2 : a.n_bars - 1, j, f2);
    const float p2 = a.prices[bar + 2 < a.n_bars ? bar + 2 : a.n_bars - 1];
    // with recycling, the restart bar this step would take if the episode
    // ended, and its first two bars, loaded ahead the same way
    int64_t rbar = 0;
    float fr0[4], fr1[4], pr0 = 0.0f, pr1 = 0.0f;
    if constexpr (RECYCLE) {
      rbar = t + 1 < a.L ? (int64_t)rb_pool.take(slot16, lane) : bar;
      load_features(a.features, rbar, j, fr0);
      load_features(a.features, rbar + 1, j, fr1);
      pr0 = a.prices[rbar];
      pr1 = a.prices[rbar + 1];
      a.bars[o] = (int32_t)bar;  // the value kernel's next-bar index
    }

    // ---- steps 1-2: state = 51 features, V/V0 - 1, exposure held, spread --
    // (the features are already in the operand buffer)
    const float vn = V / V0 - 1.0f;
    if (j == 0) put_state<BF16>(sbuf, e, 51, vn);
    if (j == 1) put_state<BF16>(sbuf, e, 52, e_prev);
    {
      // The step's memory stores carry no branches, so every path leaves
      // the same number of memory operations in flight and the wait for the
      // bars loaded ahead does not cover this step's stores: every lane
      // stores (lanes past the row's 54 elements repeat the last one), and
      // rows past N repeat episode N-1, whose very trajectory they run, so
      // repeated stores write the same bytes.
      float* srow = a.states + o * kState;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int k = j + 16 * h;
        float x = f0[h];
        if (h == 3 && k >= kFeatures) x = k == kFeatures ? vn : (k == kFeatures + 1 ? e_prev : ep.spread);
        srow[k < kState ? k : kState - 1] = x;
      }
    }
    stamp(0);       // state assembly and stores
    lds_barrier();  // state operands complete; last step's logits read
    if constexpr (RECYCLE) {
      // an episode restarted last step: its new features replaced those the
      // first-layer feature part was computed from, so recompute it
      const int again = s_restart[(t + 1) & 1];
      if (threadIdx.x == 0) s_restart[t & 1] = 0;
      if (again) {
        pre[0] = w1.bias[0];
        pre[1] = w1.bias[1];
        reg_mfma<0, kTail>(w1, sbuf, pre, lane);
      }
    }
    // the table part of the next step
    f32x4 pre_next[2];
    if constexpr (TABLE)
      load_table_part(a.ftable, (int64_t)(t + 1 < a.L ? t + 1 : t) * a.N + n_m, q, lane, pre_next);

    stamp(1);  // state barrier
    // the step's draw depends only on (seed, episode, step)
    const float u = __uint_as_float(u_pool.take(slot16, lane));
    // the layer chain and the draw run at a raised wave priority, so where
    // the two workgroups of a CU meet, the one in them issues first (the
    // environment step below returns to the base priority)
    __builtin_amdgcn_s_setprio(2);

    // ---- step 3: actor, a quarter of each layer per wave ------------------
    // (MFMA layout: lane l computes rows l % 16 of the workgroup)
    {
      f32x4 h[2] = {pre[0], pre[1]};
      reg_mfma<kTail, kS1>(w1, sbuf, h, lane);
      if constexpr (BF16)
        relu_store_bf16<2>(h, reinterpret_cast<uint4*>(bufA), q, lane);
      else
        relu_store<2>(h, bufA, q, lane);
    }
    stamp(2);  // first layer
    lds_barrier();
    stamp(3);
    // next step's features into the operand buffer (this step's state has
    // been read); the next feature part reads them after the next barrier
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (j + 16 * h < kFeatures) put_state<BF16>(sbuf, e, j + 16 * h, f1[h]);
    {
      f32x4 h[1] = {w2.bias[0]};
      reg_mfma<0, kS2>(w2, bufA, h, lane);
      if constexpr (BF16)
        relu_store_bf16<1>(h, reinterpret_cast<uint4*>(bufB), q, lane);
      else
        relu_store<1>(h, bufB, q, lane);
    }
    stamp(4);  // second layer (and the next step's features into LDS)
    lds_barrier();
    stamp(5);
    {
      f32x4 h[1] = {w3.bias[0]};
      reg_mfma<0, kS3>(w3, bufB, h, lane);
      // raw logits, fp32 (tile 3 is padding), over the first-layer output,
      // which every wave finished reading before the previous barrier:
      // logit k of row e at bufA[(k / 16) * 64 + e + 16 * (k % 16 / 4)][k % 4]
      bufA[q * 64 + lane] = h[0];
    }
    stamp(6);  // third layer
    lds_barrier();
    stamp(7);

    // first-layer feature part of the next step: its k-steps are spread
    // over the draw and environment below (one k-step per point, pinned by
    // scheduling fences), so the MFMAs run while the VALU works
    if constexpr (TABLE) {
      pre[0] = pre_next[0];
      pre[1] = pre_next[1];
    } else {
      pre[0] = w1.bias[0];
      pre[1] = w1.bias[1];
    }
    PreStepper<BF16, kS1, kTail, !TABLE> ps(w1, sbuf, lane);

    // ---- step 4: softmax, CDF, inverse-CDF draw, log-prob -----------------
    // lane j of the episode's row holds logits k = 3j + h, h = 0..2 (lane 15
    // none), so the CDF is one scan over the row of the lanes' sums plus
    // each lane's own prefix of its three
    const float* lg = reinterpret_cast<const float*>(bufA);
    float l[3], ex[3];
    bool ok[3];
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      const int k = 3 * j + h;  // (< 48: inside the four logit tiles)
      ok[h] = k < kActions;
      l[h] = lg[((k >> 4) * 64 + e + 16 * ((k & 15) >> 2)) * 4 + (k & 3)];
    }
    ps.template step<0>(pre);
    int bad = 0;
    float m = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (ok[h]) {
        bad |= !isfinite(l[h]);
        m = fmaxf(m, l[h]);
      }
    m = row_max(m);
    ps.template step<1>(pre);
#pragma unroll
    for (int h = 0; h < 3; ++h) ex[h] = ok[h] ? expf(l[h] - m) : 0.0f;
    ps.template step<2>(pre);
    // CDF_k = (sum of the lanes before j) + (this lane's prefix up to k)
    float pre3[3];
    pre3[0] = ex[0];
    pre3[1] = ex[0] + ex[1];
    pre3[2] = pre3[1] + ex[2];
    const float S = row_sum(pre3[2]);
    const float before = dpp_f<0x111>(row_scan(pre3[2]));  // row_shr:1 (lane 0 reads 0)
    ps.template step<3>(pre);
    // first k with u < CDF_k, as u * S < (sum of e up to k)
    const float uS = u * S;
    int cand = 64;
#pragma unroll
    for (int h = 2; h >= 0; --h)
      if (ok[h] && uS < before + pre3[h]) cand = 3 * j + h;
    int act_a = row_min_i(cand);
    ps.template step<4>(pre);
    if (act_a == 64) {  // rounding left u >= CDF_44: last action with weight
      int lastk = -1;
#pragma unroll
      for (int h = 0; h < 3; ++h)
        if (ok[h] && ex[h] > 0.0f) lastk = 3 * j + h;
      lastk = row_max_i(lastk);
      act_a = lastk >= 0 ? lastk : kActions - 1;
    }
    float la = -INFINITY;
#pragma unroll
    for (int h = 0; h < 3; ++h)
      if (3 * j + h == act_a) la = l[h];
    la = row_max(la);
    const float logp = (la - m) - logf(S);
    ps.template step<5>(pre);
    bad = row_max_i(bad);
    stamp(8);  // draw

    __builtin_amdgcn_s_setprio(0);
    // ---- step 6: portfolio (exposure fraction of equity, turnover cost) ---
    const int xi = act_a / 9;
    const int oi = (act_a % 9) / 3;
    const int ui = act_a % 3;
    // the exposure and cost-rate tables by selects on the kernel arguments
    // (no table lookup in the step's dependent chain)
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
    ps.template step<6>(pre);

    // ---- step 7: triple barrier on raw prices ------------------------------
    // (selects: the four episodes of a wave take different branches)
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
    ps.template step<7>(pre);
    const bool lng = side > 0;
    const float take_px = entry * (lng ? ep.up_pt : ep.dn_pt);
    const float stop_px = entry * (lng ? ep.dn_sl : ep.up_sl);
    const bool take = lng ? p1 >= take_px : p1 <= take_px;
    const bool stop = lng ? p1 <= stop_px : p1 >= stop_px;
    const bool expire = t + 1 - t_open >= ep.max_hold;
    const int hit = armed ? (take ? 1 : (stop ? -1 : 0)) : 0;
    const int code = armed ? (take ? 1 : (stop ? 2 : (expire ? 3 : 0))) : 0;

    // ---- step 8: diversity window, 3-class entropy in nats -----------------
    // H = ln n - (sum_c n_c ln n_c) / n, compared as n ln n - sum n_c ln n_c
    // < threshold * n; ln of the counts 0..32 comes from an LDS table
    const int cat = xi <= 1 ? 0 : (xi == 2 ? 1 : 2);
    ps.template step<8>(pre);
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
    ps.template step<9>(pre);
    const float hn = (float)nn * s_ln[nn] -
                     (((float)cnt0 * s_ln[cnt0] + (float)cnt1 * s_ln[cnt1]) + (float)cnt2 * s_ln[cnt2]);
    const float div = hn < ep.div_threshold * (float)nn ? ep.div_penalty : 0.0f;

    stamp(9);  // environment
    // ---- steps 10-11: partial reward and stores (lane 0 of the row) -------
    const float partial = pnl * (1.0f + ep.barrier_scale * (float)hit) + div;
    ps.template step<10>(pre);
    const int done = code != 0;
    // every lane of the row holds the same results: all store (see the
    // state stores above)
    a.actions[o] = act_a;
    a.log_probs[o] = logp;
    a.rewards[o] = partial;
    a.dones[o] = (uint8_t)done;
    a.barrier[o] = (uint8_t)code;
    n_bad += (bad && valid && j == 0) ? 1u : 0u;
    if (a.logits) {
      float* lrow = a.logits + o * kActions;
      // lane 15 holds no logit: it repeats logit 44 (lane 14's third)
      const float l44 = dpp_f<0x111>(l[2]);
#pragma unroll
      for (int h = 0; h < 3; ++h) lrow[ok[h] ? 3 * j + h : kActions - 1] = ok[h] ? l[h] : l44;
    }

    // ---- step 12: reset on done; the bar pointer keeps advancing ------------
    ps.template step<11>(pre);
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
    // the bars of the next step: the following ones, or (recycling) the
    // restart bar, whose features replace the next step's operands
    const bool restart = RECYCLE && done && t + 1 < a.L;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f0[h] = restart ? fr0[h] : f1[h];
      f1[h] = restart ? fr1[h] : f2[h];
    }
    p0 = restart ? pr0 : p1;
    p1 = restart ? pr1 : p2;
    bar = restart ? rbar : bar + 1;
    if constexpr (RECYCLE) {
      if (restart) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          if (j + 16 * h < kFeatures) put_state<BF16>(sbuf, e, j + 16 * h, f0[h]);
        if (j == 0) s_restart[t & 1] = 1;
      }
    }
    stamp(10);  // stores and reset
  }
  if constexpr (STAMPS) {
    const uint64_t loop = __builtin_amdgcn_s_memtime() - t_loop;
    if (lane == 0) {
      // one wave per slot; the launches of a collection are stream-ordered
      uint64_t* s = a.stamps + ((int64_t)blockIdx.x * kSplit + q) * kStampWords;
#pragma unroll
      for (int k = 0; k < kStampPhases; ++k) s[k] += ph[k];
      s[kStampPhases] += (uint64_t)(a.t_end - a.t_begin);
      s[kStampPhases + 1] += loop;
    }
  }
  if (n_bad && a.counters) atomicAdd(a.counters, n_bad);
  if (a.t_end < a.L && valid && j == 0) {
    int32_t* c = a.carry + (int64_t)n * kCarryWords;
    c[0] = (int32_t)(uint32_t)bar; c[1] = (int32_t)(bar >> 32);
    c[2] = __float_as_int(V); c[3] = __float_as_int(e_prev); c[4] = __float_as_int(entry);
    c[5] = armed; c[6] = side; c[7] = t_open;
    c[8] = cnt0; c[9] = cnt1; c[10] = cnt2; c[11] = pushed; c[12] = pos;
    c[13] = (int32_t)(uint32_t)ring; c[14] = (int32_t)(uint32_t)(ring >> 32);
  }
}

}  // namespace

int actor_lds_bytes(bool bf16, bool recycle) {
  auto kernel = bf16 ? (recycle ? actor_rollout_kernel<true, true, false, false>
                                : actor_rollout_kernel<true, false, false, false>)
                     : (recycle ? actor_rollout_kernel<false, true, false, false>
                                : actor_rollout_kernel<false, false, false, false>);
  hipFuncAttributes at;
  if (hipFuncGetAttributes(&at, reinterpret_cast<const void*>(kernel)) != hipSuccess) return -1;
  return (int)at.sharedSizeBytes;
}

hipError_t launch_actor_rollout(const RolloutArgs& a, hipStream_t st) {
  if (a.N <= 0 || a.L <= 0) return hipSuccess;
  // a launch covers steps [t_begin, t_end); one that starts after step 0
  // or ends before L reads or leaves the episode state in `carry`
  if (a.t_begin < 0 || a.t_end > a.L || a.t_begin >= a.t_end ||
      ((a.t_begin > 0 || a.t_end < a.L) && !a.carry))
    return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.N + kRowsPerWave - 1) / kRowsPerWave);
  if (a.ftable && a.bars) return hipErrorInvalidValue;  // no table with recycling
  auto pick = [&](auto stamps, auto table) {
    constexpr bool S = decltype(stamps)::value, T = decltype(table)::value;
    return a.bf16 ? (a.bars ? actor_rollout_kernel<true, true, S, false> : actor_rollout_kernel<true, false, S, T>)
                  : (a.bars ? actor_rollout_kernel<false, true, S, false> : actor_rollout_kernel<false, false, S, T>);
  };
  auto kernel = a.ftable ? (a.stamps ? pick(std::true_type{}, std::true_type{})
                                     : pick(std::false_type{}, std::true_type{}))
                         : (a.stamps ? pick(std::true_type{}, std::false_type{})
                                     : pick(std::false_type{}, std::false_type{}));
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(64 * kSplit), 0, st, a);
  return hipGetLastError();
}

int feature_table_lds_bytes(bool bf16) {
  hipFuncAttributes at;
  const void* k = bf16 ? reinterpret_cast<const void*>(feature_table_kernel<true>)
                       : reinterpret_cast<const void*>(feature_table_kernel<false>);
  if (hipFuncGetAttributes(&at, k) != hipSuccess) return -1;
  return (int)at.sharedSizeBytes;
}

hipError_t launch_feature_table(const float* weights, const float* features, const int32_t* starts,
                                int64_t n_bars, int32_t N, int32_t L, bool bf16, float* table,
                                int64_t row0, int64_t row1, int grid, int lds_pad,
                                hipStream_t st) {
  const int64_t rows = (int64_t)L * N;
  if (N <= 0 || L <= 0 || row0 < 0 || row1 > rows || row0 > row1 || grid < 1 || lds_pad < 0)
    return hipErrorInvalidValue;
  if (row0 == row1) return hipSuccess;
  const int64_t groups = (row1 - row0 + kRowsPerWave - 1) / kRowsPerWave;
  const unsigned blocks = (unsigned)(groups < grid ? groups : grid);
  // (lds_pad reserves LDS the kernel does not use, which only limits where
  // its workgroups can be placed)
  hipLaunchKernelGGL(bf16 ? feature_table_kernel<true> : feature_table_kernel<false>, dim3(blocks),
                     dim3(64 * kSplit), (unsigned)lds_pad, st, weights, features, starts, n_bars, N,
                     L, row0, row1, table);
  return hipGetLastError();
}

}  // namespace rl
