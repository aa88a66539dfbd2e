// Batched part of PPO experience collection: the critic value (PPO CUDA
// Pipeline Design, Kernel Phases, Phase A step 5) and the curiosity bonus
// (step 9, the forward model of GPU Pipeline Phase 2b, Kernel Components 2)
// of every stored step, then the final reward (step 10).
//
// Neither output feeds a later step, so the L*N stored states are evaluated
// as one batch.  A workgroup holds RT row tiles of 16 consecutive (t, n)
// rows of the [L][N] layout; its W waves (fp32: 4 waves, 2 row tiles; bf16:
// 8 waves, 8 row tiles, one workgroup per CU) share all RT tiles and each
// computes 1/W of the wide layers' outputs for all of them:
//   critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (MFMA, ReLU) -> 1 (VALU),
//   curiosity [state, one-hot(a)] -> 128 (ReLU) -> 51, MSE against the next
//   bar's 51 features, bonus = coef * MSE.
// fp32: the two 4-tile layers (128 -> 64, 128 -> 51) give wave q tile q % 4
// of the row tiles of its group of four, through LDS like the wide layers.
// bf16: after 256 -> 128 each wave finishes its own row tile alone (critic
// 128 -> 64 -> 1, both curiosity layers, MSE, reward) from weights staged in
// LDS once per group, with the curiosity activations kept in registers and
// no barrier between these layers.
// Every weight operand a wave loads feeds one MFMA per row tile, and the
// next layer's first weight steps are loaded before the barriers that end
// the current layer.  Activations live in LDS (a layer's input is read by
// every wave, its output written back after a barrier).  The packed weights
// (1.46 MB fp32, 0.73 MB bf16) stay resident in every XCD's L2.
// The one-hot half of the curiosity input is a column gather, not a dense
// product.
// Precision: fp32 (v_mfma_f32_16x16x4_f32) or bf16 weights and layer inputs
// with fp32 accumulation (v_mfma_f32_16x16x32_bf16); biases, the last-layer
// outputs, the MSE and the reward stay fp32 in both.
#include "collect.hpp"

#include <math.h>

#include <atomic>

namespace rl {

namespace {

constexpr PackedOffsets kP = packed_offsets();

template <bool BF16>
struct ValueShape {
  static constexpr int W = value_waves(BF16);  // waves per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int RT = value_row_tiles(BF16);
  // The two 4-tile layers (critic 128 -> 64, curiosity 128 -> 51) split 4
  // ways on outputs and RH ways on rows: wave q computes output tile q % 4
  // for the RTS row tiles from (q / 4) * RTS.
  static constexpr int RH = W / kSplit;
  static constexpr int RTS = RT / RH;
  // output tiles per wave of the wide layers
  static constexpr int O1 = (BF16 ? kCriticB[0].ot : kCritic[0].ot) / W;
  static constexpr int O2 = (BF16 ? kCriticB[1].ot : kCritic[1].ot) / W;
  static constexpr int O3 = (BF16 ? kCriticB[2].ot : kCritic[2].ot) / W;
  static constexpr int O4 = (BF16 ? kCriticB[3].ot : kCritic[3].ot) / W;
  static constexpr int OC1 = (BF16 ? kCurB[0].ot : kCur[0].ot) / W;
  // 16-byte LDS operands per row tile of the widest activation (512)
  static constexpr int kTile = BF16 ? 16 * 64 : 32 * 64;
  // floats of the workgroup's state rows, and 16-byte first-layer operands
  // per row tile (bf16: 2 k-steps, fp32: 4 groups of 4 k-steps, x 64 lanes)
  static constexpr int kRaw = RT * kRowsPerWave * kState;
  static constexpr int kOpTile = BF16 ? 2 * 64 : 4 * 64;
  // row tiles whose epilogue (action, next bar, partial reward, value and
  // reward) one wave handles: wave q takes row tiles q + W e, e < ER
  static constexpr int ER = (RT + W - 1) / W;
  // waves per SIMD: fp32 runs two 4-wave workgroups per CU; bf16 one
  // workgroup per CU (its 128 rows of activations fill the LDS) of one or
  // two waves per SIMD
  static constexpr int kWavesPerEU = BF16 && W == kSplit ? 1 : 2;
  static_assert(RT >= 1 && ER <= 2, "at most two row tiles per wave in the epilogue");
  static_assert(W % kSplit == 0 && RT % RH == 0, "the 4-tile layers cover every row tile");
  static_assert(O1 * W == (BF16 ? kCriticB[0].ot : kCritic[0].ot) &&
                    O2 * W == (BF16 ? kCriticB[1].ot : kCritic[1].ot) &&
                    O3 * W == (BF16 ? kCriticB[2].ot : kCritic[2].ot) &&
                    O4 * W == (BF16 ? kCriticB[3].ot : kCritic[3].ot) &&
                    OC1 * W == (BF16 ? kCurB[0].ot : kCur[0].ot),
                "whole output tiles per wave");
  static_assert((BF16 ? kCriticB[4].ot : kCritic[4].ot) == kSplit &&
                    (BF16 ? kCurB[1].ot : kCur[1].ot) == kSplit,
                "one output tile per wave in the 4-tile layers");
};

// An empty asm that takes and returns every accumulator of a layer: the
// layer's MFMAs are then all issued before it, so the compiler cannot sink
// them past the barrier and loads that follow in program order (an inline
// asm orders memory operations only).
template <int RT, int OTW>
__device__ __forceinline__ void pin_tiles(f32x4 (&acc)[RT][OTW]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < OTW; ++i) asm volatile("" : "+v"(acc[rt][i]));
}

// The packed block as a buffer resource plus its base pointer (biases and
// small tables are read through the pointer).
struct Weights {
  GlobalWeights gw;
  const float* W;
};

template <int S, bool BF16, int OTW, int D, int SPLIT>
__device__ __forceinline__ void begin(WeightStream<BF16, OTW, D, SPLIT>& st, const Weights& w,
                                      int64_t w32, int64_t wb, int64_t b_off, int q, int lane) {
  stream_begin<S>(st, w.gw, (uint32_t)(4 * (BF16 ? wb : w32)), w.W + b_off, q, lane);
}

// SK: the fp32 k-steps that hold inputs (the first layers' 54 inputs fill 14
// of their 16 steps; the rest is zero padding and issues no MFMA)
template <int S, int SK = S, bool BF16, int OTW, int D, int SPLIT, int RT, class BL>
__device__ __forceinline__ void run(WeightStream<BF16, OTW, D, SPLIT>& st, const Weights& w,
                                    int64_t w32, int64_t wb, const BL& bl,
                                    f32x4 (&acc)[RT][OTW], int q, int lane) {
  if constexpr (BF16)
    stream_layer<S, OTW, D, RT>(st, w.gw, (uint32_t)(4 * wb), bl, acc, q, lane);
  else
    stream_layer<S, OTW, D, RT, SK>(st, w.gw, (uint32_t)(4 * w32), bl, acc, q, lane);
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
__global__ __launch_bounds__(ValueShape<BF16>::kThreads)
__attribute__((amdgpu_waves_per_eu(ValueShape<BF16>::kWavesPerEU)))
void value_kernel(ValueArgs a) {
  using Sh = ValueShape<BF16>;
  constexpr int RT = Sh::RT;
  constexpr int RTS = Sh::RTS;
  constexpr int W = Sh::W;
  constexpr int kThreads = Sh::kThreads;
  constexpr int TS = Sh::kTile;
  // layer k-steps (fp32 / bf16 forms differ)
  constexpr int S1 = BF16 ? kCriticB[0].steps : kCritic[0].steps;
  constexpr int S2 = BF16 ? kCriticB[1].steps : kCritic[1].steps;
  constexpr int S3 = BF16 ? kCriticB[2].steps : kCritic[2].steps;
  constexpr int S4 = BF16 ? kCriticB[3].steps : kCritic[3].steps;
  constexpr int S5 = BF16 ? kCriticB[4].steps : kCritic[4].steps;
  constexpr int SC1 = BF16 ? kCurB[0].steps : kCur[0].steps;
  constexpr int SC2 = BF16 ? kCurB[1].steps : kCur[1].steps;
  __shared__ f32x4 s_buf[RT * TS];
  __shared__ f32x4 s_opnd[RT * Sh::kOpTile];
  __shared__ float s_part[2][RT][kSplit][16];
  // action and next bar (curiosity target) of each row of the group
  __shared__ int s_act[RT * kRowsPerWave], s_nbar[RT * kRowsPerWave];
  __shared__ float s_env[kEnvTable];
  fill_env_table(a.ep, s_env, (int)threadIdx.x);  // read after the loop's first barrier
  // bf16 keeps the third and fourth layers' outputs at their own k-step
  // counts per row tile (8 and 4), so the tail's staged weights and biases
  // (uint4 units from kTailAt: kTailW of weights, then 80 of biases and the
  // 64 -> 1 row) fit beside the third layer's output
  constexpr int TS3 = BF16 ? 8 * 64 : TS;
  constexpr int TS4 = BF16 ? 4 * 64 : TS;
  constexpr int kTailW = 3 * 1024;
  constexpr int kTailN = kTailW + 80;
  constexpr int kTailAt = RT * TS3;
  constexpr int kStageN = BF16 ? (kTailN + kThreads - 1) / kThreads : 1;
  static_assert(!BF16 || (kTailAt + kTailN <= RT * TS && S5 == 4 && SC1 == 2 && SC2 == 4 &&
                          RT * TS4 <= kTailAt),
                "bf16 tail layout");
  static_assert(!BF16 || (kP.bcur_w[0] == kP.bcritic_w[4] + 4 * kTailW / 3 &&
                          kP.bcur_w[1] == kP.bcur_w[0] + 4 * kTailW / 3 &&
                          packed_layer_floats_bf16(kCurB[1]) == 4 * kTailW / 3),
                "the three tail layers are one run of the packed block");
  uint32_t n_bad = 0;  // rows with a non-finite value or reward (bf16 tail)

  const int64_t rows = (int64_t)a.L * a.N;
  const int64_t groups = ((rows + kRowsPerWave - 1) / kRowsPerWave + RT - 1) / RT;

  // Persistent workgroups: the grid is the resident capacity; a workgroup
  // starts on group blockIdx.x and takes its next group from a work counter
  // (gridDim.x + ticket), so faster workgroups take more groups.  Across
  // iterations every LDS buffer's last read and next write are separated by
  // at least one of the body's barriers, so the loop adds none.
  __shared__ unsigned long long s_next;
  // The state rows of the next group are loaded into registers during an
  // iteration (once that group is known) and written to the first-layer
  // operand layout as soon as this group's curiosity layer has read it.
  // Thread tid handles the 16-byte operand chunks c = i * kThreads + tid:
  // chunk c of the operand buffer is (row tile, k-group, lane) = (c / (64 G),
  // c / 64 % G, c % 64), i.e. the inputs k0 .. k0 + kCF - 1 of row
  // 16 rt + lane % 16 for lane group lane / 16; they are consecutive floats
  // of the state row, and the chunk store is one 16-byte LDS write.  In
  // bf16 wave q handles the chunks of row tile q (its own rows in the tail,
  // which then needs no barrier before the store).
  constexpr int kG = BF16 ? 2 : 4;          // k-groups per row tile
  constexpr int kCF = BF16 ? 8 : 4;         // floats per chunk
  constexpr int kCPT = RT * Sh::kOpTile / kThreads;
  static_assert(RT * Sh::kOpTile % kThreads == 0, "whole chunks per thread");
  static_assert(!BF16 || (RT == W && kCPT * 64 == Sh::kOpTile), "bf16: one row tile per wave");
  auto chunk_of = [](int i, int tid_) {
    return BF16 ? (tid_ >> 6) * Sh::kOpTile + i * 64 + (tid_ & 63) : i * kThreads + tid_;
  };
  // floats of a group's state rows present in [L][N][54]
  auto avail_of = [&](int64_t g_) -> int {
    const int64_t av = (rows - g_ * RT * kRowsPerWave) * kState;
    return av < Sh::kRaw ? (int)av : Sh::kRaw;
  };
  auto chunk_k0 = [](int c) {
    const int gg = (c & 63) >> 4, grp = (c >> 6) & (kG - 1);
    return BF16 ? 32 * grp + 8 * gg : kFirstSteps * gg + 4 * grp;
  };
  // the group's rows through a buffer resource whose extent ends at the last
  // row present (reads past it return 0: the rows past the end)
  auto load_states = [&](int64_t g_, int tid_, float (&v)[kCPT][kCF]) {
    const BufRsrc rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.states + g_ * RT * kRowsPerWave * kState), 0, 4 * avail_of(g_),
        0x00020000);
#pragma unroll
    for (int i = 0; i < kCPT; ++i) {
      const int c = chunk_of(i, tid_);
      const int row = (c >> 6) / kG * kRowsPerWave + (c & 15);
      const uint32_t off = 4u * (uint32_t)(row * kState + chunk_k0(c));
#pragma unroll
      for (int j = 0; j < kCF; j += 2) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4u * j, 0, 0);
        v[i][j] = __uint_as_float(w.x);
        v[i][j + 1] = __uint_as_float(w.y);
      }
    }
  };
  // zero where the k-permutation points past the 54 inputs, then one
  // 16-byte store per chunk
  auto scatter_states = [&](int tid_, const float (&v)[kCPT][kCF]) {
#pragma unroll
    for (int i = 0; i < kCPT; ++i) {
      const int c = chunk_of(i, tid_);
      const int k0 = chunk_k0(c);
      float x[kCF];
#pragma unroll
      for (int j = 0; j < kCF; ++j) {
        const bool ok = BF16 ? k0 + j < kState
                             : (((c >> 6) & (kG - 1)) * 4 + j < kFirstSteps && k0 + j < kState);
        x[j] = ok ? v[i][j] : 0.0f;
      }
      if constexpr (BF16) {
        uint4 w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        w.z = pack_bf16x2(x[4], x[5]);
        w.w = pack_bf16x2(x[6], x[7]);
        reinterpret_cast<uint4*>(s_opnd)[c] = w;
      } else {
        s_opnd[c] = f32x4{x[0], x[1], x[2], x[3]};
      }
    }
  };
  // bf16: the first layer (two k-steps, all prefetched) loads at the end of
  // the previous iteration, so its short MFMA run does not wait on L2
  Stream<BF16, Sh::O1, W> w1;
  if constexpr (BF16) {
    const Weights wt0{GlobalWeights{weights_rsrc(a.weights, (uint32_t)(4 * kP.total))}, a.weights};
    begin<S1>(w1, wt0, kP.critic_w[0], kP.bcritic_w[0], kP.critic_b[0], (int)threadIdx.x >> 6,
              (int)threadIdx.x & 63);
  }
  int64_t grp = blockIdx.x;
  if (grp < groups) {
    float v0[kCPT][kCF];
    load_states(grp, (int)threadIdx.x, v0);
    scatter_states((int)threadIdx.x, v0);
  }
  __syncthreads();
#pragma unroll 1
  while (grp < groups) {
  const int64_t tile0 = grp * RT;
  // the weight loads are the same every iteration; an opaque zero offset on
  // the pointer and an opaque copy of the thread index keep the compiler
  // from hoisting them (and the registers they would hold) out of the loop
  int32_t opaque0 = 0;  // (an offset, so W keeps the global address space)
  asm volatile("" : "+s"(opaque0));
  const float* Wp = a.weights + opaque0;
  const Weights wt{GlobalWeights{weights_rsrc(Wp, (uint32_t)(4 * kP.total))}, Wp};
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int q = tid >> 6;  // wave: output tiles of the wide layers
  const int q4 = Sh::RH > 1 ? q & (kSplit - 1) : q;  // 4-tile layers: output tile q4 ...
  const int rs0 = Sh::RH > 1 ? (q >> 2) * RTS : 0;   // ... of row tiles rs0 .. rs0 + RTS - 1
  const int g = lane >> 4;

  constexpr int ER = Sh::ER;
  // the epilogue's rows: row tile q + W e, lane % 16 (tail rows recompute
  // the last row)
  int64_t my_raw[ER], my_row[ER];
#pragma unroll
  for (int e = 0; e < ER; ++e) {
    my_raw[e] = (tile0 + q + W * e) * kRowsPerWave + (lane & 15);
    my_row[e] = my_raw[e] < rows ? my_raw[e] : rows - 1;
  }
  // (t, n) of the workgroup's first row; a row tile's rows are row0 + off
  const int64_t row0 = tile0 * kRowsPerWave;
  const uint64_t t_base = (uint64_t)(row0 / a.N);
  const uint32_t n_base = (uint32_t)(row0 - (int64_t)t_base * a.N);
  // (t, n) of row 16 rt + lane % 16 of the group (rows past the end: the last row)
  auto row_tn = [&](int rt, int32_t& t, int32_t& n) {
    const uint32_t x = n_base + (uint32_t)(rt * kRowsPerWave + (lane & 15));
    const uint32_t dt = x / (uint32_t)a.N;
    n = (int32_t)(x - dt * (uint32_t)a.N);
    t = (int32_t)(t_base + dt);
    if (t_base + dt >= (uint64_t)a.L) {
      t = a.L - 1;
      n = a.N - 1;
    }
  };

  // ticket for the next group, taken before the loads below and published
  // after the first layer (when it has long arrived)
  unsigned long long ticket = 0;
  if (tid == 0) ticket = atomicAdd(a.sched, 1ull);
  if constexpr (!BF16) begin<S1>(w1, wt, kP.critic_w[0], kP.bcritic_w[0], kP.critic_b[0], q, lane);
  // (this group's operands were scattered before the previous barrier)
  const LdsOperands states_in{s_opnd, Sh::kOpTile};
  const LdsOperands acts{s_buf, TS};
  const LdsOperands acts_s{s_buf + rs0 * TS, TS};  // the 4-tile layers' row tiles

  // ---- critic -----------------------------------------------------------
  // the first layer reads the state operands, so s_buf is free for its output
  Stream<BF16, Sh::O2, W> w2;
  if constexpr (BF16 && RT % 2 == 0) {
    // all k-steps of the bf16 first layer sit in the ring: two passes of
    // RT / 2 row tiles over the same weight registers halve the accumulators
    static_assert(S1 < ring_depth(true, Sh::O1), "first layer fully prefetched");
    constexpr int H = RT / 2;
    f32x4 h1[H][Sh::O1];
    run<S1>(w1, wt, kP.critic_w[0], kP.bcritic_w[0], states_in, h1, q, lane);
    store<BF16, Sh::O1, H>(h1, s_buf, TS, q, lane);
    run<S1>(w1, wt, kP.critic_w[0], kP.bcritic_w[0], LdsOperands{s_opnd + H * Sh::kOpTile, Sh::kOpTile},
            h1, q, lane);
    begin<S2>(w2, wt, kP.critic_w[1], kP.bcritic_w[1], kP.critic_b[1], q, lane);
    store<BF16, Sh::O1, H>(h1, s_buf + H * TS, TS, q, lane);
  } else {
    f32x4 h1[RT][Sh::O1];
    run<S1, kFirstSteps>(w1, wt, kP.critic_w[0], kP.bcritic_w[0], states_in, h1, q, lane);
    begin<S2>(w2, wt, kP.critic_w[1], kP.bcritic_w[1], kP.critic_b[1], q, lane);
    store<BF16, Sh::O1, RT>(h1, s_buf, TS, q, lane);
  }
  // every wave read the previous s_next before the barrier above
  if (tid == 0) s_next = gridDim.x + ticket;
  lds_barrier();  // the output is complete

  f32x4 h2[RT][Sh::O2];
  run<S2>(w2, wt, kP.critic_w[1], kP.bcritic_w[1], acts, h2, q, lane);
  Stream<BF16, Sh::O3, W> w3;
  begin<S3>(w3, wt, kP.critic_w[2], kP.bcritic_w[2], kP.critic_b[2], q, lane);
  // the next group (published after the first layer): its state rows load
  // past the register peak of the wide layers (fp32 here, bf16 two layers
  // later), in flight until the scatter below; unconditional (clamped
  // group), since a conditional load would keep the old values live
  const int64_t grp_next = (int64_t)s_next;
  float v_states[kCPT][kCF];
  auto prefetch_next = [&]() {
    int tid2 = tid;  // an opaque copy: nothing computed for the scatter is kept live
    asm volatile("" : "+v"(tid2));
    load_states(grp_next < groups ? grp_next : groups - 1, tid2, v_states);
  };
  if constexpr (!BF16) prefetch_next();
  lds_barrier();
  store<BF16, Sh::O2, RT>(h2, s_buf, TS, q, lane);
  lds_barrier();

  f32x4 h3[RT][Sh::O3];
  run<S3>(w3, wt, kP.critic_w[2], kP.bcritic_w[2], acts, h3, q, lane);
  Stream<BF16, Sh::O4, W> w4;
  begin<S4>(w4, wt, kP.critic_w[3], kP.bcritic_w[3], kP.critic_b[3], q, lane);
  // what the curiosity and reward epilogue reads, loaded past the register
  // peak of the wide layers so it arrives during the rest: wave q < RT
  // loads the action and the next bar (the MSE target) of row tile q's
  // rows (fp32: they go through LDS to every wave after the next layer)
  // (one load per value, with no branch around it: a load behind a branch
  // writes the registers another path loads into, and the compiler then
  // waits for every load in flight)
  if constexpr (BF16) pin_tiles(h3);  // the layer's MFMAs stay ahead of the staging below
  int my_act[ER], my_nbar[ER];
  float partial[ER];
#pragma unroll
  for (int e = 0; e < ER; ++e) {
    const int rt = q + W * e < RT ? q + W * e : RT - 1;
    int32_t t, n;
    row_tn(rt, t, n);
    const int64_t o = (int64_t)t * a.N + n;
    my_act[e] = a.actions[o];
    // the bar of the step (recorded, or start + step), + 1 added at its use
    my_nbar[e] = a.bars ? a.bars[o] : a.start_used[n];
    if (!a.bars) my_nbar[e] += a.t_off + t;
    partial[e] = a.rewards[my_row[e]];
  }
  lds_barrier();
  // bf16: the tail layers' weights (critic 128 -> 64, curiosity 1 and 2:
  // one 48 KB run of the packed block), their biases and the 64 -> 1 row,
  // loaded now (past the register peak) and written into LDS next to the
  // third layer's output once the fourth layer has run; every wave then runs
  // the tail on its own row tile with no barrier between layers
  uint4 stage[kStageN];
  if constexpr (BF16) {
    static_assert(kTailW % kThreads == 0 && kTailN - kTailW <= kThreads, "one bias round");
#pragma unroll
    for (int i = 0; i < kStageN - 1; ++i)  // weights: 16-byte chunk i * kThreads + tid
      stage[i] = wt.gw.u4(4u * (uint32_t)(kP.bcritic_w[4] + 4 * (i * kThreads + tid)), 0u);
    // then chunk b of the biases (critic 128 -> 64: 16, curiosity 1: 32,
    // curiosity 2: 16) and the 64 -> 1 row (16), b clamped (duplicates
    // store equal bytes); the offset as sums of selects, not branches
    const int b = tid < kTailN - kTailW ? tid : kTailN - kTailW - 1;
    const uint32_t fo = (uint32_t)(kP.critic_b[4] + 4 * b) +
                        (b >= 16 ? (uint32_t)(kP.cur_b[0] - kP.critic_b[4] - 64) : 0u) +
                        (b >= 48 ? (uint32_t)(kP.cur_b[1] - kP.cur_b[0] - 128) : 0u) +
                        (b >= 64 ? (uint32_t)(kP.bcritic_w6 - kP.cur_b[1] - 64) : 0u);
    stage[kStageN - 1] = wt.gw.u4(4u * fo, 0u);
  }
  store<BF16, Sh::O3, RT>(h3, s_buf, TS3, q, lane);
  lds_barrier();

  f32x4 h4[RT][Sh::O4];
  run<S4>(w4, wt, kP.critic_w[3], kP.bcritic_w[3], LdsOperands{s_buf, TS3}, h4, q, lane);
  if constexpr (BF16) {
    uint4* st4 = reinterpret_cast<uint4*>(s_buf) + kTailAt;
#pragma unroll
    for (int i = 0; i < kStageN - 1; ++i) st4[i * kThreads + tid] = stage[i];
    st4[kTailW + (tid < kTailN - kTailW ? tid : kTailN - kTailW - 1)] = stage[kStageN - 1];
    // ---- tail: wave q evaluates the rest for row tile q alone -------------
    prefetch_next();
    // the row's action (clamped for the gather) and the MSE targets: the
    // next bar's features at this lane's outputs 16 i + 4 g + r of the
    // curiosity head, one 16-byte load each (rows start 4-byte aligned; the
    // row's last four where the four run past it, 48 .. 50 then moved down
    // one; outputs past the row are zero).  Without recycling the next bar's
    // features are also the first 51 elements of the episode's next state,
    // N rows on, which this launch holds for every step but its last: read
    // there, a group's targets are one contiguous run of state rows (read
    // again as states a little later) instead of a scattered feature row each.
    const int act = my_act[0] < 0 ? 0 : (my_act[0] >= kActions ? kActions - 1 : my_act[0]);
    const int64_t nrow = my_raw[0] + a.N;
    const float* fn = !a.bars && nrow < rows ? a.states + nrow * kState
                                             : a.features + (int64_t)(my_nbar[0] + 1) * kFeatures;
    f32x4 feat[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j0 = 16 * i + 4 * g;
      const int jl = j0 + 3 < kFeatures ? j0 : kFeatures - 4;
      const f32x4 v = *reinterpret_cast<const f32x4_a4*>(fn + jl);
      const bool shift = jl != j0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s1 = r < 3 ? v[r + 1] : 0.0f;
        feat[i][r] = j0 + r < kFeatures ? (shift ? s1 : v[r]) : 0.0f;
      }
    }
    // the action's one-hot columns of the curiosity input layer
    const float* oh = Wp + kP.bcur_onehot + act * 128 + 4 * g;
    f32x4 ohv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ohv[i] = *reinterpret_cast<const f32x4*>(oh + 16 * i);
    lds_barrier();  // every wave has read the third layer's output
    store<BF16, Sh::O4, RT>(h4, s_buf, TS4, q, lane);
    lds_barrier();

    const uint4* tw = reinterpret_cast<const uint4*>(s_buf) + kTailAt;
    const float* tb = reinterpret_cast<const float*>(tw + kTailW);
    // critic 128 -> 64: all four output tiles (weights [s][tile][lane])
    f32x4 h5[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h5[i] = *reinterpret_cast<const f32x4*>(tb + 16 * i + 4 * g);
    const uint4* x4 = reinterpret_cast<const uint4*>(s_buf) + q * TS4;
#pragma unroll
    for (int s = 0; s < S5; ++s) {
      const uint4 bx = x4[s * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) h5[i] = mfma_bf16(tw[(4 * s + i) * 64 + lane], bx, h5[i]);
    }
    // 64 -> 1 on the VALU: per output tile a dot product over the lane's
    // four units, reduced over the lane groups; tiles added in a fixed order
    float vp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 w6v = *reinterpret_cast<const f32x4*>(tb + 256 + 16 * i + 4 * g);
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part += w6v[r] * bf16_round(fmaxf(h5[i][r], 0.0f));
      part += lane_xor16f(part, lane);
      part += lane_xor32f(part, lane);
      vp[i] = part;
    }
    const float value = Wp[kP.critic_b6] + ((vp[0] + vp[1]) + (vp[2] + vp[3]));

    // curiosity layer 1: the row tile's state operands (all 8 output tiles),
    // plus the one-hot gather
    f32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = *reinterpret_cast<const f32x4*>(tb + 64 + 16 * i + 4 * g);
    const uint4* xs = reinterpret_cast<const uint4*>(s_opnd) + q * Sh::kOpTile;
#pragma unroll
    for (int s = 0; s < SC1; ++s) {
      const uint4 bx = xs[s * 64 + lane];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        c[i] = mfma_bf16(tw[1024 + (8 * s + i) * 64 + lane], bx, c[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] += ohv[i];
    // this row tile's state operands are read (by this wave only): the next
    // group's take their place (past the last group the values are unused)
    scatter_states(tid, v_states);

    // curiosity layer 2: the input never leaves the registers, since k-step
    // s of the packed order is output tiles 2s and 2s + 1 as this lane holds
    // them
    f32x4 pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = *reinterpret_cast<const f32x4*>(tb + 192 + 16 * i + 4 * g);
#pragma unroll
    for (int s = 0; s < SC2; ++s) {
      uint4 bx;
      bx.x = pack_bf16x2(fmaxf(c[2 * s][0], 0.0f), fmaxf(c[2 * s][1], 0.0f));
      bx.y = pack_bf16x2(fmaxf(c[2 * s][2], 0.0f), fmaxf(c[2 * s][3], 0.0f));
      bx.z = pack_bf16x2(fmaxf(c[2 * s + 1][0], 0.0f), fmaxf(c[2 * s + 1][1], 0.0f));
      bx.w = pack_bf16x2(fmaxf(c[2 * s + 1][2], 0.0f), fmaxf(c[2 * s + 1][3], 0.0f));
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = mfma_bf16(tw[2048 + (4 * s + i) * 64 + lane], bx, pr[i]);
    }
    begin<S1>(w1, wt, kP.critic_w[0], kP.bcritic_w[0], kP.critic_b[0], q, lane);
    lds_barrier();  // the tail's LDS reads are done; the next group's operands are written

    // MSE against the next bar's features, then step 10: reward = partial +
    // curiosity - risk
    float sq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float se = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = 16 * i + 4 * g + r < kFeatures ? pr[i][r] - feat[i][r] : 0.0f;
        se += d * d;
      }
      se += lane_xor16f(se, lane);
      se += lane_xor32f(se, lane);
      sq[i] = se;
    }
    const float sum = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    const float bonus = a.ep.curiosity_coef * (sum / (float)kFeatures);
    const float ex = s_env[act / 9];
    const float reward = (partial[0] + bonus) - a.ep.risk_coef * fabsf(ex);
    // one store per row (lane group 0) through buffer resources that end at
    // the last row present: the other lanes and rows past the end are
    // dropped by the range check, so no store sits behind a branch
    const int64_t left = rows - row0;
    const int nrec = 4 * (int)(left < RT * kRowsPerWave ? left : RT * kRowsPerWave);
    const uint32_t so = g == 0 ? 4u * (uint32_t)(q * kRowsPerWave + (lane & 15)) : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(
        __float_as_uint(value),
        __builtin_amdgcn_make_buffer_rsrc(a.values + row0, 0, nrec, 0x00020000), (int)so, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(
        __float_as_uint(reward),
        __builtin_amdgcn_make_buffer_rsrc(a.rewards + row0, 0, nrec, 0x00020000), (int)so, 0, 0);
    n_bad += (g == 0 && my_raw[0] < rows && (!isfinite(value) || !isfinite(reward))) ? 1u : 0u;
  } else {
  Stream<BF16, 1> w5;
  begin<S5>(w5, wt, kP.critic_w[4], kP.bcritic_w[4], kP.critic_b[4], q4, lane);
#pragma unroll
  for (int e = 0; e < ER; ++e)
    if (q + W * e < RT && g == 0) {
      const int v = my_act[e];
      s_act[(q + W * e) * kRowsPerWave + lane] = v < 0 ? 0 : (v >= kActions ? kActions - 1 : v);
      s_nbar[(q + W * e) * kRowsPerWave + lane] = my_nbar[e] + 1;
    }
  lds_barrier();
  // next-bar features of this wave's row tiles for the curiosity MSE: lane
  // holds features j0 .. j0 + 3, j0 = 16 q4 + 4g, one 16-byte load per row
  // (rows start 4-byte aligned) with no branch around it: the row's last
  // four where j0 + 3 lies past it (48 .. 50 are then moved down one; lanes
  // past the row keep zeros).  Without recycling they are read from the
  // episode's next state row, N rows on, for every step but the launch's
  // last (as in the bf16 tail).
  f32x4 feat[RTS];
  const int j0 = 16 * q4 + 4 * g;
  const int jl = j0 + 3 < kFeatures ? j0 : kFeatures - 4;
#pragma unroll
  for (int rt = 0; rt < RTS; ++rt) {
    const int64_t nrow = row0 + (rs0 + rt) * kRowsPerWave + (lane & 15) + a.N;
    const float* fn =
        !a.bars && nrow < rows
            ? a.states + nrow * kState
            : a.features + (int64_t)s_nbar[(rs0 + rt) * kRowsPerWave + (lane & 15)] * kFeatures;
    const f32x4 v = *reinterpret_cast<const f32x4_a4*>(fn + jl);
    const bool shift = jl != j0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s1 = r < 3 ? v[r + 1] : 0.0f;
      feat[rt][r] = j0 + r < kFeatures ? (shift ? s1 : v[r]) : 0.0f;
    }
  }
  store<BF16, Sh::O4, RT>(h4, s_buf, TS4, q, lane);
  lds_barrier();

  f32x4 h5[RTS][1];
  run<S5>(w5, wt, kP.critic_w[4], kP.bcritic_w[4], acts_s, h5, q4, lane);
  Stream<BF16, Sh::OC1, W> c1;
  begin<SC1>(c1, wt, kP.cur_w[0], kP.bcur_w[0], kP.cur_b[0], q, lane);
  {
    // 64 -> 1 on the VALU: this wave holds hidden units 16 q4 .. 16 q4 + 15
    const float* w6 = Wp + kP.critic_w6 + 16 * q4 + 4 * g;
    const f32x4 w6v = *reinterpret_cast<const f32x4*>(w6);
#pragma unroll
    for (int rt = 0; rt < RTS; ++rt) {
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part += w6v[r] * fmaxf(h5[rt][0][r], 0.0f);
      part += lane_xor16f(part, lane);
      part += lane_xor32f(part, lane);
      if (g == 0) s_part[0][rs0 + rt][q4][lane] = part;
    }
  }

  // ---- curiosity layer 1 (reads the state operands, not s_buf) ----------
  f32x4 c[RT][Sh::OC1];
  run<SC1, kFirstSteps>(c1, wt, kP.cur_w[0], kP.bcur_w[0], states_in, c, q, lane);
  Stream<BF16, 1> c2;
  begin<SC2>(c2, wt, kP.cur_w[1], kP.bcur_w[1], kP.cur_b[1], q4, lane);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int act = s_act[rt * kRowsPerWave + (lane & 15)];
    const float* oh = Wp + kP.cur_onehot + act * 128 + 4 * g;
#pragma unroll
    for (int i = 0; i < Sh::OC1; ++i)
      c[rt][i] += *reinterpret_cast<const f32x4*>(oh + 16 * (Sh::OC1 * q + i));
  }
  lds_barrier();  // critic input no longer read; value partials visible
  // the next group's state operands (the last reader of this group's was
  // the curiosity layer above); the final barrier makes them visible
  if (grp_next < groups) scatter_states(tid, v_states);
  float value[ER];
#pragma unroll
  for (int e = 0; e < ER; ++e) {
    const int rt = q + W * e < RT ? q + W * e : 0;
    value[e] = Wp[kP.critic_b6] + ((s_part[0][rt][0][lane & 15] + s_part[0][rt][1][lane & 15]) +
                                   (s_part[0][rt][2][lane & 15] + s_part[0][rt][3][lane & 15]));
  }
  store<BF16, Sh::OC1, RT>(c, s_buf, TS, q, lane);
  lds_barrier();

  // ---- curiosity layer 2, MSE against the next bar's features -------------
  f32x4 pr[RTS][1];
  run<SC2>(c2, wt, kP.cur_w[1], kP.bcur_w[1], acts_s, pr, q4, lane);
#pragma unroll
  for (int rt = 0; rt < RTS; ++rt) {
    float se = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * q4 + 4 * g + r;
      if (j < kFeatures) {
        const float d = pr[rt][0][r] - feat[rt][r];
        se += d * d;
      }
    }
    se += lane_xor16f(se, lane);
    se += lane_xor32f(se, lane);
    if (g == 0) s_part[1][rs0 + rt][q4][lane] = se;
  }
  lds_barrier();

  // ---- step 10: reward = partial + curiosity - risk (wave q: row tiles
  // q + W e) ---------------------------------------------------------------
#pragma unroll
  for (int e = 0; e < ER; ++e) {
    const int rt = q + W * e;
    if (rt < RT && g == 0 && my_raw[e] < rows) {
      const float sum = (s_part[1][rt][0][lane] + s_part[1][rt][1][lane]) +
                        (s_part[1][rt][2][lane] + s_part[1][rt][3][lane]);
      const float bonus = a.ep.curiosity_coef * (sum / (float)kFeatures);
      const float ex = s_env[s_act[rt * kRowsPerWave + lane] / 9];
      const float reward = (partial[e] + bonus) - a.ep.risk_coef * fabsf(ex);
      a.values[my_row[e]] = value[e];
      a.rewards[my_row[e]] = reward;
      if (a.counters && (!isfinite(value[e]) || !isfinite(reward))) atomicAdd(a.counters, 1u);
    }
  }
  }  // fp32 tail
  // the same value in every lane: keep the loop control scalar
  grp = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)grp_next) |
        ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(grp_next >> 32)) << 32);
  }  // row-tile groups
  if (n_bad && a.counters) atomicAdd(a.counters, n_bad);
}

__global__ void zero_u64_kernel(unsigned long long* p) { p[threadIdx.x] = 0ull; }

// Resident workgroups of a value kernel on the current device (all CUs at
// the kernel's occupancy), cached per device (callers on several host
// threads may fill an entry concurrently; they store the same value).
template <bool BF16>
int resident_groups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int known = cache[dev].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, value_kernel<BF16>,
                                                   ValueShape<BF16>::kThreads, 0) !=
          hipSuccess)
    return 0;
  const int groups = cus * (per_cu > 0 ? per_cu : 1);
  cache[dev].store(groups, std::memory_order_relaxed);
  return groups;
}

}  // namespace

int value_lds_bytes(bool bf16) {
  hipFuncAttributes at;
  const void* k = bf16 ? reinterpret_cast<const void*>(value_kernel<true>)
                       : reinterpret_cast<const void*>(value_kernel<false>);
  if (hipFuncGetAttributes(&at, k) != hipSuccess) return -1;
  return (int)at.sharedSizeBytes;
}

hipError_t launch_value(const ValueArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.L * a.N;
  if (rows <= 0) return hipSuccess;
  const int64_t tiles = (rows + kRowsPerWave - 1) / kRowsPerWave;
  const int RT = a.bf16 ? ValueShape<true>::RT : ValueShape<false>::RT;
  const int64_t groups = (tiles + RT - 1) / RT;
  const int resident = a.bf16 ? resident_groups<true>() : resident_groups<false>();
  if (resident <= 0) return hipErrorInvalidDevice;
  int64_t cap = resident;
  if (a.max_grid > 0 && a.max_grid < cap) cap = a.max_grid;
  const unsigned grid = (unsigned)(groups < cap ? groups : cap);
  if (!a.sched || a.lds_pad < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, st, a.sched);
  // (lds_pad reserves LDS the kernel does not use, which only limits where
  // and how many of its workgroups the dispatcher can place)
  const unsigned pad = (unsigned)a.lds_pad;
  if (a.bf16)
    hipLaunchKernelGGL(value_kernel<true>, dim3(grid), dim3(ValueShape<true>::kThreads), pad, st, a);
  else
    hipLaunchKernelGGL(value_kernel<false>, dim3(grid), dim3(ValueShape<false>::kThreads), pad, st, a);
  return hipGetLastError();
}

}  // namespace rl
