// Packed network weights, environment constants and the MFMA layer
// evaluator shared by the actor-rollout and value kernels.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace rl {

// ---------------------------------------------------------------------------
// Layers are evaluated by kSplit cooperating waves on the same 16 rows: wave
// q computes output tiles [q*OTW, (q+1)*OTW) with OTW = OT / kSplit.  The
// packed A operands of one layer are laid out so that each wave reads one
// contiguous block per k-step:
//   pk[((s * kSplit + q) * 64 + lane) * OTW + i] = W[o][k]
//   o = 16 * (q * OTW + i) + lane % 16,   k = kperm(s, lane / 16)
// (zero when o >= OUT or k >= IN).  First layers (state input) use 16
// k-steps with kperm(s, g) = 14 g + s (s < 14; steps 14, 15 are zero), the
// actor's with kperm(s, g) = 4 s + g; chained layers use
// kperm(s, g) = 16 (s / 4) + 4 g + s % 4, S = IN / 4.
// Bias: pb[16 * ot + j] = b[16 * ot + j], zero padded to 16 * OT.
// ---------------------------------------------------------------------------
constexpr int kSplit = 4;

struct LayerDesc {
  int in, out, steps, first, ot;  // ot = out tiles (a multiple of kSplit)
  int pad;                         // zero k-steps after the layer (ring prefetch reach)
};

// Row tiles of 16 rows per value-kernel work item: every work item streams
// the whole critic and curiosity weight block once, so rows per work item
// set the weight-stream bytes per row.
#ifndef RL_VALUE_RT_F32
#define RL_VALUE_RT_F32 2
#endif
#ifndef RL_VALUE_RT_BF16
#define RL_VALUE_RT_BF16 8
#endif
__host__ __device__ constexpr int value_row_tiles(bool bf16) {
  return bf16 ? RL_VALUE_RT_BF16 : RL_VALUE_RT_F32;
}
// Waves of a value-kernel workgroup.  The wide layers split their output
// tiles over all of them; bf16 uses 8 waves (one workgroup per CU, 128 rows
// in LDS), so each 16-byte weight operand feeds 8 row tiles: the stream of
// operands through the CU's vector-memory data path is half that of four
// waves with 4 row tiles each, at the same accumulator count per wave.
__host__ __device__ constexpr int value_waves(bool bf16) { return bf16 ? 8 : kSplit; }

// Weight-ring slots of a streamed layer (value kernel): layers with few
// output tiles per wave issue little MFMA work per k-step, so they keep more
// steps in flight (fp32: the whole layer for one tile per wave; bf16: up to
// 8 steps of 16-byte operands).  Streamed layers need no zero padding.
__host__ __device__ constexpr int ring_depth(bool bf16, int otw) {
  return bf16 ? (otw >= 4 ? 3 : otw == 3 ? 4 : otw == 2 ? 6 : 8)
              : (otw >= 4 ? 4 : otw == 2 ? 16 : 32);
}

// Actor: 54 -> 128 -> 64 -> 45 (PPO CUDA Pipeline Design, Weight Layout).
// Its first layer takes the state in natural order (first = 2: k = 4 s + g),
// so the portfolio inputs k >= 48 sit in k-steps 12 and 13 only.
constexpr LayerDesc kActor[3] = {{54, 128, 16, 2, 8, 0}, {128, 64, 32, 0, 4, 0}, {64, 45, 16, 0, 4, 0}};
constexpr int kActorOut1 = 128;  // first-layer outputs of the actor
// Critic: 54 -> 512 -> 384 -> 256 -> 128 -> 64 (-> 1 handled on the VALU).
constexpr LayerDesc kCritic[5] = {{54, 512, 16, 1, 32, 0},
                                  {512, 384, 128, 0, 24, 0},
                                  {384, 256, 96, 0, 16, 0},
                                  {256, 128, 64, 0, 8, 0},
                                  {128, 64, 32, 0, 4, 0}};
// Curiosity forward model: 54 dense inputs (+45 one-hot, gathered) -> 128 -> 51.
constexpr LayerDesc kCur[2] = {{54, 128, 16, 1, 8, 0}, {128, 51, 32, 0, 4, 0}};

// bf16 forms (v_mfma_f32_16x16x32_bf16): a k-step covers 32 inputs, 8 per
// lane group.  First layers: kperm(s, g, j) = 32 s + 8 g + j (54 -> 2 steps).
// Chained layers: kperm(s, g, j) = 16 (2 s + j / 4) + 4 g + j % 4, i.e. the
// output tiles 2s and 2s+1 of the previous layer form k-step s.
constexpr LayerDesc kActorB[3] = {{54, 128, 2, 1, 8, 0}, {128, 64, 4, 0, 4, 0}, {64, 45, 2, 0, 4, 0}};
constexpr LayerDesc kCriticB[5] = {{54, 512, 2, 1, 32, 0},
                                   {512, 384, 16, 0, 24, 0},
                                   {384, 256, 12, 0, 16, 0},
                                   {256, 128, 8, 0, 8, 0},
                                   {128, 64, 4, 0, 4, 0}};
constexpr LayerDesc kCurB[2] = {{54, 128, 2, 1, 8, 0}, {128, 51, 4, 0, 4, 0}};

// Packed weights of a layer, plus d.pad zero k-steps (the DQN's first layers
// stream 16 k-steps for their 14).
__host__ __device__ constexpr int64_t packed_layer_floats(const LayerDesc& d) {
  return (int64_t)(d.steps + d.pad) * 64 * d.ot;
}
// bf16 layer: 8 bf16 (16 bytes, 4 float slots) per lane, tile and k-step.
__host__ __device__ constexpr int64_t packed_layer_floats_bf16(const LayerDesc& d) {
  return (int64_t)(d.steps + d.pad) * 64 * d.ot * 4;
}

struct PackedOffsets {
  // fp32 actor layers and biases (loaded into registers by the rollout kernel)
  int64_t actor_w[3], actor_b[3];
  int64_t critic_w[5], critic_b[5], critic_w6, critic_b6;
  int64_t cur_w[2], cur_b[2], cur_onehot;
  // bf16 forms: the actor layers with their own copy of the biases, the
  // bf16 critic and curiosity layers (biases shared with the fp32 block),
  // and bf16-rounded copies (as fp32) of the critic's 64 -> 1 row and of the
  // curiosity one-hot columns
  int64_t bact_w[3], bact_b[3];
  int64_t bcritic_w[5], bcur_w[2], bcritic_w6, bcur_onehot;
  int64_t total;
};

__host__ __device__ constexpr int64_t align64(int64_t x) { return (x + 63) / 64 * 64; }

__host__ __device__ constexpr PackedOffsets packed_offsets() {
  PackedOffsets p{};
  int64_t off = 0;
  for (int l = 0; l < 3; ++l) {
    p.actor_w[l] = off;
    off = align64(off + packed_layer_floats(kActor[l]));
  }
  for (int l = 0; l < 3; ++l) {
    p.actor_b[l] = off;
    off = align64(off + 16 * kActor[l].ot);
  }
  for (int l = 0; l < 5; ++l) {
    p.critic_w[l] = off;
    off = align64(off + packed_layer_floats(kCritic[l]));
  }
  for (int l = 0; l < 5; ++l) {
    p.critic_b[l] = off;
    off = align64(off + 16 * kCritic[l].ot);
  }
  p.critic_w6 = off;
  off = align64(off + 64);
  p.critic_b6 = off;
  off = align64(off + 1);
  for (int l = 0; l < 2; ++l) {
    p.cur_w[l] = off;
    off = align64(off + packed_layer_floats(kCur[l]));
  }
  for (int l = 0; l < 2; ++l) {
    p.cur_b[l] = off;
    off = align64(off + 16 * kCur[l].ot);
  }
  p.cur_onehot = off;
  off = align64(off + 45 * 128);
  for (int l = 0; l < 3; ++l) {
    p.bact_w[l] = off;
    off = align64(off + packed_layer_floats_bf16(kActorB[l]));
  }
  for (int l = 0; l < 3; ++l) {
    p.bact_b[l] = off;
    off = align64(off + 16 * kActorB[l].ot);
  }
    for (int l = 0; l < 5; ++l) {
    p.bcritic_w[l] = off;
    off = align64(off + packed_layer_floats_bf16(kCriticB[l]));
  }
  for (int l = 0; l < 2; ++l) {
    p.bcur_w[l] = off;
    off = align64(off + packed_layer_floats_bf16(kCurB[l]));
  }
  p.bcritic_w6 = off;
  off = align64(off + 64);
  p.bcur_onehot = off;
  off = align64(off + 45 * 128);
  p.total = off;
  return p;
}

// ---------------------------------------------------------------------------
// DQN collection ("GPU Pipeline Phase 2b", Kernel Components 1, with the
// configured widths): a dueling Q-network, online and target copies, and the
// curiosity forward model, all fp32.  The two heads share their input, so
// each network is four streamed layers:
//   Q1  54 -> 256 (ReLU)   state operands in natural order (first = 2),
//                          14 k-steps packed plus 2 zero steps so the
//                          stream runs whole groups of 4
//   Q2  256 -> 128 (ReLU)
//   QH1 128 -> 128 (ReLU)  [value head 1 (outputs 0..63); advantage head 1
//                          (outputs 64..127)]
//   QH2 128 -> 64          outputs 0..44 the advantages (from inputs
//                          64..127), output 45 the value (from inputs
//                          0..63), 46..63 zero
// and the curiosity model is the dense state part of its first layer plus a
// column gather of the action's one-hot weights, then 128 -> 51.
constexpr LayerDesc kQ1 = {54, 256, 14, 2, 16, 2};
constexpr LayerDesc kQ2 = {256, 128, 64, 0, 8, 0};
constexpr LayerDesc kQH1 = {128, 128, 32, 0, 8, 0};
constexpr LayerDesc kQH2 = {128, 64, 32, 0, 4, 0};
constexpr LayerDesc kQC1 = {54, 128, 14, 2, 8, 2};
constexpr LayerDesc kQC2 = {128, 51, 32, 0, 4, 0};
constexpr int kQValueRow = 45;  // QH2 output holding the value

struct DqnOffsets {
  int64_t w[2][4], b[2][4];  // [online, target][Q1, Q2, QH1, QH2]
  int64_t cw[2], cb[2], c_onehot;
  int64_t total;
};

__host__ __device__ constexpr DqnOffsets dqn_packed_offsets() {
  DqnOffsets p{};
  const LayerDesc ls[4] = {kQ1, kQ2, kQH1, kQH2};
  int64_t off = 0;
  for (int net = 0; net < 2; ++net) {
    for (int l = 0; l < 4; ++l) {
      p.w[net][l] = off;
      off = align64(off + packed_layer_floats(ls[l]));
    }
    for (int l = 0; l < 4; ++l) {
      p.b[net][l] = off;
      off = align64(off + 16 * ls[l].ot);
    }
  }
  p.cw[0] = off;
  off = align64(off + packed_layer_floats(kQC1));
  p.cw[1] = off;
  off = align64(off + packed_layer_floats(kQC2));
  p.cb[0] = off;
  off = align64(off + 16 * kQC1.ot);
  p.cb[1] = off;
  off = align64(off + 16 * kQC2.ot);
  p.c_onehot = off;
  off = align64(off + 45 * 128);
  p.total = off;
  return p;
}

// State element held by lane group g at first-layer k-step slot s (16 slots
// per lane): fp32 form k = 14 g + s (s < 14), bf16 form k = 32 (s / 8) + 8 g
// + s % 8.  Values for k >= 54 are zero.
template <bool BF16>
__host__ __device__ constexpr int state_k(int g, int s) {
  return BF16 ? 32 * (s / 8) + 8 * g + (s % 8) : (s < 14 ? 14 * g + s : 1 << 20);
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

// The exposure and cost-rate tables as a small LDS array (exposure of a/9
// at [0, 5), cost rate of (a%9)/3 at [5, 8)).  Selected with a runtime index
// from the kernel argument they would become a load from kernel-argument
// memory, whose wait also drains every outstanding load and store.
constexpr int kEnvTable = 8;
__device__ __forceinline__ void fill_env_table(const EnvParams& p, float* t, int tid) {
  if (tid < kEnvTable) {
    const float v[kEnvTable] = {p.ex0, p.ex1, p.ex2, p.ex3, p.ex4, p.cost0, p.cost1, p.cost2};
    float x = v[0];
#pragma unroll
    for (int i = 1; i < kEnvTable; ++i) x = tid == i ? v[i] : x;
    t[tid] = x;
  }
}

// OTW consecutive floats of a lane's packed block (OTW in 1, 2, 4, 6, 8).
template <int OTW>
__device__ __forceinline__ void load_operands(const float* p, float (&a)[OTW]) {
  if constexpr (OTW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < OTW; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
      a[i] = v[0]; a[i + 1] = v[1]; a[i + 2] = v[2]; a[i + 3] = v[3];
    }
  } else if constexpr (OTW % 2 == 0) {
#pragma unroll
    for (int i = 0; i < OTW; i += 2) {
      const float2 v = *reinterpret_cast<const float2*>(p + i);
      a[i] = v.x; a[i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < OTW; ++i) a[i] = p[i];
  }
}

// ---------------------------------------------------------------------------
// ReLU this wave's accumulators into its tiles of the shared buffer.
template <int OTW>
__device__ __forceinline__ void relu_store(const f32x4 (&acc)[OTW], f32x4* buf, int q, int lane) {
#pragma unroll
  for (int i = 0; i < OTW; ++i) {
    f32x4 v = acc[i];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = fmaxf(v[r], 0.0f);
    buf[(q * OTW + i) * 64 + lane] = v;
  }
}

// ReLU, round to bf16 and store this wave's tiles as the next layer's k-step
// operands: tile t lands in half t % 2 of k-step t / 2.
template <int OTW>
__device__ __forceinline__ void relu_store_bf16(const f32x4 (&acc)[OTW], uint4* bufb, int q,
                                                int lane) {
  uint2* half = reinterpret_cast<uint2*>(bufb);
#pragma unroll
  for (int i = 0; i < OTW; ++i) {
    const int t = q * OTW + i;
    const f32x4 v = acc[i];
    uint2 w;
    w.x = pack_bf16x2(fmaxf(v[0], 0.0f), fmaxf(v[1], 0.0f));
    w.y = pack_bf16x2(fmaxf(v[2], 0.0f), fmaxf(v[3], 0.0f));
    half[((t >> 1) * 64 + lane) * 2 + (t & 1)] = w;
  }
}

// ---------------------------------------------------------------------------
// Weight stream of one layer for a wave that evaluates RT row tiles (16 rows
// each) at once: every A operand loaded from global memory feeds RT MFMAs,
// which divides the weight traffic per flop by RT.  The ring has D slots
// (k-step s in slot s % D) and runs D - 1 steps ahead; the last group of D
// steps is peeled so no load reaches past the layer.  stream_begin loads the
// bias tiles and the first min(D - 1, S) k-steps; callers issue it for layer
// j + 1 before the barriers and stores that end layer j, so those loads are
// in flight while the waves synchronise.  B operands come from a loader
// (LDS operand layout, or the raw state rows for first layers) and are read
// one group of steps ahead.
// ---------------------------------------------------------------------------
template <bool BF16, int OTW, int D, int SPLIT = kSplit>
struct WeightStream {
  using Op = typename std::conditional<BF16, uint4, float>::type;
  static constexpr int kStep = SPLIT * 64 * OTW;  // Op elements per k-step (SPLIT waves)
  Op a[D][OTW];
  f32x4 bias[OTW];
};

template <bool BF16, int OTW, int SPLIT = kSplit>
using Stream = WeightStream<BF16, OTW, ring_depth(BF16, OTW), SPLIT>;

// Weight loads through a buffer resource over the packed block: a 32-bit
// per-lane byte offset (one VGPR per layer) plus a wave-uniform byte offset
// (SGPR) for the k-step and tile, so the streams need no 64-bit addresses.
using BufRsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ BufRsrc weights_rsrc(const float* block, uint32_t bytes) {
  // raw buffer (stride 0), 32-bit dword format word of the gfx9 family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(block), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload_u4(BufRsrc r, uint32_t vo, uint32_t so) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int OTW>
__device__ __forceinline__ void bload_operands(BufRsrc r, uint32_t vo, uint32_t so,
                                               float (&a)[OTW]) {
  if constexpr (OTW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < OTW; i += 4) {
      const uint4 v = bload_u4(r, vo, so + 4u * i);
      a[i] = __uint_as_float(v.x); a[i + 1] = __uint_as_float(v.y);
      a[i + 2] = __uint_as_float(v.z); a[i + 3] = __uint_as_float(v.w);
    }
  } else if constexpr (OTW % 2 == 0) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < OTW; i += 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so + 4u * i, 0);
      a[i] = __uint_as_float(v.x); a[i + 1] = __uint_as_float(v.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < OTW; ++i)
      a[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so + 4u * i, 0));
  }
}

// Weight source of a streamed layer: byte offsets (lane part + wave-uniform
// step part) into the packed block in global memory, through the buffer
// resource.
struct GlobalWeights {
  BufRsrc rs;
  template <int OTW>
  __device__ __forceinline__ void f32(uint32_t lane_b, uint32_t step_b, float (&a)[OTW]) const {
    bload_operands<OTW>(rs, lane_b, step_b, a);
  }
  __device__ __forceinline__ uint4 u4(uint32_t lane_b, uint32_t step_b) const {
    return bload_u4(rs, lane_b, step_b);
  }
};
// pk_b: byte offset of the layer's packed weights in the block; pb: biases.
template <int S, bool BF16, int OTW, int D, int SPLIT, class WS>
__device__ __forceinline__ void stream_begin(WeightStream<BF16, OTW, D, SPLIT>& st, const WS& ws,
                                             uint32_t pk_b, const float* pb, int q, int lane) {
  constexpr uint32_t kStepB = WeightStream<BF16, OTW, D, SPLIT>::kStep * (BF16 ? 16u : 4u);
  constexpr int kFirst = D - 1 < S ? D - 1 : S;
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < OTW; ++i)
    st.bias[i] = *reinterpret_cast<const f32x4*>(pb + 16 * (q * OTW + i) + 4 * g);
  const uint32_t lane_b = (uint32_t)((q * 64 + lane) * OTW) * (BF16 ? 16u : 4u);
#pragma unroll
  for (int j = 0; j < kFirst; ++j) {
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < OTW; ++i) st.a[j][i] = ws.u4(lane_b, pk_b + j * kStepB + 16u * i);
    } else {
      ws.template f32<OTW>(lane_b, pk_b + j * kStepB, st.a[j]);
    }
  }
}

// B operands in the LDS operand layout: fp32 group of 4 k-steps / bf16 k-step
// grp of row tile rt at buf[rt * tile_stride + grp * 64 + lane].
struct LdsOperands {
  const f32x4* buf;
  int tile_stride;
  __device__ __forceinline__ f32x4 f32(int rt, int grp, int lane) const {
    return buf[rt * tile_stride + grp * 64 + lane];
  }
  __device__ __forceinline__ uint4 bf16(int rt, int grp, int lane) const {
    return reinterpret_cast<const uint4*>(buf)[rt * tile_stride + grp * 64 + lane];
  }
};

// fp32: S k-steps of 4 inputs (S % D == 0); a row tile's f32x4 B operand
// covers a group of 4 steps, read one group ahead.  Steps from SK on carry
// only zero padding (first layers: 54 inputs in 14 of 16 steps): their
// weights stream with the rest but issue no MFMA.
template <int S, int OTW, int D, int RT, int SK = S, int SPLIT, class WS, class BL>
__device__ __forceinline__ void stream_layer(WeightStream<false, OTW, D, SPLIT>& st, const WS& ws,
                                             uint32_t pk_b, const BL& bl, f32x4 (&acc)[RT][OTW],
                                             int q, int lane) {
  static_assert(D % 4 == 0 && S % D == 0, "whole groups of D steps");
  static_assert(SK > S - D && SK <= S, "padding only in the last group");
  constexpr int KT = S / D;
  constexpr int G = S / 4;
  constexpr uint32_t kStepB = WeightStream<false, OTW, D, SPLIT>::kStep * 4u;
  const uint32_t lane_b = (uint32_t)((q * 64 + lane) * OTW) * 4u;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < OTW; ++i) acc[rt][i] = st.bias[i];
  f32x4 b[RT], bn[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) b[rt] = bl.f32(rt, 0, lane);
  auto group = [&](int kt, auto last) {
    constexpr bool LAST = decltype(last)::value;
    const uint32_t wk = pk_b + (uint32_t)(D * kt + D - 1) * kStepB;
#pragma unroll
    for (int r = 0; r < D; ++r) {
      if (!LAST || r == 0) ws.template f32<OTW>(lane_b, wk + r * kStepB, st.a[(r + D - 1) % D]);
      if (r % 4 == 0 && !(LAST && r / 4 == D / 4 - 1)) {
        const int gn = kt * (D / 4) + r / 4 + 1;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) bn[rt] = bl.f32(rt, gn < G ? gn : G - 1, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!LAST || D * (S / D - 1) + r < SK) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < OTW; ++i)
            acc[rt][i] = mfma4(st.a[r][i], b[rt][r % 4], acc[rt][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (r % 4 == 3) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) b[rt] = bn[rt];
      }
    }
  };
#pragma unroll 1
  for (int kt = 0; kt < KT - 1; ++kt) group(kt, std::false_type{});
  group(KT - 1, std::true_type{});
}

// bf16: S k-steps of 32 inputs; one uint4 of B per row tile and step.
template <int S, int OTW, int D, int RT, int SPLIT, class WS, class BL>
__device__ __forceinline__ void stream_layer(WeightStream<true, OTW, D, SPLIT>& st, const WS& ws,
                                             uint32_t pk_b, const BL& bl, f32x4 (&acc)[RT][OTW],
                                             int q, int lane) {
  constexpr int KT = S / D;
  constexpr int TAIL = S % D;
  constexpr uint32_t kStepB = WeightStream<true, OTW, D, SPLIT>::kStep * 16u;
  const uint32_t lane_b = (uint32_t)((q * 64 + lane) * OTW) * 16u;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < OTW; ++i) acc[rt][i] = st.bias[i];
  uint4 b[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) b[rt] = bl.bf16(rt, 0, lane);
  // one step: weights of step s + D - 1 (when inside the layer), then per
  // row tile the MFMAs of step s from slot `slot` followed by the reload of
  // that tile's B operand with step s + 1 (one register set for B: the
  // reloads spread over the step, each a step ahead of its use)
  auto step = [&](int s, int slot, uint32_t wsrc, bool load_w, bool load_b) {
    if (load_w) {
#pragma unroll
      for (int i = 0; i < OTW; ++i) st.a[(slot + D - 1) % D][i] = ws.u4(lane_b, wsrc + 16u * i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < OTW; ++i) {
        acc[rt][i] = mfma_bf16(st.a[slot][i], b[rt], acc[rt][i]);
        // (the MFMA is issued here: without this the compiler may defer the
        // MFMAs of a fully prefetched layer past all its B reads, which then
        // all stay live)
        asm volatile("" : "+v"(acc[rt][i]));
      }
      // (the scheduling barrier does not order memory reads: the empty asm
      // keeps every operand load in program order, so the B operands of
      // later steps cannot be read early and held)
      asm volatile("" ::: "memory");
      if (load_b) b[rt] = bl.bf16(rt, s + 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (KT > 0) {
#pragma unroll 1
    for (int kt = 0; kt < KT - 1; ++kt) {
      const uint32_t wk = pk_b + (uint32_t)(D * kt + D - 1) * kStepB;
#pragma unroll
      for (int r = 0; r < D; ++r) step(D * kt + r, r, wk + r * kStepB, true, true);
    }
    const uint32_t wk = pk_b + (uint32_t)(D * (KT - 1) + D - 1) * kStepB;
#pragma unroll
    for (int r = 0; r < D; ++r)
      step(D * (KT - 1) + r, r, wk + r * kStepB, r <= TAIL, D * (KT - 1) + r + 1 < S);
  }
  // remaining steps (S % D): already in slots 0 .. TAIL-1
#pragma unroll
  for (int r = 0; r < TAIL; ++r) step(D * KT + r, r, pk_b, false, D * KT + r + 1 < S);
}

// ReLU store of RT row tiles (row tile rt at buf + rt * tile_stride).
template <int OTW, int RT>
__device__ __forceinline__ void relu_store_tiles(const f32x4 (&acc)[RT][OTW], f32x4* buf,
                                                 int tile_stride, int q, int lane) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) relu_store<OTW>(acc[rt], buf + rt * tile_stride, q, lane);
}
template <int OTW, int RT>
__device__ __forceinline__ void relu_store_tiles_bf16(const f32x4 (&acc)[RT][OTW], uint4* buf,
                                                      int tile_stride, int q, int lane) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) relu_store_bf16<OTW>(acc[rt], buf + rt * tile_stride, q, lane);
}

}  // namespace rl
