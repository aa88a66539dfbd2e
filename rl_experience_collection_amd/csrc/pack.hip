// Weight repacking: caller-layout [out, in] fp32 tensors -> the MFMA operand
// order of nets.hpp (per k-step, one contiguous block per cooperating wave).  Runs on the device, stream-ordered, at create and at
// every weight update.
#include "pack.hpp"

namespace rl {

namespace {

// One thread per packed float: pk[((s*kSplit + q)*64 + lane)*OTW + i].
__global__ void pack_layer_kernel(const float* __restrict__ W, int in, int ld, int out, int steps,
                                  int pad, int first, int otw, float* __restrict__ pk) {
  const int64_t total = (int64_t)(steps + pad) * kSplit * 64 * otw;  // incl. zero padding
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int i = (int)(idx % otw);
  const int lane = (int)((idx / otw) % 64);
  const int q = (int)((idx / ((int64_t)otw * 64)) % kSplit);
  const int s = (int)(idx / ((int64_t)otw * 64 * kSplit));
  const int o = 16 * (q * otw + i) + (lane & 15);
  const int g = lane >> 4;
  int k;
  bool ok;
  if (first == 2) {  // natural order: k = 4 s + g
    k = 4 * s + g;
    ok = s < steps;
  } else if (first) {
    k = kFirstSteps * g + s;
    ok = s < kFirstSteps;
  } else {
    k = 16 * (s >> 2) + 4 * g + (s & 3);
    ok = s < steps;
  }
  ok = ok && o < out && k < in;
  pk[idx] = ok ? W[(int64_t)o * ld + k] : 0.0f;
}

// bf16 form: pk[(((s*split + q)*64 + lane)*OTW + i)*8 + j], 8 bf16 per
// (k-step, lane, tile), k = kperm(s, lane / 16, j) of nets.hpp; `split`
// waves share a k-step, OTW = ot / split tiles each.
__global__ void pack_layer_bf16_kernel(const float* __restrict__ W, int in, int ld, int out,
                                       int steps, int pad, int first, int split, int otw,
                                       uint16_t* __restrict__ pk) {
  const int64_t total = (int64_t)(steps + pad) * split * 64 * otw * 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int j = (int)(idx % 8);
  const int i = (int)((idx / 8) % otw);
  const int lane = (int)((idx / (8 * (int64_t)otw)) % 64);
  const int q = (int)((idx / (8 * (int64_t)otw * 64)) % split);
  const int s = (int)(idx / (8 * (int64_t)otw * 64 * split));
  const int o = 16 * (q * otw + i) + (lane & 15);
  const int g = lane >> 4;
  const int k = first ? 32 * s + 8 * g + j : 16 * (2 * s + j / 4) + 4 * g + (j % 4);
  const bool ok = s < steps && o < out && k < in;
  pk[idx] = ok ? (uint16_t)bf16_bits(W[(int64_t)o * ld + k]) : (uint16_t)0;
}

// bf16-rounded copies (kept as fp32) of a plain array and of the curiosity
// one-hot columns.
__global__ void round_copy_kernel(const float* __restrict__ src, int n, float* __restrict__ dst) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) dst[j] = bf16_round(src[j]);
}
__global__ void pack_onehot_bf16_kernel(const float* __restrict__ W, float* __restrict__ oh) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kActions * 128) return;
  const int a = idx / 128, o = idx % 128;
  oh[idx] = bf16_round(W[(int64_t)o * (kState + kActions) + kState + a]);
}

__global__ void pack_bias_kernel(const float* __restrict__ b, int out, int padded,
                                 float* __restrict__ pb) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < padded) pb[j] = j < out ? b[j] : 0.0f;
}

// Transposed one-hot block of the curiosity input layer: oh[a][o] = W[o][54 + a].
__global__ void pack_onehot_kernel(const float* __restrict__ W, float* __restrict__ oh) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kActions * 128) return;
  const int a = idx / 128, o = idx % 128;
  oh[idx] = W[(int64_t)o * (kState + kActions) + kState + a];
}

__global__ void copy_kernel(const float* __restrict__ src, int n, float* __restrict__ dst) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) dst[j] = src[j];
}

hipError_t pack_layer(const float* W, const LayerDesc& d, int ld, float* pk, hipStream_t st) {
  const int64_t total = packed_layer_floats(d);
  hipLaunchKernelGGL(pack_layer_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, W,
                     d.in, ld, d.out, d.steps, d.pad, d.first, d.ot / kSplit, pk);
  return hipGetLastError();
}

hipError_t pack_layer_bf16(const float* W, const LayerDesc& d, int ld, float* pk, hipStream_t st,
                           int split = kSplit) {
  if (split < 1 || d.ot % split != 0) return hipErrorInvalidValue;
  const int64_t total = packed_layer_floats_bf16(d) * 2;  // bf16 elements
  hipLaunchKernelGGL(pack_layer_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     W, d.in, ld, d.out, d.steps, d.pad, d.first, split, d.ot / split,
                     reinterpret_cast<uint16_t*>(pk));
  return hipGetLastError();
}

hipError_t pack_bias(const float* b, const LayerDesc& d, float* pb, hipStream_t st) {
  const int out = d.out;
  const int padded = 16 * d.ot;
  hipLaunchKernelGGL(pack_bias_kernel, dim3((padded + 255) / 256), dim3(256), 0, st, b, out, padded,
                     pb);
  return hipGetLastError();
}

// The two head layers of a dueling Q-network as dense [out, in] matrices (see
// kQH1 / kQH2): h1 = [Wv1; Wa1] (128 x 128), h2 (64 x 128) with the
// advantage rows 0..44 over inputs 64..127 and the value row 45 over inputs
// 0..63.  Layout of `dst`: h1 weights, h1 bias (128), h2 weights, h2 bias (64).
constexpr int kHeadFloats = 128 * 128 + 128 + 64 * 128 + 64;
__global__ void assemble_heads_kernel(const float* __restrict__ wv1, const float* __restrict__ bv1,
                                      const float* __restrict__ wv2, const float* __restrict__ bv2,
                                      const float* __restrict__ wa1, const float* __restrict__ ba1,
                                      const float* __restrict__ wa2, const float* __restrict__ ba2,
                                      float* __restrict__ dst) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kHeadFloats) return;
  float v = 0.0f;
  if (idx < 128 * 128) {
    const int o = idx / 128, k = idx % 128;
    v = o < 64 ? wv1[o * 128 + k] : wa1[(o - 64) * 128 + k];
  } else if (idx < 128 * 128 + 128) {
    const int o = idx - 128 * 128;
    v = o < 64 ? bv1[o] : ba1[o - 64];
  } else if (idx < 128 * 128 + 128 + 64 * 128) {
    const int r = idx - (128 * 128 + 128);
    const int o = r / 128, k = r % 128;
    if (o < kActions && k >= 64) v = wa2[o * 64 + (k - 64)];
    else if (o == kQValueRow && k < 64) v = wv2[k];
  } else {
    const int o = idx - (128 * 128 + 128 + 64 * 128);
    v = o < kActions ? ba2[o] : (o == kQValueRow ? bv2[0] : 0.0f);
  }
  dst[idx] = v;
}

}  // namespace

size_t dqn_pack_scratch_floats() { return 2 * (size_t)kHeadFloats; }

hipError_t pack_dqn_weights(const float* const online[12], const float* const target[12],
                            const float* const cur[4], float* block, float* scratch,
                            hipStream_t st) {
  const DqnOffsets P = dqn_packed_offsets();
  hipError_t e = hipSuccess;
#define RL_TRY(x)           \
  do {                      \
    e = (x);                \
    if (e != hipSuccess) return e; \
  } while (0)
  for (int net = 0; net < 2; ++net) {
    const float* const* w = net == 0 ? online : target;
    if (!w) continue;  // keep the packed copy of this network
    float* heads = scratch + net * kHeadFloats;
    hipLaunchKernelGGL(assemble_heads_kernel, dim3((kHeadFloats + 255) / 256), dim3(256), 0, st,
                       w[4], w[5], w[6], w[7], w[8], w[9], w[10], w[11], heads);
    RL_TRY(hipGetLastError());
    const float* h1w = heads;
    const float* h1b = heads + 128 * 128;
    const float* h2w = h1b + 128;
    const float* h2b = h2w + 64 * 128;
    RL_TRY(pack_layer(w[0], kQ1, kQ1.in, block + P.w[net][0], st));
    RL_TRY(pack_bias(w[1], kQ1, block + P.b[net][0], st));
    RL_TRY(pack_layer(w[2], kQ2, kQ2.in, block + P.w[net][1], st));
    RL_TRY(pack_bias(w[3], kQ2, block + P.b[net][1], st));
    RL_TRY(pack_layer(h1w, kQH1, 128, block + P.w[net][2], st));
    RL_TRY(pack_bias(h1b, kQH1, block + P.b[net][2], st));
    RL_TRY(pack_layer(h2w, kQH2, 128, block + P.w[net][3], st));
    RL_TRY(pack_bias(h2b, kQH2, block + P.b[net][3], st));
  }
  if (cur) {
    RL_TRY(pack_layer(cur[0], kQC1, kState + kActions, block + P.cw[0], st));
    RL_TRY(pack_bias(cur[1], kQC1, block + P.cb[0], st));
    RL_TRY(pack_layer(cur[2], kQC2, kQC2.in, block + P.cw[1], st));
    RL_TRY(pack_bias(cur[3], kQC2, block + P.cb[1], st));
    hipLaunchKernelGGL(pack_onehot_kernel, dim3((kActions * 128 + 255) / 256), dim3(256), 0, st,
                       cur[0], block + P.c_onehot);
    RL_TRY(hipGetLastError());
  }
#undef RL_TRY
  return hipSuccess;
}

hipError_t pack_weights(const float* const actor[6], const float* const critic[12],
                        const float* const cur[4], float* block, hipStream_t st) {
  const PackedOffsets P = packed_offsets();
  hipError_t e = hipSuccess;
#define RL_TRY(x)           \
  do {                      \
    e = (x);                \
    if (e != hipSuccess) return e; \
  } while (0)
  for (int l = 0; l < 3; ++l) {
    RL_TRY(pack_layer(actor[2 * l], kActor[l], kActor[l].in, block + P.actor_w[l], st));
    RL_TRY(pack_bias(actor[2 * l + 1], kActor[l], block + P.actor_b[l], st));
  }
  for (int l = 0; l < 5; ++l) {
    RL_TRY(pack_layer(critic[2 * l], kCritic[l], kCritic[l].in, block + P.critic_w[l], st));
    RL_TRY(pack_bias(critic[2 * l + 1], kCritic[l], block + P.critic_b[l], st));
  }
  hipLaunchKernelGGL(copy_kernel, dim3(1), dim3(64), 0, st, critic[10], 64, block + P.critic_w6);
  RL_TRY(hipGetLastError());
  hipLaunchKernelGGL(copy_kernel, dim3(1), dim3(64), 0, st, critic[11], 1, block + P.critic_b6);
  RL_TRY(hipGetLastError());
  RL_TRY(pack_layer(cur[0], kCur[0], kState + kActions, block + P.cur_w[0], st));
  RL_TRY(pack_bias(cur[1], kCur[0], block + P.cur_b[0], st));
  RL_TRY(pack_layer(cur[2], kCur[1], kCur[1].in, block + P.cur_w[1], st));
  RL_TRY(pack_bias(cur[3], kCur[1], block + P.cur_b[1], st));
  hipLaunchKernelGGL(pack_onehot_kernel, dim3((kActions * 128 + 255) / 256), dim3(256), 0, st, cur[0],
                     block + P.cur_onehot);
  RL_TRY(hipGetLastError());
  // bf16 forms
  for (int l = 0; l < 3; ++l) {
    RL_TRY(pack_layer_bf16(actor[2 * l], kActorB[l], kActorB[l].in, block + P.bact_w[l], st));
    RL_TRY(pack_bias(actor[2 * l + 1], kActorB[l], block + P.bact_b[l], st));
  }
  // the value kernel's wide layers split over its waves, the two 4-tile
  // layers (critic 128 -> 64, curiosity 128 -> 51) over 4
  for (int l = 0; l < 5; ++l)
    RL_TRY(pack_layer_bf16(critic[2 * l], kCriticB[l], kCriticB[l].in, block + P.bcritic_w[l], st,
                           l < 4 ? value_waves(true) : kSplit));
  RL_TRY(pack_layer_bf16(cur[0], kCurB[0], kState + kActions, block + P.bcur_w[0], st,
                         value_waves(true)));
  RL_TRY(pack_layer_bf16(cur[2], kCurB[1], kCurB[1].in, block + P.bcur_w[1], st, kSplit));
  hipLaunchKernelGGL(round_copy_kernel, dim3(1), dim3(64), 0, st, critic[10], 64, block + P.bcritic_w6);
  RL_TRY(hipGetLastError());
  hipLaunchKernelGGL(pack_onehot_bf16_kernel, dim3((kActions * 128 + 255) / 256), dim3(256), 0, st,
                     cur[0], block + P.bcur_onehot);
  RL_TRY(hipGetLastError());
#undef RL_TRY
  return hipSuccess;
}

}  // namespace rl
