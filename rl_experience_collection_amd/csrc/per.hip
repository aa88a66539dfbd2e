// Prioritized replay on the device ("GPU-Resident Prioritized Experience
// Replay", Sampling Kernels: proportional sampling, IS weights, gather,
// priority update; Error Handling: the NaN/Inf clamp).
//
// Proportional sampling picks, for a uniform u in [0, 1), the first k whose
// inclusive prefix sum of priorities exceeds u * total.  Instead of writing
// the full prefix-sum array (8 bytes per priority) and binary-searching it,
// the priorities are cut into blocks of 2048 (one wave, 32 contiguous
// priorities per lane):
//   1. block_sums_kernel: one wave per block stages the block through LDS
//      with coalesced loads, sums each lane's 32 priorities in order (fp64)
//      and scans the 64 lane sums; it keeps the 64 in-block lane prefixes,
//      and the block's total is the scan's last lane;
//   2. block_scan_kernel: one workgroup turns the block totals into
//      inclusive block prefixes (fp64, fixed order);
//   3. sample_kernel: one wave per draw finds the block with a 64-way search
//      over the block prefixes, reads that block's 64 lane prefixes, and the
//      lane whose range holds the target loads and walks its 32 priorities;
//      the raw weight (n p / T)^-beta is fp64;
//   4. weights_kernel: one workgroup divides by the batch's largest weight.
// So each call reads the priorities once (4 bytes each), writes 8 bytes per
// 32 of them, and reads about 1.7 KB per draw; every sum is formed in a
// fixed order: results are deterministic.
// Negative and NaN priorities count as zero; a total that is not positive
// and finite gives uniform draws floor(u n) with weight 1.  Draws are 53-bit
// uniforms from Philox (counter (draw, 0, 4, 0), key = the seed).
#include "per.hpp"

#include <math.h>

namespace rl {

namespace {

constexpr int kLanes = 64;
constexpr int kPerLane = kPerBlock / kLanes;  // 32 contiguous priorities per lane
constexpr int kStride = kPerLane + 1;         // LDS row stride (bank-conflict padding)

__device__ __forceinline__ double per_value(float p) { return p > 0.0f ? (double)p : 0.0; }

__device__ __forceinline__ double per_uniform(uint64_t seed, uint32_t draw) {
  const uint4 r = philox10(make_uint4(draw, 0u, 4u, 0u), (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t m = ((uint64_t)r.x << 21) | (uint64_t)(r.y >> 11);
  return (double)m * (1.0 / 9007199254740992.0);
}

// Inclusive scan over the 64 lanes of a wave, in a fixed order.
__device__ __forceinline__ double wave_scan(double x, int lane) {
#pragma unroll
  for (int d = 1; d < kLanes; d <<= 1) {
    const double y = __shfl_up(x, d, kLanes);
    if (lane >= d) x += y;
  }
  return x;
}

// Stage block `blk` of the priorities into this wave's LDS rows (lane l's 32
// priorities at row l), loads coalesced, past-the-end entries zero.
// (the resource starts at the block; the wave's own LDS rows are complete
// and visible to all its lanes on return)
__device__ __forceinline__ void stage_block(__amdgpu_buffer_rsrc_t rs, float* rows, int lane) {
  float v[kPerLane];  // all 32 loads in flight before the first LDS write
#pragma unroll
  for (int j = 0; j < kPerLane; ++j)
    v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (j * kLanes + lane), 0, 0));
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int e = j * kLanes + lane;  // element of the block
    rows[(e / kPerLane) * kStride + (e % kPerLane)] = v[j];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const float* p, int64_t n, int64_t blk) {
  const int64_t first = blk * kPerBlock;
  const int64_t left = n - first;
  const int64_t count = left < kPerBlock ? left : kPerBlock;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p + first), 0, (int)(4 * count),
                                           0x00020000);
}

// This lane's in-order sum of its 32 staged priorities.
__device__ __forceinline__ double lane_sum(const float* rows, int lane) {
  double s = 0.0;
#pragma unroll 8
  for (int j = 0; j < kPerLane; ++j) s += per_value(rows[lane * kStride + j]);
  return s;
}

__global__ __launch_bounds__(256) void block_sums_kernel(const float* __restrict__ p, int64_t n,
                                                         int64_t nblocks, double* __restrict__ sums,
                                                         double* __restrict__ lanes) {
  __shared__ float s_rows[4][kLanes * kStride];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t blk = (int64_t)blockIdx.x * 4 + w;
  if (blk >= nblocks) return;  // wave-uniform; no workgroup barrier below
  float* rows = s_rows[w];
  stage_block(block_rsrc(p, n, blk), rows, lane);
  const double incl = wave_scan(lane_sum(rows, lane), lane);
  lanes[blk * kLanes + lane] = incl;
  if (lane == kLanes - 1) sums[blk] = incl;
}

// The 32 priorities of lane `lane` of a block (zeros past the end).
__device__ __forceinline__ void lane_priorities(__amdgpu_buffer_rsrc_t rs, int lane,
                                                float (&v)[kPerLane]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < kPerLane; i += 4) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, 4u * (lane * kPerLane + i), 0, 0);
    v[i] = __uint_as_float(x.x);
    v[i + 1] = __uint_as_float(x.y);
    v[i + 2] = __uint_as_float(x.z);
    v[i + 3] = __uint_as_float(x.w);
  }
}

// One workgroup: sums[0..nblocks) -> inclusive prefixes, in a fixed order:
// thread t owns a contiguous run of blocks, the 1024 run totals are scanned
// by wave scans and a scan of the 16 wave totals.
__global__ __launch_bounds__(1024) void block_scan_kernel(double* __restrict__ sums, int64_t nblocks) {
  __shared__ double s_wave[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t per = (nblocks + 1023) / 1024;
  const int64_t lo = t * per, hi = lo + per < nblocks ? lo + per : nblocks;
  double run = 0.0;
  for (int64_t i = lo; i < hi; ++i) run += sums[i];
  const double incl = wave_scan(run, lane);
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  if (w == 0) {
    const double x = lane < 16 ? s_wave[lane] : 0.0;
    const double wi = wave_scan(x, lane);
    if (lane < 16) s_wave[lane] = wi - x;  // exclusive prefix of the wave totals
  }
  __syncthreads();
  double off = s_wave[w] + (incl - run);  // exclusive offset of this thread's run
  for (int64_t i = lo; i < hi; ++i) {
    off += sums[i];
    sums[i] = off;
  }
}

__global__ __launch_bounds__(256) void sample_kernel(const float* __restrict__ p, int64_t n,
                                                     const double* __restrict__ prefix,
                                                     const double* __restrict__ lanes,
                                                     int64_t nblocks, int32_t batch, uint64_t seed,
                                                     float beta, int32_t* __restrict__ indices,
                                                     double* __restrict__ raw) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t b = blockIdx.x * 4 + w;
  if (b >= batch) return;  // wave-uniform
  const double u = per_uniform(seed, (uint32_t)b);
  const double T = prefix[nblocks - 1];
  int64_t k;
  double wr = 1.0;
  if (!(T > 0.0) || isinf(T)) {
    k = (int64_t)(u * (double)n);
    if (k >= n) k = n - 1;
  } else {
    const double target = u * T;
    // 64-way search for the first block whose prefix exceeds the target,
    // known to lie in [lo, hi] with prefix[hi] > target: lane i probes
    // lo + min(i step, hi - lo) with step = ceil((hi - lo) / 63), so lane 63
    // probes hi and some lane is always above; the first lane above bounds
    // the answer from above, the lane before it from below, and the range
    // shrinks to at most step - 1 per round
    int64_t lo = 0, hi = nblocks - 1;
    while (lo < hi) {
      const int64_t span = hi - lo;
      const int64_t step = (span + kLanes - 2) / (kLanes - 1);
      const int64_t off = (int64_t)lane * step;
      const uint64_t m = __ballot(prefix[lo + (off < span ? off : span)] > target);
      const int first = m ? __builtin_ctzll(m) : kLanes - 1;  // m = 0 only if target >= T
      const int64_t f_off = (int64_t)first * step;
      const int64_t p_off = (int64_t)(first - 1) * step;
      const int64_t new_hi = lo + (f_off < span ? f_off : span);
      const int64_t new_lo = first > 0 ? lo + (p_off < span ? p_off : span) + 1 : lo;
      hi = new_hi;
      lo = new_lo < new_hi ? new_lo : new_hi;
    }
    const int64_t blk = lo < nblocks ? lo : nblocks - 1;
    const double base = blk > 0 ? prefix[blk - 1] : 0.0;
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(p, n, blk);
    // this lane's inclusive prefix within the block (formed by
    // block_sums_kernel, so the same values as the block totals)
    const double incl = lanes[blk * kLanes + lane];
    const double excl = __shfl_up(incl, 1, kLanes);
    const double start = lane > 0 ? excl : 0.0;
    // the first lane whose range ends above the target walks its priorities
    const uint64_t m = __ballot(base + incl > target);
    int found = -1;
    if (m) {
      const int first = __builtin_ctzll(m);
      if (lane == first) {
        float v[kPerLane];
        lane_priorities(rs, lane, v);
        double run = start;
        for (int j = 0; j < kPerLane; ++j) {
          run += per_value(v[j]);
          if (base + run > target) { found = lane * kPerLane + j; break; }
        }
      }
      found = __shfl(found, first, kLanes);
    }
    if (found < 0) {
      // rounding left the target past every running sum of the block: the
      // last priority of the block that carries weight
      float v[kPerLane];
      lane_priorities(rs, lane, v);
      int last = -1;
      for (int j = 0; j < kPerLane; ++j)
        if (per_value(v[j]) > 0.0) last = lane * kPerLane + j;
      found = last;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const int o = __shfl_xor(found, d, kLanes);
        found = o > found ? o : found;
      }
      if (found < 0) found = 0;
    }
    k = blk * kPerBlock + found;
    if (k >= n) k = n - 1;
    wr = pow((double)n * per_value(p[k]) / T, -(double)beta);
  }
  if (lane == 0) {
    indices[b] = (int32_t)k;
    raw[b] = wr;
  }
}

// One workgroup: weights = raw / max(raw), rounded to float.
__global__ __launch_bounds__(1024) void weights_kernel(const double* __restrict__ raw, int32_t batch,
                                                       float* __restrict__ weights) {
  __shared__ double s_max[1024];
  double m = 0.0;
  for (int32_t b = threadIdx.x; b < batch; b += 1024) m = raw[b] > m ? raw[b] : m;
  s_max[threadIdx.x] = m;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s)
      s_max[threadIdx.x] = s_max[threadIdx.x + s] > s_max[threadIdx.x] ? s_max[threadIdx.x + s]
                                                                       : s_max[threadIdx.x];
    __syncthreads();
  }
  const double mx = s_max[0];
  for (int32_t b = threadIdx.x; b < batch; b += 1024) weights[b] = (float)(raw[b] / mx);
}

// Gather of the sampled transitions: row i of the [L][N] outputs is
// transition i (t = i / N, episode i % N).
__global__ __launch_bounds__(256) void gather_kernel(PerGatherArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.batch * kState;
  if (idx >= total) return;
  const int32_t b = (int32_t)(idx / kState);
  const int c = (int)(idx % kState);
  int64_t i = a.indices[b];
  i = i < 0 ? 0 : (i >= a.n ? a.n - 1 : i);
  if (a.states) a.out_states[idx] = a.states[i * kState + c];
  if (a.next_states) a.out_next_states[idx] = a.next_states[i * kState + c];
  if (c == 0) {
    if (a.actions) a.out_actions[b] = a.actions[i];
    if (a.rewards) a.out_rewards[b] = a.rewards[i];
    if (a.dones) a.out_dones[b] = a.dones[i];
  }
}

// Priority update: priority[i_b] = clamp(|td_b|^alpha + eps, eps, max), NaN
// -> eps; indices out of range are skipped.  Of repeated indices the
// largest new value is kept: the entries first clear their slots, then
// each takes the integer maximum of the (non-negative) float bits, which
// orders them as floats, so the result does not depend on timing.
__device__ __forceinline__ float new_priority(float td, float alpha, float eps, float pmax) {
  float v = powf(fabsf(td), alpha) + eps;
  if (!(v >= eps)) v = eps;
  return v > pmax ? pmax : v;
}

__global__ __launch_bounds__(256) void update_clear_kernel(float* __restrict__ pr, int64_t n,
                                                           const int32_t* __restrict__ indices,
                                                           int32_t batch) {
  const int32_t b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  const int32_t i = indices[b];
  if (i >= 0 && (int64_t)i < n) pr[i] = 0.0f;
}

__global__ __launch_bounds__(256) void update_max_kernel(float* __restrict__ pr, int64_t n,
                                                         const int32_t* __restrict__ indices,
                                                         const float* __restrict__ td,
                                                         int32_t batch, float alpha, float eps,
                                                         float pmax) {
  const int32_t b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  const int32_t i = indices[b];
  if (i < 0 || (int64_t)i >= n) return;
  const float v = new_priority(td[b], alpha, eps, pmax);
  atomicMax(reinterpret_cast<int*>(pr) + i, __float_as_int(v));
}

}  // namespace

hipError_t per_sample_launch(const float* p, int64_t n, int32_t batch, uint64_t seed, float beta,
                             int32_t* indices, float* weights, double* block_prefix,
                             double* lane_prefix, double* raw_weights, hipStream_t st) {
  const int64_t nblocks = per_blocks(n);
  hipLaunchKernelGGL(block_sums_kernel, dim3((unsigned)((nblocks + 3) / 4)), dim3(256), 0, st, p, n,
                     nblocks, block_prefix, lane_prefix);
  hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(1024), 0, st, block_prefix, nblocks);
  if (batch > 0) {
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)((batch + 3) / 4)), dim3(256), 0, st, p, n,
                       block_prefix, lane_prefix, nblocks, batch, seed, beta, indices, raw_weights);
    hipLaunchKernelGGL(weights_kernel, dim3(1), dim3(1024), 0, st, raw_weights, batch, weights);
  }
  return hipGetLastError();
}

hipError_t per_gather_launch(const PerGatherArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.batch * kState;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t per_update_launch(float* priorities, int64_t n, const int32_t* indices, const float* td,
                             int32_t batch, float alpha, float eps, float pmax, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((batch + 255) / 256);
  hipLaunchKernelGGL(update_clear_kernel, dim3(grid), dim3(256), 0, st, priorities, n, indices, batch);
  hipLaunchKernelGGL(update_max_kernel, dim3(grid), dim3(256), 0, st, priorities, n, indices, td,
                     batch, alpha, eps, pmax);
  return hipGetLastError();
}

}  // namespace rl
