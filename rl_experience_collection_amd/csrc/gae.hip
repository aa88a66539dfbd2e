// GAE backward scan over time-major [L][N] buffers (PPO CUDA Pipeline
// Design, Kernel Phases, Phase B), single pass at HBM speed.
//
// The recurrence A_t = delta_t + c_t A_{t+1} (c_t = gamma lambda (1 - d_t))
// is affine in A_{t+1}: a run of steps [t0, t1) maps A_{t1} to
// A_{t0} = alpha + beta A_{t1}, with beta = 0 as soon as the run holds a done.
//
// Layout: a workgroup owns a column of COLS episodes x a super-chunk of
// kGaeWaves * 64 / COLS time slots of kGaeChunk steps.  With COLS = 32 (one
// 128-byte row of floats per step, 512-step super-chunks) each wave holds
// two slots (lanes 0-31 and 32-63); with COLS = 64 (256-step super-chunks)
// one.  Each thread keeps kGaeChunk consecutive steps of one episode in
// registers, so every load instruction reads whole rows.  Every thread folds its chunk into (alpha, beta);
// one lane per episode then forms, in one backward pass over the slots, the
// map of all later slots for each slot, and every thread applies its own to
// the incoming carry and writes A and R.
//
// A rollout of at most 512 steps runs with COLS = 32 as one super-chunk: no
// carry crosses workgroups, and workgroups map to columns by index, with the column order
// permuted so that the columns that share a 128-byte line of dones sit on
// one XCD (workgroups are dispatched round-robin over the 8 XCDs).
//
// Longer rollouts run with COLS = 64, whose shorter super-chunks keep more
// of them in flight, and chain the super-chunks of a column by a
// decoupled look-back: workgroups take super-chunks in reverse-time order
// from an atomic ticket, publish their aggregate alpha_S (or at once their
// inclusive value when the super-chunk holds a done or is the latest), look
// back to the nearest published inclusive value, fold the aggregates in
// between innermost-first and publish their own inclusive value
// alpha_S + beta_S * carry.  Every published value is one 64-bit word
// (value | epoch and status tag) stored and polled with device-coherent
// relaxed atomics, so no fences are needed.  A reader rebuilds the beta_S of
// an aggregate (no done inside) as the same product of gl^kGaeChunk factors
// the owner formed, so every carry is the same floating-point expression
// whatever the timing: results are bit-deterministic.  Every wait is on a
// workgroup holding an earlier ticket (already running) and the latest
// super-chunk never waits, so all waits end.  HBM traffic is the algorithmic
// 17 B per element plus 8 B per episode per super-chunk.
#include "gae.hpp"

#include <hip/hip_runtime.h>

namespace rl {

namespace {

constexpr uint32_t kAgg = 1u, kIncl = 2u;
constexpr int kWalk = 8;   // aggregates held before waiting on an inclusive
constexpr int kBatch = 4;  // later super-chunks read per look-back round

__device__ __forceinline__ void put_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack_word(float value, uint32_t tag) {
  return (uint64_t)__float_as_uint(value) | ((uint64_t)tag << 32);
}

// Column of a position in [0, NC): columns c, c+1, ... land on one XCD when
// NC is a multiple of 8 and the position follows the dispatch order.
__device__ __forceinline__ int32_t column_of(uint32_t p, int32_t NC) {
  if (NC & 7) return (int32_t)p;
  return (int32_t)(p & 7u) * (NC >> 3) + (int32_t)(p >> 3);
}

template <int COLS>
__global__ __launch_bounds__(64 * kGaeWaves) void gae_scan_kernel(
    const float* __restrict__ rew, const float* __restrict__ val, const uint8_t* __restrict__ don,
    const float* __restrict__ last_values, int32_t L, int32_t N, float gamma, float gl,
    float* __restrict__ adv, float* __restrict__ ret, GaeScratchView sc, int32_t NC, int32_t NK,
    uint32_t* __restrict__ status, uint32_t spin_limit) {
  constexpr int kSlots = gae_slots(COLS);
  constexpr int kSuper = gae_super(COLS);
  __shared__ uint32_t s_tile;
  __shared__ float s_a[kSlots][COLS];
  __shared__ float s_b[kSlots][COLS];

  const int lane = threadIdx.x & 63;
  const int e = lane & (COLS - 1);
  const int slot = (int)(threadIdx.x / COLS);
  uint32_t tile = blockIdx.x;
  if (NK > 1) {
    if (threadIdx.x == 0)
      s_tile = __hip_atomic_fetch_add(sc.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
               sc.ticket_base;
    __syncthreads();
    tile = s_tile;
    if (tile >= (uint32_t)NC * (uint32_t)NK) return;  // stale ticket base: never expected (uniform)
  }
  const int32_t S = NK - 1 - (int32_t)(tile / (uint32_t)NC);
  const int32_t c = column_of(tile % (uint32_t)NC, NC);
  const int32_t n = c * COLS + e;
  const bool active = n < N;
  const int32_t t0 = S * kSuper + slot * kGaeChunk;
  const int32_t cnt = active ? max(0, min(kGaeChunk, L - t0)) : 0;

  // ---- load this thread's chunk ------------------------------------------
  // Every load is issued before any is waited on: indices are clamped into
  // the buffers (steps past the chunk and idle lanes read a valid element
  // that is never used), so no load sits behind a branch.
  float r[kGaeChunk], v[kGaeChunk], d[kGaeChunk];
  uint32_t db[kGaeChunk];
  const int32_t nl = active ? n : N - 1;
#pragma unroll
  for (int i = 0; i < kGaeChunk; ++i) {
    const int32_t t = min(t0 + i, L - 1);
    const int64_t o = (int64_t)t * N + nl;
    r[i] = rew[o];
    v[i] = val[o];
    db[i] = don[o];
  }
  const int32_t tn = min(t0 + cnt, L - 1);
  const float v_after = val[(int64_t)tn * N + nl];
  const float v_last = last_values ? last_values[nl] : 0.0f;
#pragma unroll
  for (int i = 0; i < kGaeChunk; ++i) d[i] = (float)db[i];
  float vnext = 0.0f;
  if (cnt > 0) vnext = (t0 + cnt < L) ? v_after : v_last;

  // ---- chunk map: delta_t in place of r_t, A_t0 = alpha + beta A_t1 --------
  float alpha = 0.0f, beta = 1.0f;
  {
    float vn = vnext;
#pragma unroll
    for (int i = kGaeChunk - 1; i >= 0; --i) {
      if (i < cnt) {
        const float nd = 1.0f - d[i];
        const float delta = r[i] + gamma * vn * nd - v[i];
        const float ci = gl * nd;
        alpha = delta + ci * alpha;
        beta = ci * beta;
        r[i] = delta;
        vn = v[i];
      }
    }
  }
  s_a[slot][e] = alpha;
  s_b[slot][e] = beta;
  __syncthreads();

  // ---- suffix maps and super-chunk carry (lanes 0-31 of wave 0) ----------
  // The carry into slot j is the map of slots j+1..kSlots-1 applied to the
  // super-chunk's carry.  One lane per episode forms every suffix map in one
  // backward pass (in place of the slot maps), publishes and looks back with
  // the whole-super-chunk map, and leaves each slot's carry in s_a.
  if (threadIdx.x < COLS) {
    float aS = 0.0f, bS = 1.0f;
#pragma unroll
    for (int g0 = kSlots - 8; g0 >= 0; g0 -= 8) {
      float ca[8], cb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        ca[q] = s_a[g0 + q][e];
        cb[q] = s_b[g0 + q][e];
      }
#pragma unroll
      for (int q = 7; q >= 0; --q) {
        s_a[g0 + q][e] = aS;
        s_b[g0 + q][e] = bS;
        aS = ca[q] + cb[q] * aS;
        bS = cb[q] * bS;
      }
    }
    if (NK > 1) {
      const bool doneS = bS == 0.0f;
      const uint32_t tag = sc.epoch << 3;
      uint64_t* my = sc.words + (int64_t)S * N + n;
      float carry = 0.0f;
      if (active) {
        const bool incl_now = (S == NK - 1) || doneS;
        put_u64(my, pack_word(aS, tag | (incl_now ? kIncl : kAgg)));
        if (S != NK - 1) {
          // beta of a full super-chunk without dones, built like the owner's bS
          float gl_c = 1.0f;
#pragma unroll
          for (int i = 0; i < kGaeChunk; ++i) gl_c = gl * gl_c;
          float gl_s = 1.0f;
#pragma unroll
          for (int w = 0; w < kSlots; ++w) gl_s = gl_c * gl_s;
          float ag[kWalk];
          int m = 0;
          uint32_t spins = 0;
          float x = 0.0f;
          // a limit of 0 polls gives up without waiting (set by the host
          // only to exercise the reporting below)
          bool gave_up = spin_limit == 0;
          while (!gave_up) {
            uint64_t wd[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
              const int32_t j = S + 1 + m + q;
              wd[q] = j < NK ? get_u64(sc.words + (int64_t)j * N + n) : 0ull;
            }
            bool found = false, stop = false;
            int got = 0;
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
              if (stop) continue;
              const uint32_t hi = (uint32_t)(wd[q] >> 32);
              if (S + 1 + m + q >= NK || (hi >> 3) != sc.epoch) { stop = true; continue; }
              if ((hi & 3u) == kIncl) {
                x = __uint_as_float((uint32_t)wd[q]);
                found = stop = true;
                continue;
              }
              if (m + q >= kWalk) { stop = true; continue; }  // window full: wait here
#pragma unroll
              for (int z = 0; z < kWalk; ++z)
                if (z == m + q) ag[z] = __uint_as_float((uint32_t)wd[q]);
              ++got;
            }
            m += got;
            if (found) break;
            if (got == 0) {
              if (++spins > spin_limit) {
                gave_up = true;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
          }
          if (gave_up) {
            // never expected: the wait ended so the grid drains, and the
            // carry is NaN, so this column's results from here back to
            // step 0 are NaN instead of silently wrong
            if (status)
              __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            x = __builtin_nanf("");
            m = 0;
          }
#pragma unroll
          for (int z = kWalk - 1; z >= 0; --z)
            if (z < m) x = ag[z] + gl_s * x;  // innermost first
          carry = x;
          if (!doneS) put_u64(my, pack_word(aS + bS * carry, tag | kIncl));
        }
      }
#pragma unroll
      for (int w = 0; w < kSlots; ++w) s_a[w][e] = s_a[w][e] + s_b[w][e] * carry;
    }
  }
  __syncthreads();

  // ---- carry into this thread's chunk, then A and R -----------------------
  if (cnt <= 0) return;
  float A = s_a[slot][e];
#pragma unroll
  for (int i = kGaeChunk - 1; i >= 0; --i) {
    if (i < cnt) {
      A = r[i] + (gl * (1.0f - d[i])) * A;
      const int64_t o = (int64_t)(t0 + i) * N + n;
      // streaming stores: written once here, not read again by the scan
      __builtin_nontemporal_store(A, adv + o);
      __builtin_nontemporal_store(A + v[i], ret + o);
    }
  }
}

}  // namespace

GaeShape gae_shape(int32_t L, int32_t N) {
  GaeShape s;
  s.cols = L <= gae_super(32) ? 32 : 64;
  s.nc = cdiv_i(N, s.cols);
  s.nk = cdiv_i(L, gae_super(s.cols));
  return s;
}

hipError_t gae_launch(const GaeArgs& a, const GaeShape& shape, const GaeScratchView& sc,
                      hipStream_t stream) {
  auto kernel = shape.cols == 32 ? gae_scan_kernel<32> : gae_scan_kernel<64>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)shape.tiles()), dim3(64 * kGaeWaves), 0, stream,
                     a.rewards, a.values, a.dones, a.last_values, a.L, a.N, a.gamma,
                     a.gamma * a.lambda, a.advantages, a.returns, sc, shape.nc, shape.nk,
                     a.status, a.spin_limit);
  return hipGetLastError();
}

namespace {
__global__ void zero_words_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

hipError_t zero_words(uint32_t* p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256),
                     0, stream, p, words);
  return hipGetLastError();
}

}  // namespace rl
