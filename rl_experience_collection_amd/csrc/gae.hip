// GAE backward scan over time-major [L][N] buffers (PPO CUDA Pipeline
// Design, Kernel Phases, Phase B), single pass at HBM speed.
//
// The recurrence A_t = delta_t + c_t A_{t+1} (c_t = gamma lambda (1 - d_t))
// is affine in A_{t+1}: a run of steps [t0, t1) maps A_{t1} to
// A_{t0} = alpha + beta A_{t1}, with beta = 0 as soon as the run holds a done.
//
// Layout: a workgroup of 16 waves owns a column of COLS episodes x a
// super-chunk of 512 steps, cut into time slots of consecutive steps, one
// slot per thread and episode.  Each thread keeps its slot's steps in
// registers, so every load instruction reads whole rows of the column.
// Every thread folds its slot into (alpha, beta); one lane per episode then
// forms, in one backward pass over the slots, the map of all later slots for
// each slot, and every thread applies its own to the incoming carry and
// writes A and R.
//
// A rollout of at most 512 steps is one super-chunk: COLS = 32 (one
// 128-byte row of floats per step, two 16-step slots per wave), no carry
// crosses workgroups, and workgroups map to columns by index, with the
// column order permuted so that the columns that share a 128-byte line of
// dones sit on one XCD (workgroups are dispatched round-robin over the 8
// XCDs).
//
// Longer rollouts run with COLS = 64 and 32-step slots (one per wave), so a
// super-chunk is still 512 steps and a launch holds as few of them as
// possible: each costs a look-back, and a launch that fits the chip in one
// round of workgroups never waits for a second round's loads.  The values
// wait in LDS between the two passes, which keeps the registers held across
// the look-back within a 1024-thread workgroup's budget.  The super-chunks
// of a column are chained by a decoupled look-back: workgroups take
// super-chunks in reverse-time order from an atomic ticket, publish their
// aggregate alpha_S (or at once their inclusive value when the super-chunk
// holds a done or is the latest), look back to the nearest published
// inclusive value, fold the aggregates in between innermost-first and
// publish their own inclusive value alpha_S + beta_S * carry.  Every
// published value is one 64-bit word (value | epoch and status tag) stored
// and polled with device-coherent relaxed atomics, so no fences are needed.  A reader
// rebuilds the beta_S of an aggregate (no done inside) as the same product
// of gl^32 factors the owner formed, so every carry is the same
// floating-point expression whatever the timing: results are
// bit-deterministic.  Every wait is on a workgroup holding an earlier
// ticket (already running) and the latest super-chunk never waits, so all
// waits end.  HBM traffic is the algorithmic 17 B per element
// plus 8 B per episode per super-chunk.
#include "gae.hpp"

#include <hip/hip_runtime.h>

namespace rl {

namespace {

constexpr uint32_t kAgg = 1u, kIncl = 2u;
constexpr int kWalk = 8;   // aggregates held before waiting on an inclusive
constexpr int kBatch = 2;  // later super-chunks read per look-back round

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

// COLS = 32: one super-chunk per column; COLS = 64: chained super-chunks.
// OFF32: the host has checked that a super-chunk's bytes stay below 4 GiB.
template <int COLS, bool OFF32>
__global__ __launch_bounds__(64 * kGaeWaves) void gae_scan_kernel(
    const float* __restrict__ rew, const float* __restrict__ val, const uint8_t* __restrict__ don,
    const float* __restrict__ last_values, int32_t L, int32_t N, float gamma, float gl,
    float* __restrict__ adv, float* __restrict__ ret, GaeScratchView sc, int32_t NC, int32_t NK,
    uint32_t* __restrict__ status, uint32_t spin_limit) {
  constexpr int kSlots = gae_slots(COLS);
  constexpr int kSuper = gae_super(COLS);
  constexpr int kChunk = gae_chunk(COLS);
  constexpr bool kChain = COLS == 64;
  constexpr int kG = 8;  // slots' maps held in registers at a time
  static_assert(kChunk <= 32, "dones of a slot are kept as one 32-bit mask");
  static_assert(kSlots % kG == 0, "suffix maps are formed kG slots at a time");
  __shared__ uint32_t s_tile;
  __shared__ float s_a[kSlots][COLS];
  __shared__ float s_b[kSlots][COLS];
  // chained shape: each thread's values, between the two passes
  __shared__ float s_v[kChain ? kChunk : 1][kChain ? 64 * kGaeWaves : 1];

  const int e = (int)threadIdx.x & (COLS - 1);
  const int slot = (int)(threadIdx.x / COLS);
  int32_t S = 0, c;
  uint32_t tile = blockIdx.x;
  if constexpr (kChain) {
    // tiles in ticket order: the latest super-chunks of every column first
    if (threadIdx.x == 0)
      s_tile = __hip_atomic_fetch_add(sc.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
               sc.ticket_base;
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(s_tile);
    if (tile >= (uint32_t)NC * (uint32_t)NK) return;  // stale ticket base: never expected
    S = NK - 1 - (int32_t)(tile / (uint32_t)NC);
  }
  c = column_of(tile % (uint32_t)NC, NC);
  const int32_t n = c * COLS + e;
  const bool active = n < N;
  const int32_t t0 = S * kSuper + slot * kChunk;
  const int32_t cnt = active ? max(0, min(kChunk, L - t0)) : 0;

  // ---- load this thread's slot --------------------------------------------
  // Every load is issued before any is waited on: indices are clamped into
  // the buffers (steps past the slot and idle lanes read a valid element
  // that is never used), so no load sits behind a branch.
  float r[kChunk], v[kChunk];
  uint32_t db[kChunk];
  const int32_t nl = active ? n : N - 1;
  if constexpr (OFF32) {
    // addresses are a workgroup-uniform base plus one running 32-bit offset
    // instead of a 64-bit address per load
    const int64_t base = (int64_t)S * kSuper * N + (int64_t)c * COLS;
    const char* rb = reinterpret_cast<const char*>(rew + base);
    const char* vb = reinterpret_cast<const char*>(val + base);
    const char* db0 = reinterpret_cast<const char*>(don + base);
    uint32_t off = (uint32_t)(min(t0, L - 1) - S * kSuper) * (uint32_t)N + (uint32_t)(nl - c * COLS);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      r[i] = *reinterpret_cast<const float*>(rb + (off << 2));
      v[i] = *reinterpret_cast<const float*>(vb + (off << 2));
      db[i] = *reinterpret_cast<const uint8_t*>(db0 + off);
      off += (t0 + i + 1 < L) ? (uint32_t)N : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int32_t t = min(t0 + i, L - 1);
      const int64_t o = (int64_t)t * N + nl;
      r[i] = rew[o];
      v[i] = val[o];
      db[i] = don[o];
    }
  }
  const int32_t tn = min(t0 + cnt, L - 1);
  const float v_after = val[(int64_t)tn * N + nl];
  // no load behind a branch: without last values, read a value and drop it
  const float v_lrd = (last_values ? last_values : val)[nl];
  const float v_last = last_values ? v_lrd : 0.0f;
  float vnext = 0.0f;
  if (cnt > 0) vnext = (t0 + cnt < L) ? v_after : v_last;

  // ---- slot map: delta_t in place of r_t, A_t0 = alpha + beta A_t1 ---------
  // The dones leave the registers here as a bit mask for the second pass.
  float alpha = 0.0f, beta = 1.0f;
  uint32_t dmask = 0u;
  {
    float vn = vnext;
#pragma unroll
    for (int i = kChunk - 1; i >= 0; --i) {
      // steps past the slot's end leave the map unchanged (selects, not
      // branches)
      const bool in = i < cnt;
      dmask |= (db[i] != 0u ? 1u : 0u) << i;
      const float nd = 1.0f - (float)db[i];
      const float delta = r[i] + gamma * vn * nd - v[i];
      const float ci = gl * nd;
      alpha = in ? delta + ci * alpha : alpha;
      beta = in ? ci * beta : beta;
      r[i] = delta;
      vn = in ? v[i] : vn;
    }
  }
  if constexpr (kChain) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) s_v[i][threadIdx.x] = v[i];
  }
  s_a[slot][e] = alpha;
  s_b[slot][e] = beta;
  __syncthreads();

  // ---- suffix maps and super-chunk carry (one lane per episode) -----------
  // The carry into slot j is the map of slots j+1..kSlots-1 applied to the
  // super-chunk's carry.  One lane per episode forms every suffix map in one
  // backward pass (in place of the slot maps), publishes and looks back with
  // the whole-super-chunk map, and leaves each slot's carry in s_a.
  if (threadIdx.x < COLS) {
    float aS = 0.0f, bS = 1.0f;
#pragma unroll 1
    for (int g0 = kSlots - kG; g0 >= 0; g0 -= kG) {
      float ca[kG], cb[kG];
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        ca[q] = s_a[g0 + q][e];
        cb[q] = s_b[g0 + q][e];
      }
#pragma unroll
      for (int q = kG - 1; q >= 0; --q) {
        s_a[g0 + q][e] = aS;
        s_b[g0 + q][e] = bS;
        aS = ca[q] + cb[q] * aS;
        bS = cb[q] * bS;
      }
    }
    if constexpr (kChain) {
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
          for (int i = 0; i < kChunk; ++i) gl_c = gl * gl_c;
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

  // ---- carry into this thread's slot, then A and R ------------------------
  if (cnt <= 0) return;
  float A = s_a[slot][e];
#pragma unroll
  for (int i = kChunk - 1; i >= 0; --i) {
    if (i < cnt) {
      // gl * (1 - d) for a done d of 0 or 1
      A = r[i] + (((dmask >> i) & 1u) ? 0.0f : gl) * A;
      const int64_t o = (int64_t)(t0 + i) * N + n;
      const float vi = kChain ? s_v[i][threadIdx.x] : v[i];
      // streaming stores: written once here, not read again by the scan
      __builtin_nontemporal_store(A, adv + o);
      __builtin_nontemporal_store(A + vi, ret + o);
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
  const bool off32 = (int64_t)gae_super(shape.cols) * a.N * 4 < ((int64_t)1 << 32);
  auto kernel = shape.cols == 32 ? (off32 ? gae_scan_kernel<32, true> : gae_scan_kernel<32, false>)
                                 : (off32 ? gae_scan_kernel<64, true> : gae_scan_kernel<64, false>);
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
