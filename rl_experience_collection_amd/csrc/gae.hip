// GAE backward scan over time-major [L][N] buffers (PPO CUDA Pipeline
// Design, Kernel Phases, Phase B), single pass at HBM speed.
//
// The recurrence A_t = delta_t + c_t A_{t+1} (c_t = gamma lambda (1 - d_t))
// is affine in A_{t+1}, so a chunk of steps [t0, t1) maps A_{t1} to
// A_{t0} = alpha + beta A_{t1}.  The grid is cut into tiles of
// (256 * EPT episodes) x (TC steps).  Each workgroup
//   1. takes the next tile in reverse-time order from an atomic ticket,
//   2. loads its r, V, d once into registers (coalesced across episodes),
//   3. publishes its chunk aggregate (alpha, beta) per episode,
//   4. looks back at later-in-time tiles of the same episode columns until
//      it finds one that has published its inclusive value A_{t0}, then
//      folds the aggregates in between innermost-first, so the carry equals
//      the sequential composition whatever the timing (bit-deterministic),
//   5. publishes its own inclusive value, then writes A and R = A + V.
// Every wait is on a tile holding an earlier ticket, i.e. a workgroup that
// is already running, and the latest chunk never waits, so all waits end.
// HBM traffic is the algorithmic 17 B per element plus 12 B per episode per
// chunk of carry state.
#include "gae.hpp"

#include <hip/hip_runtime.h>

namespace rl {

namespace {

constexpr uint32_t kAgg = 1u, kIncl = 2u;
constexpr uint32_t kSpinLimit = 1u << 24;

__device__ __forceinline__ uint32_t flag_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f32(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}

template <int EPT>
struct Vec;
template <>
struct Vec<1> {
  typedef float F;
  typedef uint8_t D;
  static __device__ __forceinline__ float f(const F& v, int) { return v; }
  static __device__ __forceinline__ float d(const D& v, int) { return (float)v; }
  static __device__ __forceinline__ void set(F& v, int, float x) { v = x; }
};
template <>
struct Vec<2> {
  typedef float2 F;
  typedef uint16_t D;
  static __device__ __forceinline__ float f(const F& v, int e) { return e ? v.y : v.x; }
  static __device__ __forceinline__ float d(const D& v, int e) { return (float)((v >> (8 * e)) & 0xFF); }
  static __device__ __forceinline__ void set(F& v, int e, float x) { if (e) v.y = x; else v.x = x; }
};
template <>
struct Vec<4> {
  typedef float4 F;
  typedef uint32_t D;
  static __device__ __forceinline__ float f(const F& v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
  }
  static __device__ __forceinline__ float d(const D& v, int e) { return (float)((v >> (8 * e)) & 0xFF); }
  static __device__ __forceinline__ void set(F& v, int e, float x) {
    if (e == 0) v.x = x; else if (e == 1) v.y = x; else if (e == 2) v.z = x; else v.w = x;
  }
};

template <int EPT, int TC>
__global__ __launch_bounds__(256) void gae_lookback_kernel(
    const float* __restrict__ rew, const float* __restrict__ val, const uint8_t* __restrict__ don,
    const float* __restrict__ last_values, int32_t L, int32_t N, float gamma, float gl,
    float* __restrict__ adv, float* __restrict__ ret, GaeScratchView sc, int32_t NC, int32_t NK) {
  typedef Vec<EPT> V;
  typedef typename V::F F;
  typedef typename V::D D;
  __shared__ uint32_t s_tile;
  __shared__ int32_t s_found;

  if (threadIdx.x == 0)
    s_tile = __hip_atomic_fetch_add(sc.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
             sc.ticket_base;
  __syncthreads();
  const uint32_t tile = s_tile;
  if (tile >= (uint32_t)NC * (uint32_t)NK) return;  // stale ticket base: never expected
  const int32_t k = NK - 1 - (int32_t)(tile / (uint32_t)NC);
  const int32_t c = (int32_t)(tile % (uint32_t)NC);
  const int32_t n0 = (c * 256 + (int32_t)threadIdx.x) * EPT;
  const bool active = n0 < N;  // N is a multiple of EPT
  const int32_t t0 = k * TC;
  const int32_t cnt = min(TC, L - t0);

  // ---- load the chunk (one vector per step) -------------------------------
  F r[TC], v[TC];
  D d[TC];
  F vnext;
#pragma unroll
  for (int i = 0; i < TC; ++i) {
    if (active && i < cnt) {
      const int64_t o = (int64_t)(t0 + i) * N + n0;
      r[i] = *reinterpret_cast<const F*>(rew + o);
      v[i] = *reinterpret_cast<const F*>(val + o);
      d[i] = *reinterpret_cast<const D*>(don + o);
    }
  }
  if (active) {
    if (t0 + cnt < L) {
      vnext = *reinterpret_cast<const F*>(val + (int64_t)(t0 + cnt) * N + n0);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) V::set(vnext, e, last_values ? last_values[n0 + e] : 0.0f);
    }
  }

  // ---- local pass: delta_t in place of r_t, chunk aggregate (alpha, beta) --
  float alpha[EPT], beta[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    alpha[e] = 0.0f;
    beta[e] = 1.0f;
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float vn = V::f(vnext, e), A = 0.0f, B = 1.0f;
#pragma unroll
      for (int i = TC - 1; i >= 0; --i) {
        if (i < cnt) {
          const float nd = 1.0f - V::d(d[i], e);
          const float vi = V::f(v[i], e);
          const float delta = V::f(r[i], e) + gamma * vn * nd - vi;
          const float ci = gl * nd;
          A = delta + ci * A;
          B = ci * B;
          V::set(r[i], e, delta);
          vn = vi;
        }
      }
      alpha[e] = A;
      beta[e] = B;
    }
  }

  const uint32_t tag = sc.epoch << 2;
  uint32_t* flags = sc.flags + (int64_t)0;
  float carry[EPT];
  if (k == NK - 1) {
    // latest chunk: A_L = 0, so its aggregate is already inclusive
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      carry[e] = 0.0f;
      if (active) put_f32(sc.incl + (int64_t)k * N + n0 + e, alpha[e]);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) flag_store(flags + (int64_t)k * NC + c, tag | kIncl);
  } else {
    if (active) {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        put_u64(sc.agg + (int64_t)k * N + n0 + e, pack2(alpha[e], beta[e]));
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      flag_store(flags + (int64_t)k * NC + c, tag | kAgg);
      // find the nearest later tile with an inclusive value
      int32_t j = k + 1;
      uint32_t spins = 0;
      for (;;) {
        const uint32_t f = flag_load(flags + (int64_t)j * NC + c);
        if ((f >> 2) == sc.epoch && (f & 3u) == kIncl) break;
        if ((f >> 2) == sc.epoch && (f & 3u) == kAgg && j + 1 < NK) {
          ++j;
          continue;
        }
        if (++spins > kSpinLimit) {  // never expected: keeps the grid draining
          __hip_atomic_fetch_add(sc.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      s_found = j;
    }
    __syncthreads();
    const int32_t j = s_found;
    if (active) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float x = get_f32(sc.incl + (int64_t)j * N + n0 + e);
        for (int32_t i = j - 1; i > k; --i) {
          const uint64_t ab = get_u64(sc.agg + (int64_t)i * N + n0 + e);
          x = __uint_as_float((uint32_t)ab) + __uint_as_float((uint32_t)(ab >> 32)) * x;
        }
        carry[e] = x;
        put_f32(sc.incl + (int64_t)k * N + n0 + e, alpha[e] + beta[e] * x);
      }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) flag_store(flags + (int64_t)k * NC + c, tag | kIncl);
  }

  // ---- fix-up: A_t from the carry, write A and R = A + V ------------------
  if (!active) return;
  float A[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) A[e] = carry[e];
#pragma unroll
  for (int i = TC - 1; i >= 0; --i) {
    if (i < cnt) {
      F a_out, r_out;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float nd = 1.0f - V::d(d[i], e);
        A[e] = V::f(r[i], e) + (gl * nd) * A[e];
        V::set(a_out, e, A[e]);
        V::set(r_out, e, A[e] + V::f(v[i], e));
      }
      const int64_t o = (int64_t)(t0 + i) * N + n0;
      *reinterpret_cast<F*>(adv + o) = a_out;
      *reinterpret_cast<F*>(ret + o) = r_out;
    }
  }
}

template <int EPT, int TC>
hipError_t launch(const GaeArgs& a, const GaeScratchView& sc, hipStream_t stream) {
  const int32_t NC = cdiv_i(a.N, 256 * EPT), NK = cdiv_i(a.L, TC);
  hipLaunchKernelGGL((gae_lookback_kernel<EPT, TC>), dim3((unsigned)(NC * NK)), dim3(256), 0, stream,
                     a.rewards, a.values, a.dones, a.last_values, a.L, a.N, a.gamma,
                     a.gamma * a.lambda, a.advantages, a.returns, sc, NC, NK);
  return hipGetLastError();
}

}  // namespace

GaeShape gae_shape(int32_t L, int32_t N, bool aligned16, bool aligned8) {
  GaeShape s;
  s.ept = (N % 4 == 0 && aligned16) ? 4 : ((N % 2 == 0 && aligned8) ? 2 : 1);
  s.tc = kGaeChunk;
  s.nc = cdiv_i(N, 256 * s.ept);
  s.nk = cdiv_i(L, s.tc);
  return s;
}

hipError_t gae_launch(const GaeArgs& a, const GaeShape& shape, const GaeScratchView& sc,
                      hipStream_t stream) {
  switch (shape.ept) {
    case 4: return launch<4, kGaeChunk>(a, sc, stream);
    case 2: return launch<2, kGaeChunk>(a, sc, stream);
    default: return launch<1, kGaeChunk>(a, sc, stream);
  }
}

}  // namespace rl
