// Device-side building blocks for the gfx950 collection kernels: the
// counter-based draw, fp32/bf16 MFMA wrappers and the packed-weight layout
// shared by the pack kernels and the MLP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rl {

typedef float f32x4 __attribute__((ext_vector_type(4)));
// four floats at a 4-byte aligned address (rows of 51 features): one
// 16-byte load where all four are wanted
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kFeatures = 51;
constexpr int kState = 54;
constexpr int kActions = 45;
constexpr int kWave = 64;
constexpr int kRowsPerWave = 16;  // MFMA N dimension: 16 episodes / rows per wave
constexpr int kFirstSteps = 14;   // first layer: 54 inputs -> 4 lane groups x 14

// --------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplications whose high halves are xored with the other words and the
// round key; the key advances by the golden-ratio Weyl constants.
// --------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Uniform in [0, 1) on a 2^-24 grid for (seed, episode, step, stream).
__device__ __forceinline__ float draw_uniform(uint64_t seed, uint32_t episode, uint32_t step,
                                              uint32_t stream) {
  const uint4 r = philox10(make_uint4(episode, step, stream, 0u), (uint32_t)seed,
                           (uint32_t)(seed >> 32));
  return (float)(r.x >> 8) * 5.9604644775390625e-8f;
}

// --------------------------------------------------------------------------
// MFMA v_mfma_f32_16x16x4_f32 in the transposed form used throughout:
//   D[out 16 x rows 16] += W[out 16 x k 4] * X^T[k 4 x rows 16]
// lane l supplies W[l%16][k(l/16)] and X[row l%16][k(l/16)], and holds
// D[4*(l/16) + r][l%16] in register r.  Each lane thus holds 4 consecutive
// outputs of one row; those registers are the next layer's X operand once the
// next layer's k order is permuted to match (packed into its weights).
// --------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8*(l/16) + j] and
// B[8*(l/16) + j][l%16] for j = 0..7; D as for the fp32 form.
__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 with round-to-nearest-even (the hardware conversion).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
// Two floats rounded to bf16 (nearest even) in one 32-bit word, lo in the
// low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_round(float x) {
  return __builtin_bit_cast(float, bf16_bits(x) << 16);
}

// Value held by lane l ^ 16 / l ^ 32 (gfx950 lane-swap instructions: no LDS
// round trip).  permlane16_swap exchanges rows 1, 3 of its first operand with
// rows 0, 2 of its second; permlane32_swap the upper half of the first with
// the lower half of the second.
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float lane_xor16f(float v, int lane) {
  return __uint_as_float(lane_xor16(__float_as_uint(v), lane));
}
__device__ __forceinline__ float lane_xor32f(float v, int lane) {
  return __uint_as_float(lane_xor32(__float_as_uint(v), lane));
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations
// (not its outstanding global loads and stores, which __syncthreads() would
// also drain), then s_barrier.  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace rl
