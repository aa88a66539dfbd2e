/*
 * per.h -- C ABI of the prioritized-replay kernels in librollout.so (gfx950):
 * proportional sampling with importance weights, the gather of the sampled
 * transitions and the priority update ("GPU-Resident Prioritized Experience
 * Replay", Sampling Kernels: proportional steps 1-5 and the priority update;
 * Error Handling: the NaN/Inf clamp).  Same conventions as rollout.h: DEVICE
 * buffers owned by the caller, asynchronous on the given stream (NULL = the
 * default stream), ROLLOUT_OK or a negative ROLLOUT_E* code with the message
 * in rollout_last_error(), no CPU fallback.
 *
 * Sampling: draw b (0 <= b < batch) uses u_b in [0, 1), the 53-bit uniform
 * ((w0 << 21) | (w1 >> 11)) * 2^-53 of the Philox4x32-10 block with counter
 * (b, 0, 4, 0) and key (seed low, seed high).  With C_k the inclusive prefix
 * sums of the priorities (negative and NaN priorities count as 0) and
 * T = C_{n-1}, the sample is the first k with C_k > u_b T, and its weight is
 * (n p_k / T)^(-beta) divided by the largest weight of the batch.  If T is not
 * positive and finite the draws are uniform, k = floor(u_b n), weight 1.  The
 * prefix sums are fp64, formed in a fixed order (results are deterministic);
 * near a boundary, where u_b T lies within rounding of a C_k, the choice
 * between the two neighbours follows that order.
 */
#ifndef PER_H
#define PER_H

#include <stdint.h>

#include "rollout.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct per_s *per_handle; /* opaque: scratch for up to `capacity` priorities */

/* Allocate the sampler's scratch (520 bytes per 2048 priorities: the block
 * prefix and 64 in-block lane prefixes in fp64; 8 bytes per draw).  Errors: ROLLOUT_EINVAL (capacity < 1, max_batch < 1 or
 * > 1048576, capacity > 2^31 - 1), ROLLOUT_ENOMEM. */
int per_create(int64_t capacity, int32_t max_batch, per_handle *out);

/* Draw `batch` transitions from `priorities` [n] f32 (n <= capacity, batch <=
 * max_batch): indices [batch] i32 in [0, n), weights [batch] f32.  Calls on
 * one handle must not overlap (they share its scratch). */
int per_sample(per_handle h, const float *priorities, int64_t n, int32_t batch, uint64_t seed,
               float beta, int32_t *indices, float *weights, void *hip_stream);

/* Gather the sampled transitions from flat replay arrays of n transitions
 * (for the collection outputs, transition i is element i of the [L][N]
 * arrays: step i / N of episode i % N).  Any source may be NULL (its output
 * is then not written).  Indices outside [0, n) are clamped.
 * Shapes: states/next_states [n][54], actions/rewards/dones [n];
 * outputs [batch][54] / [batch]. */
int per_gather(const int32_t *indices, int32_t batch, int64_t n, const float *states,
               const float *next_states, const int32_t *actions, const float *rewards,
               const uint8_t *dones, float *out_states, float *out_next_states,
               int32_t *out_actions, float *out_rewards, uint8_t *out_dones, void *hip_stream);

/* Priority update after a training step:
 *   priorities[indices[b]] = clamp(|td[b]|^alpha + epsilon, epsilon, max_priority)
 * with a NaN giving epsilon and +-Inf max_priority.  An index repeated in the
 * batch keeps the largest of its new values (independent of timing); indices
 * outside [0, n) are skipped.  epsilon must be >= 0.
 * Errors: ROLLOUT_EINVAL (NULL, batch < 0 or > 1048576, epsilon < 0 or
 * epsilon > max_priority). */
int per_update(float *priorities, int64_t n, const int32_t *indices, const float *td,
               int32_t batch, float alpha, float epsilon, float max_priority, void *hip_stream);

/* Release the sampler (NULL-safe); work using it must be complete. */
void per_destroy(per_handle h);

#ifdef __cplusplus
}
#endif
#endif
