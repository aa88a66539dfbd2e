/*
 * dqn.h -- C ABI of the DQN experience collection in librollout.so (gfx950).
 * Same conventions as rollout.h: plain pointers and sizes, DEVICE buffers
 * owned by the caller, [L][N] time-major outputs, asynchronous on the given
 * stream, ROLLOUT_OK or a negative ROLLOUT_E* code with the message in
 * rollout_last_error(), no CPU fallback.
 *
 * What is computed ("GPU Pipeline Phase 2b: Zero-Roundtrip CUDA Experience
 * Collection", Data Flow steps 1-15, Kernel Components 1-8): N independent
 * trading episodes advance L steps in one launch.  Each step builds the
 * 54-wide state (51 market features of the bar, V/V0 - 1, the exposure held,
 * the spread), evaluates the online dueling Q-network
 *   h = ReLU(W2 ReLU(W1 s + b1) + b2)                      54 -> 256 -> 128
 *   V = Wv2 ReLU(Wv1 h + bv1) + bv2,  A = Wa2 ReLU(Wa1 h + ba1) + ba2
 *   Q_i = V + (A_i - mean_j A_j)                           45 actions
 * picks the action epsilon-greedily (a counter-based draw u1 of stream 1
 * below epsilon takes the random action floor(45 u2), u2 from stream 2;
 * otherwise the greedy action, the lowest index among equal maxima), steps
 * the portfolio, triple barrier and diversity window and forms the reward
 * with the curiosity bonus exactly as rollout_collect does, builds the next
 * state (bar + 1, portfolio after the trade, before any reset), evaluates the
 * target network on it and writes
 *   td       = r + gamma * (1 - done) * max_a Q_target(s', a) - Q_online(s, a)
 *   priority = |td|^alpha
 * (the priority rule of "GPU-Resident Prioritized Experience Replay",
 * Sampling Kernels, priority update), then resets the episode on done.
 * Draws: Philox4x32-10 with counter (episode, step, stream, 0) and key
 * (seed low, seed high); u = (word0 >> 8) * 2^-24.
 */
#ifndef DQN_H
#define DQN_H

#include <stdint.h>

#include "rollout.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dqn_s *dqn_handle; /* opaque, owned by the library */

/* Settings of one DQN collector, copied at dqn_create.  Widths are fixed by
 * this library and must match. */
typedef struct {
  int32_t n_episodes;        /* N >= 1 */
  int32_t n_steps;           /* L >= 1 */
  int32_t n_features;        /* 51 */
  int32_t state_dim;         /* 54 */
  int32_t n_actions;         /* 45 */
  int32_t trunk_dims[3];     /* 54, 256, 128 */
  int32_t value_dims[3];     /* 128, 64, 1 */
  int32_t advantage_dims[3]; /* 128, 64, 45 */
  int32_t cur_dims[3];       /* 99 (= 54 + 45 one-hot), 128, 51 */
  float epsilon;             /* exploration probability, in [0, 1] (0.1);
                                dqn_set_epsilon changes it between launches */
  float gamma;               /* TD discount (0.99) */
  float priority_alpha;      /* priority = |td|^alpha (0.6) */
  float profit_take;         /* the environment settings, as in rollout_config */
  float stop_loss;
  int32_t max_hold;
  int32_t div_window;        /* 1..32 */
  float div_threshold;
  float div_penalty;
  float curiosity_coef;
  float risk_coef;
  float spread;
  float barrier_scale;
  float exposure[5];
  float cost[3];
  float urgency_mult;
  int32_t recycle;           /* 0 (default): after a done the episode resets and
                                runs on along its bars; 1: dynamic episode
                                recycling ("GPU Pipeline Phase 2b", Future
                                Phase 3 Optimization): it restarts at bar
                                floor(x range / 2^32), x the first Philox word
                                of counter (episode, t, 5, 0), range = n_bars -
                                (L - t - 1) valid starts */
} dqn_config;

/* Output buffers: DEVICE pointers, caller-owned, [L][N] unless stated.
 * Required: states, actions, q_taken, q_next_max, rewards, dones, barrier,
 * td, priorities. */
typedef struct {
  float *states;      /* [L][N][54] f32, the state of each step */
  float *next_states; /* [L][N][54] f32 or NULL: the state after the step,
                         before any reset (the target network's input) */
  float *q_values;    /* [L][N][45] f32 or NULL: online Q of the state */
  int32_t *actions;   /* [L][N] i32, 0..44 */
  uint8_t *explored;  /* [L][N] u8 or NULL: 1 when the action is the random one */
  float *q_taken;     /* [L][N] f32, online Q of the action taken */
  float *q_next_max;  /* [L][N] f32, max over actions of the target Q of next_state */
  float *rewards;     /* [L][N] f32 */
  uint8_t *dones;     /* [L][N] u8, 1 when a barrier fired (episode reset) */
  uint8_t *barrier;   /* [L][N] u8: 0 none, 1 profit, 2 stop, 3 time */
  float *td;          /* [L][N] f32, TD error (signed) */
  float *priorities;  /* [L][N] f32, |td|^alpha */
  uint32_t *counters; /* [2] or NULL: reset then accumulated by this call:
                         [0] steps with a non-finite Q, reward or TD,
                         [1] episodes whose start had to be clamped */
  void *const *phase_events; /* NULL or [2] caller-created hipEvent_t (as
                         void*), recorded before and after the kernel */
} dqn_outputs;

/* Defaults (the values in the comments above) for N episodes of L steps. */
int dqn_config_default(dqn_config *cfg, int32_t n_episodes, int32_t n_steps);

/* Create a DQN collector.
 *  online[12], target[12] = trunk W1[256,54], b1[256], W2[128,256], b2[128],
 *      value Wv1[64,128], bv1[64], Wv2[1,64], bv2[1],
 *      advantage Wa1[64,128], ba1[64], Wa2[45,64], ba2[45]
 *      ([out, in] row-major fp32, the pages' matvec convention)
 *  curiosity[4] = W1[128,99], b1[128], W2[51,128], b2[51]
 *  features = [n_bars][51] f32, prices = [n_bars] f32 (positive), BORROWED.
 * The weights are copied and repacked (stream-ordered on hip_stream).
 * Errors: ROLLOUT_EINVAL (NULL, N or L < 1, widths differ from the built
 * nets, epsilon outside [0, 1], n_bars < L + 1, div_window outside 1..32),
 * ROLLOUT_ENOMEM, ROLLOUT_EHIP. */
int dqn_create(const dqn_config *cfg, const float *const online[12],
               const float *const target[12], const float *const curiosity[4],
               const float *features, const float *prices, int64_t n_bars, void *hip_stream,
               dqn_handle *out);

/* Replace weights; a NULL online, target or curiosity array keeps that
 * network (a target sync passes only `target`).  Stream-ordered. */
int dqn_set_weights(dqn_handle h, const float *const online[12], const float *const target[12],
                    const float *const curiosity[4], void *hip_stream);

/* Set the exploration probability of later collections ("GPU Pipeline Phase
 * 2b", Concerns and Mitigations, Epsilon Decay: epsilon is a scalar handed to
 * each launch, decayed on the host between rounds).  The value is copied into
 * the kernel arguments when dqn_collect enqueues, so it applies to every
 * collection enqueued after this call returns, on any stream, and to none
 * enqueued before; no device work, no synchronisation.  Not safe against a
 * concurrent dqn_collect on the same handle from another host thread.
 * Errors: ROLLOUT_EINVAL (NULL handle, epsilon outside [0, 1] or NaN). */
int dqn_set_epsilon(dqn_handle h, float epsilon);

/* Collect one batch of N x L transitions.  episode_starts = [N] i32 device
 * array; a start outside [0, n_bars - L - 1] is clamped on the device and
 * counted in counters[1].  Calls on one handle must not overlap. */
int dqn_collect(dqn_handle h, const int32_t *episode_starts, uint64_t seed,
                const dqn_outputs *out, void *hip_stream);

/* Release a collector (NULL-safe); work using it must be complete. */
void dqn_destroy(dqn_handle h);

#ifdef __cplusplus
}
#endif
#endif
