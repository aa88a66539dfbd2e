/*
 * rollout.h -- C ABI of the MI355X (gfx950) fused PPO experience-collection
 * library (librollout.so).  Plain pointers and sizes only; no framework types.
 *
 * What is computed (source pages cited by title and section):
 *  - "PPO CUDA Pipeline Design - Zero-Roundtrip Experience Collection
 *    (Phase 2c)", Kernel Phases: N independent trading episodes advance L steps
 *    with no host round trip; each step builds the 54-wide state (Phase A
 *    steps 1-2), runs the actor 54->128->64->45 (step 3), draws an action from
 *    the softmax by inverse CDF with its log-probability (step 4), evaluates
 *    the critic 54->512->384->256->128->64->1 (step 5), simulates portfolio,
 *    triple barrier and diversity (steps 6-8), adds the curiosity bonus
 *    (step 9), combines the reward (step 10), stores the step (step 11) and
 *    resets the episode when a barrier fires (step 12).  Phase B then scans
 *    each episode backward for GAE advantages and returns.
 *  - "GPU Pipeline Phase 2b: Zero-Roundtrip CUDA Experience Collection",
 *    Kernel Components 1-6: [out, in] weight convention, curiosity forward
 *    model, portfolio, barrier labels (-1 stop, 0 time/none, +1 profit),
 *    diversity entropy penalty and the reward combination.
 *  - "Fused CUDA Training Kernel - Implementation Plan", Task 1 step 3: the
 *    45-action factorisation exp = a/9, ord = (a%9)/3, urg = a%3.
 * The pages' LCG is replaced by a counter-based Philox4x32-10 draw keyed by
 * (seed, episode, step): u = (word0 >> 8) * 2^-24 of the block with counter
 * (episode, step, 0, 0) and key (seed low 32 bits, seed high 32 bits).
 *
 * Conventions shared by every entry point:
 *  - Every buffer argument is a DEVICE pointer on the current HIP device,
 *    owned by the caller, unless stated otherwise.  All per-step outputs are
 *    time-major: element (t, n) of an [L][N] array lives at t*N + n;
 *    states are [L][N][54] and logits [L][N][45].
 *  - `hip_stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Work is enqueued asynchronously on it; no call synchronises the host.
 *  - Return value: ROLLOUT_OK (0) or a negative ROLLOUT_E* code.  The message
 *    of the last failure on the calling thread is in rollout_last_error().
 *    Argument errors are detected on the host before anything is enqueued;
 *    asynchronous device faults surface at the caller's next synchronisation.
 *  - There is no CPU fallback: if the GPU path cannot run, the call fails.
 */
#ifndef ROLLOUT_H
#define ROLLOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROLLOUT_OK 0
#define ROLLOUT_EINVAL (-1)   /* bad argument: null pointer, size, dims, alignment */
#define ROLLOUT_ENOMEM (-2)   /* device allocation failed */
#define ROLLOUT_EHIP (-3)     /* HIP runtime/launch error (message copied) */
#define ROLLOUT_ENOTIMPL (-4) /* configuration not supported by this library */

typedef struct rollout_s *rollout_handle; /* opaque, owned by the library */

typedef enum {
  ROLLOUT_FP32 = 0, /* fp32 weights, activations and accumulation */
  ROLLOUT_BF16 = 1  /* bf16 weights and layer inputs, fp32 accumulate/state */
} rollout_precision;

/* Settings of one collector, copied at rollout_create.  The network widths
 * are fixed by this library and must match exactly; they are carried here so a
 * mismatch is an error rather than a silent misread. */
typedef struct {
  int32_t n_episodes;     /* N >= 1 */
  int32_t n_steps;        /* L >= 1 */
  int32_t n_features;     /* 51 */
  int32_t state_dim;      /* 54 = 51 features + value/V0-1, exposure, spread */
  int32_t n_actions;      /* 45 */
  int32_t actor_dims[4];  /* 54, 128, 64, 45 */
  int32_t critic_dims[7]; /* 54, 512, 384, 256, 128, 64, 1 */
  int32_t cur_dims[3];    /* 99 (= 54 + 45 one-hot), 128, 51 */
  int32_t precision;      /* rollout_precision */
  float gamma, lambda;    /* GAE discount and trace factors */
  float profit_take;      /* barrier: +fraction from entry (0.02) */
  float stop_loss;        /* barrier: -fraction from entry (0.01) */
  int32_t max_hold;       /* barrier: time exit after this many bars held */
  int32_t div_window;     /* diversity window, 1..32 actions */
  float div_threshold;    /* entropy threshold in nats (1.0) */
  float div_penalty;      /* reward term when entropy < threshold (-0.1) */
  float curiosity_coef;   /* bonus = coef * MSE of the forward model (0.01) */
  float risk_coef;        /* risk = coef * |exposure| (0.01) */
  float spread;           /* constant third portfolio feature (0.0005) */
  float barrier_scale;    /* pnl * (1 + scale * hit) (0.5) */
  float exposure[5];      /* exposure of a/9 = 0..4: -1, -0.5, 0, 0.5, 1 */
  float cost[3];          /* cost rate of (a%9)/3: 2e-4, 5e-4, 1e-3 */
  float urgency_mult;     /* cost * (1 + mult * (a%3)) (0.5) */
  int32_t recycle;        /* 0 (default): after a done the episode resets and
                             runs on along its bars; 1: dynamic episode
                             recycling ("GPU Pipeline Phase 2b", Future Phase 3
                             Optimization): it restarts at bar
                             floor(x range / 2^32), x the first Philox word of
                             counter (episode, t, 5, 0), range = n_bars -
                             (L - t - 1) valid starts; the handle then keeps
                             an [L][N] i32 record of the bars */
  int32_t overlap;        /* -1 (default): in fp32, when the rollout's
                             workgroups (16 episodes each) fill at most a
                             quarter of the CUs (N <= 1024 on 256 CUs),
                             split the rollout into 2..8 launches of
                             consecutive steps (L / 64 of them) and run the
                             value pass over each finished part on a second
                             stream of the handle, on the CUs the rollout
                             leaves free, while the next part runs; 0: never;
                             1: always.  The results do not depend on it. */
} rollout_config;

/* Output buffers of one collection: DEVICE pointers, caller-owned, [L][N].
 * All are required except `logits`, `counters` and `phase_events`. */
typedef struct {
  float *states;      /* [L][N][54] f32 */
  int32_t *actions;   /* [L][N] i32, 0..44 */
  float *log_probs;   /* [L][N] f32, log p(action) */
  float *values;      /* [L][N] f32, critic output */
  float *rewards;     /* [L][N] f32 */
  uint8_t *dones;     /* [L][N] u8, 1 when a barrier fired (episode reset) */
  uint8_t *barrier;   /* [L][N] u8: 0 none, 1 profit, 2 stop, 3 time */
  float *advantages;  /* [L][N] f32, GAE with V(L) = 0 */
  float *returns;     /* [L][N] f32, advantages + values */
  float *logits;      /* [L][N][45] f32 or NULL (debug / parity only) */
  uint32_t *counters; /* [3] or NULL: reset then accumulated by this call:
                         [0] non-finite events (a step's logit vector, its
                         value or its reward), [1] episodes whose start had
                         to be clamped, [2] GAE look-backs that gave up
                         waiting (never expected: see gae_scan; the
                         advantages and returns they reach are NaN) */
  void *const *phase_events; /* NULL or [4] caller-created hipEvent_t (as
                         void*), recorded on hip_stream before the rollout
                         kernel, after it (its last part when split), after
                         the value pass and after the GAE scan, for
                         per-phase timing */
} rollout_outputs;

/* Fill `cfg` with the default settings (the values in the comments above)
 * for N episodes of L steps in fp32.  Returns ROLLOUT_EINVAL on NULL. */
int rollout_config_default(rollout_config *cfg, int32_t n_episodes, int32_t n_steps);

/* Create a collector.
 *  actor[6]      = W1[128,54], b1[128], W2[64,128], b2[64], W3[45,64], b3[45]
 *  critic[12]    = W1[512,54], b1, W2[384,512], b2, W3[256,384], b3,
 *                  W4[128,256], b4, W5[64,128], b5, W6[1,64], b6
 *  curiosity[4]  = W1[128,99], b1[128], W2[51,128], b2[51]
 *  (PPO CUDA Pipeline Design, Weight Layout; [out, in] row-major fp32.)
 *  features      = [n_bars][51] f32, prices = [n_bars] f32 (positive).
 * The weights are copied and repacked into the library's own MFMA layout
 * (stream-ordered on hip_stream); the caller may free them afterwards.  The
 * market buffers are BORROWED and must outlive the handle; they are read at
 * every collection.  Device memory for the packed weights and per-collection
 * scratch is allocated here, and, when the rollout is split (see `overlap`),
 * a non-blocking stream of the handle and its events; rollout_destroy
 * releases them.  A collection without recycling whose episodes fill fewer
 * 16-episode workgroups than the device has compute units also keeps a
 * table of the actor's first-layer market-feature part for every step
 * (512 bytes per step and episode, when that is at most 256 MiB), filled at
 * each collection (the same bits as computing it in the step; the
 * environment variable ROLLOUT_FEATURE_TABLE=0, read here, turns it off).
 * Errors: ROLLOUT_EINVAL (NULL, N or L < 1, dims differ from the built net,
 * n_bars < L + 1, div_window outside 1..32, unknown precision, recycle not
 * 0 or 1),
 * ROLLOUT_ENOMEM, ROLLOUT_EHIP. */
int rollout_create(const rollout_config *cfg, const float *const actor[6],
                   const float *const critic[12], const float *const curiosity[4],
                   const float *features, const float *prices, int64_t n_bars,
                   void *hip_stream, rollout_handle *out);

/* Replace the weights after a policy update (PPO CUDA Pipeline Design,
 * Trainer Integration: the actor, critic and curiosity weights are synced to
 * the collector after every update).  Same layout as rollout_create; the
 * weights are repacked on the device.  Stream-ordered: a collection enqueued
 * later on the same stream sees the new weights; one enqueued earlier on
 * another stream must be complete first.
 * Errors: ROLLOUT_EINVAL (NULL handle, array or tensor), ROLLOUT_EHIP. */
int rollout_set_weights(rollout_handle h, const float *const actor[6],
                        const float *const critic[12], const float *const curiosity[4],
                        void *hip_stream);

/* Collect one batch: N episodes x L steps, then GAE (PPO CUDA Pipeline
 * Design, Kernel Phases A and B).  episode_starts = [N] i32 device array, the
 * first bar of each episode; a start outside [0, n_bars - L - 1] is clamped
 * into range on the device and counted in counters[1].  `seed` keys the
 * per-(episode, step) draws.  Calls on one handle must not overlap (they
 * share its scratch); enqueue them on one stream. */
int rollout_collect(rollout_handle h, const int32_t *episode_starts, uint64_t seed,
                    const rollout_outputs *out, void *hip_stream);

/* Profiling aid for the sequential step (PPO CUDA Pipeline Design, Kernel
 * Phases, Phase A), whose chain of dependent work sets the time of a small
 * batch.  A nonzero `enable` makes later rollout_collect calls on the handle
 * run an instrumented build of the step kernel: every wave reads the clock
 * (s_memtime, shader-clock cycles) at each phase boundary of each step and
 * adds the cycles of every phase into a device buffer of the handle
 * (allocated and cleared on the first enable); 0 switches back to the plain
 * kernel.  With `out` (host, u64) not NULL the device is synchronized, the
 * totals gathered since the previous such call are copied to `out` and
 * cleared, and *n_written (if not NULL) gets the number of words:
 * ROLLOUT_STAMP_WORDS per wave, 4 waves per workgroup of 16 episodes,
 * ceil(N / 16) workgroups, so out_len must be at least
 * 64 * ceil(N / 16).  Per wave: [0] state assembly and stores, [1] state
 * barrier, [2] first layer, [3] barrier, [4] second layer, [5] barrier,
 * [6] third layer, [7] barrier, [8] draw, [9] environment step, [10] stores
 * and reset, [11] steps counted, [12] cycles of the whole step loop.  The
 * clock is read through the scalar memory path, whose waits also cover the
 * LDS reads in flight, so the instrumented step is slower than the plain
 * one.  Errors: ROLLOUT_EINVAL (NULL handle, other device, out_len too
 * small), ROLLOUT_ENOMEM, ROLLOUT_EHIP. */
#define ROLLOUT_STAMP_WORDS 16
int rollout_phase_cycles(rollout_handle h, int32_t enable, uint64_t *out, int64_t out_len,
                         int64_t *n_written);

/* Standalone GAE backward scan (PPO CUDA Pipeline Design, Kernel Phases,
 * Phase B) over [L][N] time-major inputs:
 *   delta_t = r_t + gamma * V_{t+1} * (1 - d_t) - V_t,  V_L = last_values[n]
 *             (or 0 when last_values is NULL),
 *   A_t     = delta_t + gamma * lambda * (1 - d_t) * A_{t+1},  A_L = 0,
 *   R_t     = A_t + V_t.
 * rewards, values: [L][N] f32; dones: [L][N] u8 (0 or 1); last_values: [N]
 * f32 or NULL; advantages, returns: [L][N] f32 outputs (may not alias the
 * inputs).  L == 0 or N == 0 is a no-op.  The library keeps a small
 * per-(device, stream) scratch for the inter-chunk carries, allocated on the
 * first call for that stream; concurrent calls on the same stream are
 * serialised by the stream itself.
 * Rollouts longer than 512 steps are cut into 512-step chunks whose carries
 * pass between workgroups through a bounded wait.  A wait that reaches its bound
 * (never expected: every wait is on a workgroup that is already running)
 * ends, and its chunk's carry is NaN, so the advantages and returns of that
 * episode from the chunk back to step 0 are NaN rather than silently wrong;
 * rollout_collect also counts such events in counters[2].  The environment
 * variable ROLLOUT_GAE_SPIN_LIMIT, read at each call, lowers the bound (a
 * number of polls; it cannot raise it); 0 makes every chunk but the latest
 * give up without waiting, which exercises this path deterministically.
 * Errors: ROLLOUT_EINVAL (NULL pointer, negative size), ROLLOUT_ENOMEM,
 * ROLLOUT_EHIP. */
int gae_scan(const float *rewards, const float *values, const uint8_t *dones,
             const float *last_values, int32_t L, int32_t N, float gamma, float lambda,
             float *advantages, float *returns, void *hip_stream);

/* gae_scan without any device allocation, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layout, results (bit for bit) and errors as
 * gae_scan.  Rollouts longer than 512 steps pass carries between 512-step
 * chunks through a scratch that here is a fixed array in the library's
 * device memory (4 MiB + 256 bytes, held by each device the library runs on
 * until the process ends) instead of memory allocated on first use: such a
 * scan needs ceil(L / 512) * N <= 524288 (e.g. L = 4096 with N <= 65536);
 * larger ones are rejected with ROLLOUT_EINVAL before anything is enqueued.
 * Rollouts of at most 512 steps need no scratch and have no such limit.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (its ticket counter and tagged carries; what must start at
 * zero is cleared by a kernel on the caller's stream, never by a memset):
 * calls that overlap on one device race, so callers serialise them, e.g. on
 * one stream.  Errors: as gae_scan, plus ROLLOUT_EINVAL for a scan beyond the
 * scratch and ROLLOUT_EHIP if the array's address cannot be resolved. */
int gae_scan_noalloc(const float *rewards, const float *values, const uint8_t *dones,
                     const float *last_values, int32_t L, int32_t N, float gamma, float lambda,
                     float *advantages, float *returns, void *hip_stream);

/* Release a collector and its device memory (NULL-safe).  Work already
 * enqueued that uses the handle must be complete. */
void rollout_destroy(rollout_handle h);

/* Message of the last failing call on this thread ("" if none).  Valid until
 * the next call into the library on the same thread. */
const char *rollout_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
