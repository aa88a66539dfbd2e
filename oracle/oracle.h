/*
 * CPU ORACLE for fused PPO experience collection -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential C99.  Only the test-suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load this library; the product
 * path (the HIP library) never does, and this code shares no source, header,
 * table or helper with it.
 *
 * Source pages (cited by title and section):
 *   [PPO]  "PPO CUDA Pipeline Design - Zero-Roundtrip Experience Collection
 *           (Phase 2c)": Kernel Phases (Phase A steps 1-12, Phase B GAE),
 *           Weight Layout, Shared Device Functions Header.
 *   [DQN]  "GPU Pipeline Phase 2b: Zero-Roundtrip CUDA Experience Collection":
 *           Kernel Components 1-8 (matvec convention, curiosity encoding,
 *           portfolio, barrier, diversity entropy, reward, TD error, RNG).
 *   [FUSED] "Fused CUDA Training Kernel - Implementation Plan": Task 1 step 3
 *           (45-action factorisation exp = a/9, ord = (a%9)/3, urg = a%3).
 *   The DQN variant of the collection ([DQN] Data Flow, Kernel Components
 *           1, 7 and 8): dueling Q online on the state, epsilon-greedy,
 *           the same environment step and reward, target Q on the next
 *           state and the TD error; priority = |TD|^alpha as in the
 *           priority update of "GPU-Resident Prioritized Experience
 *           Replay" (Sampling Kernels).
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *           Easy as 1, 2, 3", SC'11 (the pages' LCG is replaced by this
 *           counter-based generator keyed by (seed, episode, step, stream)).
 *
 * Precision: the pages' kernel is written in 32-bit float throughout, so the
 * oracle computes in fp32 (ORC_FP32).  ORC_BF16 rounds weights and every
 * layer input to bfloat16 (round-to-nearest-even) and keeps fp32 accumulation.
 * ORC_FP64 is a diagnostic mode: linear layers accumulate in double (result
 * rounded to float) so the oracle's own rounding can be measured.
 *
 * Pinning status of each part is recorded in the test-suite; the composition
 * of the whole rollout (reward terms, barrier semantics) is fixed only by the
 * readings of the pages and is "parity unpinned" beyond its pinned parts.
 */
#ifndef ORC_ORACLE_H
#define ORC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP32 = 0, ORC_BF16 = 1, ORC_FP64 = 2 };

enum {
  ORC_STATE_DIM = 54,   /* 51 market features + 3 portfolio features */
  ORC_N_FEATURES = 51,
  ORC_N_ACTIONS = 45,
  ORC_MAX_WINDOW = 256,
};

/* Scalar settings of one collection run (plain values, host side). */
typedef struct {
  int32_t n_episodes, n_steps;   /* N, L */
  int32_t precision;             /* ORC_FP32 / ORC_BF16 / ORC_FP64 */
  float gamma, lambda;           /* GAE */
  float profit_take, stop_loss;  /* fractions, e.g. 0.02, 0.01 */
  int32_t max_hold;              /* time-exit horizon in bars */
  int32_t div_window;            /* diversity window length */
  float div_threshold;           /* entropy threshold, nats */
  float div_penalty;             /* added when entropy is below threshold */
  float curiosity_coef;          /* bonus = coef * MSE */
  float risk_coef;               /* risk = coef * |exposure| */
  float spread;                  /* constant third portfolio feature */
  float barrier_scale;           /* pnl * (1 + scale * hit) */
  float exposure[5];             /* exposure per exp index a/9 */
  float cost[3];                 /* cost rate per order index (a%9)/3 */
  float urgency_mult;            /* cost * (1 + mult * (a%3)) */
  int32_t recycle;               /* 0: after a done the episode continues on the next bar;
                                    1: it restarts at a fresh random bar (orc_recycle_bar) */
} orc_params;

/* Network weights, host pointers, [out, in] row-major (Candle convention). */
typedef struct {
  const float *aw[3], *ab[3];    /* actor: 54->128->64->45 */
  const float *vw[6], *vb[6];    /* critic: 54->512->384->256->128->64->1 */
  const float *cw[2], *cb[2];    /* curiosity: (54+45)->128->51 */
} orc_nets;

/* Outputs, host pointers, time-major [L][N] (states [L][N][54],
 * logits [L][N][45]).  Nullable: logits, u, cdf_gap, adv, ret. */
typedef struct {
  float *states;
  float *logits;
  float *u;          /* the uniform draw of each step */
  float *cdf_gap;    /* min_k |u - CDF_k| of each step (near-tie screening) */
  int32_t *actions;
  float *log_probs;
  float *values;
  float *rewards;
  uint8_t *dones;
  uint8_t *barrier;  /* 0 none, 1 profit, 2 stop, 3 time */
  float *adv;
  float *ret;
} orc_outputs;

/* --- counter-based RNG ---------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float orc_uniform(uint64_t seed, uint32_t episode, uint32_t step, uint32_t stream);
void orc_uniform_many(uint64_t seed, const uint32_t *episode, const uint32_t *step,
                      uint32_t stream, int64_t n, float *u);

/* --- building blocks (exported so tests can pin them one by one) ---------- */
float orc_bf16_round(float x);
void orc_linear(const float *W, const float *b, const float *x, int in_dim, int out_dim,
                int relu, int precision, float *y);
/* Stable softmax, CDF scan and inverse-CDF draw.  Returns the action,
 * writes log p[action]; cdf (nullable) receives the 45 CDF values;
 * gap (nullable) receives min_k |u - CDF_k|. */
int orc_softmax_sample(const float *logits, int n, float u, float *logp, float *cdf, float *gap);
float orc_log_softmax_at(const float *logits, int n, int a);
void orc_sample_many(const float *logits, int n, const float *u, int64_t count, int32_t *actions);
float orc_entropy3(int n0, int n1, int n2);
int orc_action_exp_index(int a);
int orc_action_ord_index(int a);
int orc_action_urg_index(int a);
float orc_action_exposure(const orc_params *p, int a);
float orc_action_cost(const orc_params *p, int a);
int orc_action_category(int a);

/* Per-episode environment state (portfolio, barrier, diversity window). */
typedef struct {
  float V, e_prev;
  int32_t armed, side, t_open;
  float entry;
  int32_t cnt[3];
  int32_t pushed;
  uint8_t ring[ORC_MAX_WINDOW];
} orc_episode;

void orc_episode_reset(orc_episode *s);
/* Dynamic episode recycling ("GPU Pipeline Phase 2b", Future Phase 3
 * Optimization): the bar at which an episode that ended at step t < L-1
 * restarts.  With R = L - t - 1 steps left, the valid starts are
 * 0 .. n_bars - 1 - R; the start is floor(x range / 2^32) with range =
 * n_bars - R and x the first word of the Philox block with counter
 * (episode, t, 5, 0) and key = the seed. */
int64_t orc_recycle_bar(uint64_t seed, uint32_t episode, int32_t t, int32_t n_steps,
                        int64_t n_bars);
/* One environment step after action a at step t with prices p0 = P[bar],
 * p1 = P[bar+1].  Writes pnl, hit (+1/-1/0), barrier code, diversity term and
 * the exposure taken; returns done (0/1).  Does NOT apply the reset. */
int orc_env_step(const orc_params *p, orc_episode *s, int a, int t, float p0, float p1,
                 float *pnl, int *hit, int *code, float *div, float *exposure);

/* --- GAE ------------------------------------------------------------------ */
void orc_gae(const float *rewards, const float *values, const uint8_t *dones,
             const float *last_values, int32_t L, int32_t N, float gamma, float lambda,
             int precision, float *adv, float *ret);

/* --- whole rollout ---------------------------------------------------------- */
/* starts: [N] first bar of each episode, must satisfy 0 <= start and
 * start + L < n_bars.  forced_actions: NULL or [L][N] (teacher forcing).
 * subset: NULL (all episodes) or n_subset episode indices; only those
 * columns of the outputs are written.  Returns 0, or -1 on bad arguments. */
int orc_rollout(const orc_params *p, const orc_nets *nets, const float *features,
                const float *prices, int64_t n_bars, const int32_t *starts, uint64_t seed,
                const int32_t *forced_actions, const int32_t *subset, int32_t n_subset,
                const orc_outputs *out, int32_t n_threads);

/* --- DQN collection -------------------------------------------------------- */
/* Dueling Q-network ([DQN] Kernel Components 1, with the configured widths):
 * h = ReLU(W2 ReLU(W1 s + b1) + b2)            trunk 54 -> 256 -> 128
 * V = Wv2 ReLU(Wv1 h + bv1) + bv2              value head 128 -> 64 -> 1
 * A = Wa2 ReLU(Wa1 h + ba1) + ba2              advantage head 128 -> 64 -> 45
 * Q_i = V + (A_i - mean(A)), mean = (sum of A left to right) / 45.
 * w/b order: trunk 1, trunk 2, value 1, value 2, advantage 1, advantage 2;
 * [out, in] row-major. */
typedef struct {
  const float *w[6], *b[6];
} orc_qnet;

typedef struct {
  orc_qnet online, target;
  const float *cw[2], *cb[2];    /* curiosity: (54+45)->128->51 */
} orc_dqn_nets;

typedef struct {
  float epsilon;                 /* exploration probability */
  float alpha;                   /* priority = |td|^alpha */
} orc_dqn_params;

/* Outputs, host pointers, [L][N] (states/next_states [L][N][54], q_values
 * [L][N][45]).  Nullable: next_states, q_values, explored, q_gap. */
typedef struct {
  float *states;
  float *next_states;  /* the state after the step, before any reset */
  float *q_values;     /* online Q of the state */
  int32_t *actions;
  uint8_t *explored;   /* 1 when the action is the random one */
  float *q_gap;        /* largest minus second-largest online Q */
  float *q_taken;      /* online Q of the action */
  float *q_next_max;   /* max over actions of the target Q of next_state */
  float *rewards;
  uint8_t *dones;
  uint8_t *barrier;
  float *td;           /* r + gamma (1 - done) q_next_max - q_taken */
  float *priority;     /* |td|^alpha */
} orc_dqn_outputs;

void orc_dueling_q(const orc_qnet *net, const float *s, int precision, float *q);
/* index of the largest element, the lowest index among equal maxima */
int orc_argmax_first(const float *x, int n);
/* the uniformly random action of a draw u in [0, 1): floor(45 u), exact */
int orc_random_action(float u);
/* One DQN collection: for each step the online Q of the state, the action
 * (random with probability epsilon: stream 1 decides, stream 2 picks), the
 * environment step and reward of the PPO collection, the next state before
 * any reset, its target Q, the TD error and the priority; then the reset on
 * done.  Precision ORC_FP32 or ORC_FP64.  Same argument rules as
 * orc_rollout; returns 0, or -1 on bad arguments. */
int orc_dqn_rollout(const orc_params *p, const orc_dqn_params *dq, const orc_dqn_nets *nets,
                    const float *features, const float *prices, int64_t n_bars,
                    const int32_t *starts, uint64_t seed, const int32_t *forced_actions,
                    const int32_t *subset, int32_t n_subset, const orc_dqn_outputs *out,
                    int32_t n_threads);

/* --- prioritized replay: sampling and priority update ----------------------
 * "GPU-Resident Prioritized Experience Replay", Sampling Kernels
 * (proportional) and Error Handling:
 *  - draw b uses the 53-bit uniform u_b of orc_per_uniform;
 *  - with C_k the inclusive prefix sums of the priorities (fp64, left to
 *    right; negative and NaN priorities count as 0) and T = C_{n-1}, the
 *    sample is the first k with C_k > u_b T;
 *  - its importance weight is (n p_k / T)^(-beta), divided by the largest
 *    weight of the batch (fp64, rounded to float at the end);
 *  - if T is not positive and finite the draw is uniform, k = floor(u_b n),
 *    with weight 1.
 * gap (nullable) receives, per draw, the distance from u_b T to the nearest
 * of C_{k-1}, C_k, divided by T (near-tie screening). */
double orc_per_uniform(uint64_t seed, uint32_t draw);
int orc_per_sample(const float *priorities, int64_t n, int32_t batch, uint64_t seed, float beta,
                   int32_t *indices, float *weights, double *gap);
/* Priority update: priority[i_b] = clamp(|td_b|^alpha + epsilon, epsilon,
 * max_priority), with NaN giving epsilon; an index repeated in the batch
 * keeps the largest of its new values (a scatter with repeats has no order
 * on the pages; the largest makes it independent of one).  Returns -1
 * (nothing written) if an index is out of range. */
int orc_per_update(float *priorities, int64_t n, const int32_t *indices, const float *td,
                   int32_t batch, float alpha, float epsilon, float max_priority);

#ifdef __cplusplus
}
#endif
#endif
