/*
 * CPU ORACLE for fused PPO experience collection -- TEST INFRASTRUCTURE ONLY.
 * See oracle.h for the pages this follows, the precision modes and who may
 * load it.  Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp (no fast-math,
 * so every float operation below is one IEEE operation in source order).
 */
#include "oracle.h"

#include <math.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================== */
/* Philox4x32-10 (Salmon et al., SC'11, section 3: the Philox S-box is a    */
/* pair of 32x32->64 multiplications; round keys are bumped by the Weyl     */
/* constants; 10 rounds).                                                    */
/* ======================================================================== */
static void philox_round(uint32_t x[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t y0 = hi1 ^ x[1] ^ k[0];
  const uint32_t y1 = lo1;
  const uint32_t y2 = hi0 ^ x[3] ^ k[1];
  const uint32_t y3 = lo0;
  x[0] = y0; x[1] = y1; x[2] = y2; x[3] = y3;
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(x, k);
  }
  out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
}

/* u = top 24 bits of the first output word times 2^-24: exactly representable
 * in fp32 and strictly below 1. Counter = (episode, step, stream, 0), key =
 * the 64-bit seed split into (low, high) words. */
float orc_uniform(uint64_t seed, uint32_t episode, uint32_t step, uint32_t stream) {
  const uint32_t ctr[4] = {episode, step, stream, 0u};
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (float)(out[0] >> 8) * (1.0f / 16777216.0f);
}

void orc_uniform_many(uint64_t seed, const uint32_t *episode, const uint32_t *step,
                      uint32_t stream, int64_t n, float *u) {
  for (int64_t i = 0; i < n; ++i) u[i] = orc_uniform(seed, episode[i], step[i], stream);
}

/* ======================================================================== */
/* bfloat16 rounding: keep the top 16 bits of the fp32 pattern, rounding to  */
/* nearest with ties to even; NaN stays NaN.                                  */
/* ======================================================================== */
float orc_bf16_round(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) {
    b |= 0x00400000u; /* quiet NaN */
    b &= 0xFFFF0000u;
  } else {
    const uint32_t lsb = (b >> 16) & 1u;
    b = b + 0x7FFFu + lsb;
    b &= 0xFFFF0000u;
  }
  float y;
  memcpy(&y, &b, 4);
  return y;
}

/* ======================================================================== */
/* Linear layer, the pages' matvec convention ([DQN] Kernel Components 1:    */
/* out[j] = bias[j]; for i: out[j] += in[i] * W[j*in + i]), then ReLU.       */
/* ======================================================================== */
void orc_linear(const float *W, const float *b, const float *x, int in_dim, int out_dim,
                int relu, int precision, float *y) {
  for (int j = 0; j < out_dim; ++j) {
    const float *row = W + (int64_t)j * in_dim;
    float v;
    if (precision == ORC_FP64) {
      double acc = (double)b[j];
      for (int i = 0; i < in_dim; ++i) acc += (double)x[i] * (double)row[i];
      v = (float)acc;
    } else if (precision == ORC_BF16) {
      /* W is expected pre-rounded by the caller; inputs rounded here.  The
       * product of two bf16 values is exact in fp32. */
      float acc = b[j];
      for (int i = 0; i < in_dim; ++i) acc += orc_bf16_round(x[i]) * row[i];
      v = acc;
    } else {
      float acc = b[j];
      for (int i = 0; i < in_dim; ++i) acc += x[i] * row[i];
      v = acc;
    }
    y[j] = (relu && !(v > 0.0f)) ? 0.0f : v;
  }
}

/* ======================================================================== */
/* Softmax + CDF scan + inverse-CDF draw ([PPO] Kernel Phases, Phase A       */
/* step 4).  Max-shifted exponentials, left-to-right sums, CDF_k = (sum of   */
/* e_0..e_k) / S, action = first k with u < CDF_k; if rounding leaves        */
/* u >= CDF_{n-1}, the last action with nonzero weight.  log p[a] is taken   */
/* as (l_a - max) - ln S, the same quantity as log(e_a / S).                  */
/* ======================================================================== */
int orc_softmax_sample(const float *logits, int n, float u, float *logp, float *cdf, float *gap) {
  float m = logits[0];
  for (int i = 1; i < n; ++i)
    if (logits[i] > m) m = logits[i];
  float e[ORC_N_ACTIONS > 64 ? ORC_N_ACTIONS : 64];
  float S = 0.0f;
  for (int i = 0; i < n; ++i) {
    e[i] = expf(logits[i] - m);
    S += e[i];
  }
  int a = -1;
  float run = 0.0f, g = INFINITY;
  for (int k = 0; k < n; ++k) {
    run += e[k];
    const float c = run / S;
    if (cdf) cdf[k] = c;
    const float d = fabsf(u - c);
    if (d < g) g = d;
    if (a < 0 && u < c) a = k;
  }
  if (a < 0) {
    for (int k = n - 1; k >= 0; --k)
      if (e[k] > 0.0f) { a = k; break; }
    if (a < 0) a = n - 1;
  }
  if (gap) *gap = g;
  if (logp) *logp = (logits[a] - m) - logf(S);
  return a;
}

/* Many draws from one fixed logit vector (used by the sampling tests). */
void orc_sample_many(const float *logits, int n, const float *u, int64_t count, int32_t *actions) {
  for (int64_t i = 0; i < count; ++i)
    actions[i] = orc_softmax_sample(logits, n, u[i], NULL, NULL, NULL);
}

float orc_log_softmax_at(const float *logits, int n, int a) {
  float m = logits[0];
  for (int i = 1; i < n; ++i)
    if (logits[i] > m) m = logits[i];
  float S = 0.0f;
  for (int i = 0; i < n; ++i) S += expf(logits[i] - m);
  return (logits[a] - m) - logf(S);
}

/* ======================================================================== */
/* 45-action factorisation ([FUSED] Task 1 step 3): exposure index a/9,      */
/* order-type index (a%9)/3, urgency index a%3.                               */
/* ======================================================================== */
int orc_action_exp_index(int a) { return a / 9; }
int orc_action_ord_index(int a) { return (a % 9) / 3; }
int orc_action_urg_index(int a) { return a % 3; }
float orc_action_exposure(const orc_params *p, int a) { return p->exposure[a / 9]; }
float orc_action_cost(const orc_params *p, int a) {
  return p->cost[(a % 9) / 3] * (1.0f + p->urgency_mult * (float)(a % 3));
}
/* Short / flat / long class of an action ([DQN] Kernel Components 2). */
int orc_action_category(int a) {
  const int x = a / 9;
  return (x <= 1) ? 0 : (x == 2 ? 1 : 2);
}

/* Shannon entropy in nats of a 3-class histogram ([DQN] Kernel Components 5,
 * natural log per the workload's "nat" threshold). */
float orc_entropy3(int n0, int n1, int n2) {
  const int n = n0 + n1 + n2;
  if (n <= 0) return 0.0f;
  const int c[3] = {n0, n1, n2};
  float H = 0.0f;
  for (int i = 0; i < 3; ++i) {
    if (c[i] > 0) {
      const float p = (float)c[i] / (float)n;
      H -= p * logf(p);
    }
  }
  return H;
}

/* ======================================================================== */
/* Environment step: portfolio ([DQN] Kernel Components 3), triple barrier    */
/* (4), diversity (5); [PPO] Kernel Phases, Phase A steps 6-8.                 */
/* ======================================================================== */
void orc_episode_reset(orc_episode *s) {
  s->V = 1.0f;
  s->e_prev = 0.0f;
  s->armed = 0;
  s->side = 0;
  s->t_open = 0;
  s->entry = 0.0f;
  s->cnt[0] = s->cnt[1] = s->cnt[2] = 0;
  s->pushed = 0;
  memset(s->ring, 0, sizeof(s->ring));
}

int orc_env_step(const orc_params *p, orc_episode *s, int a, int t, float p0, float p1,
                 float *pnl_out, int *hit_out, int *code_out, float *div_out, float *exp_out) {
  /* portfolio: exposure is a fraction of equity; turnover pays the cost rate */
  const float e = orc_action_exposure(p, a);
  const float c = orc_action_cost(p, a);
  const float ret = p1 / p0 - 1.0f;
  const float pnl = e * ret - c * fabsf(e - s->e_prev);
  s->V = s->V * (1.0f + pnl);

  /* barrier: armed when a position opens from flat or reverses side; a
   * same-side resize keeps the entry; a close disarms */
  if (e != 0.0f) {
    const int side = (e > 0.0f) ? 1 : -1;
    const int prev_side = (s->e_prev > 0.0f) ? 1 : ((s->e_prev < 0.0f) ? -1 : 0);
    if (prev_side == 0 || prev_side != side) {
      s->armed = 1;
      s->side = side;
      s->entry = p0;
      s->t_open = t;
    }
  } else {
    s->armed = 0;
  }
  int hit = 0, code = 0;
  if (s->armed) {
    const float up_pt = 1.0f + p->profit_take, dn_sl = 1.0f - p->stop_loss;
    const float dn_pt = 1.0f - p->profit_take, up_sl = 1.0f + p->stop_loss;
    if (s->side > 0) {
      if (p1 >= s->entry * up_pt) { hit = 1; code = 1; }
      else if (p1 <= s->entry * dn_sl) { hit = -1; code = 2; }
    } else {
      if (p1 <= s->entry * dn_pt) { hit = 1; code = 1; }
      else if (p1 >= s->entry * up_sl) { hit = -1; code = 2; }
    }
    if (code == 0 && (t + 1 - s->t_open) >= p->max_hold) code = 3;
  }

  /* diversity: class of this action enters the sliding window */
  const int W = p->div_window;
  const int cat = orc_action_category(a);
  const int pos = s->pushed % W;
  if (s->pushed >= W) s->cnt[s->ring[pos]] -= 1;
  s->ring[pos] = (uint8_t)cat;
  s->cnt[cat] += 1;
  s->pushed += 1;
  const float H = orc_entropy3(s->cnt[0], s->cnt[1], s->cnt[2]);
  const float div = (H < p->div_threshold) ? p->div_penalty : 0.0f;

  s->e_prev = e;
  *pnl_out = pnl;
  *hit_out = hit;
  *code_out = code;
  *div_out = div;
  *exp_out = e;
  return code != 0;
}

int64_t orc_recycle_bar(uint64_t seed, uint32_t episode, int32_t t, int32_t n_steps,
                        int64_t n_bars) {
  const int64_t remaining = (int64_t)n_steps - t - 1;
  const uint64_t range = (uint64_t)(n_bars - remaining);
  const uint32_t ctr[4] = {episode, (uint32_t)t, 5u, 0u};
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (int64_t)(((uint64_t)out[0] * range) >> 32);
}

/* ======================================================================== */
/* GAE ([PPO] Kernel Phases, Phase B): backward over t with V(L) = last value */
/* (0 when absent), delta_t = r_t + gamma V_{t+1} (1-d_t) - V_t,              */
/* A_t = delta_t + gamma lambda (1-d_t) A_{t+1}, A_L = 0, R_t = A_t + V_t.    */
/* ======================================================================== */
static void gae_column(const float *r, const float *v, const uint8_t *d, float vlast, int32_t L,
                       int64_t stride, int64_t col, float gamma, float lambda, int precision,
                       float *adv, float *ret) {
  if (precision == ORC_FP64) {
    double A = 0.0;
    double vnext = (double)vlast;
    for (int32_t t = L - 1; t >= 0; --t) {
      const int64_t i = (int64_t)t * stride + col;
      const double nd = 1.0 - (double)d[i];
      const double delta = (double)r[i] + (double)gamma * vnext * nd - (double)v[i];
      A = delta + (double)gamma * (double)lambda * nd * A;
      if (adv) adv[i] = (float)A;
      if (ret) ret[i] = (float)(A + (double)v[i]);
      vnext = (double)v[i];
    }
  } else {
    float A = 0.0f;
    float vnext = vlast;
    for (int32_t t = L - 1; t >= 0; --t) {
      const int64_t i = (int64_t)t * stride + col;
      const float nd = 1.0f - (float)d[i];
      const float delta = r[i] + gamma * vnext * nd - v[i];
      A = delta + gamma * lambda * nd * A;
      if (adv) adv[i] = A;
      if (ret) ret[i] = A + v[i];
      vnext = v[i];
    }
  }
}

void orc_gae(const float *rewards, const float *values, const uint8_t *dones,
             const float *last_values, int32_t L, int32_t N, float gamma, float lambda,
             int precision, float *adv, float *ret) {
  for (int32_t n = 0; n < N; ++n)
    gae_column(rewards, values, dones, last_values ? last_values[n] : 0.0f, L, N, n, gamma,
               lambda, precision, adv, ret);
}

/* ======================================================================== */
/* Whole rollout ([PPO] Kernel Phases, Phase A steps 1-12, then Phase B).    */
/* One episode at a time; episodes never interact, so the episode loop is    */
/* spread over host threads.                                                  */
/* ======================================================================== */
#define H_MAX 512

static int collect_episode(const orc_params *p, const orc_nets *nets, const float *features,
                           const float *prices, int64_t n_bars, const int32_t *starts, uint64_t seed,
                           const int32_t *forced, int32_t n, const orc_outputs *out) {
  const int32_t N = p->n_episodes, L = p->n_steps;
  const int prec = p->precision;
  static const int adim[4] = {54, 128, 64, 45};
  static const int vdim[7] = {54, 512, 384, 256, 128, 64, 1};
  float s[ORC_STATE_DIM], xa[H_MAX], xb[H_MAX], logits[ORC_N_ACTIONS];
  float cin[ORC_STATE_DIM + ORC_N_ACTIONS], ch[128], pred[ORC_N_FEATURES];
  orc_episode ep;
  orc_episode_reset(&ep);
  const float V0 = 1.0f;

  int64_t bar = starts[n];
  for (int32_t t = 0; t < L; ++t) {
    const int64_t o = (int64_t)t * N + n;
    /* 1-2. state = 51 market features + normalised value, position, spread */
    const float *f = features + bar * ORC_N_FEATURES;
    for (int i = 0; i < ORC_N_FEATURES; ++i) s[i] = f[i];
    s[51] = ep.V / V0 - 1.0f;
    s[52] = ep.e_prev;
    s[53] = p->spread;
    memcpy(out->states + o * ORC_STATE_DIM, s, sizeof(s));

    /* 3. actor 54 -> 128 (ReLU) -> 64 (ReLU) -> 45 logits */
    orc_linear(nets->aw[0], nets->ab[0], s, adim[0], adim[1], 1, prec, xa);
    orc_linear(nets->aw[1], nets->ab[1], xa, adim[1], adim[2], 1, prec, xb);
    orc_linear(nets->aw[2], nets->ab[2], xb, adim[2], adim[3], 0, prec, logits);
    if (out->logits) memcpy(out->logits + o * ORC_N_ACTIONS, logits, sizeof(logits));

    /* 4. softmax + categorical draw */
    const float u = orc_uniform(seed, (uint32_t)n, (uint32_t)t, 0u);
    float logp, gap;
    int a = orc_softmax_sample(logits, ORC_N_ACTIONS, u, &logp, NULL, &gap);
    if (forced) {
      a = forced[o];
      if (a < 0 || a >= ORC_N_ACTIONS) return -1;
      logp = orc_log_softmax_at(logits, ORC_N_ACTIONS, a);
    }
    if (out->u) out->u[o] = u;
    if (out->cdf_gap) out->cdf_gap[o] = gap;

    /* 5. critic 54 -> 512 -> 384 -> 256 -> 128 -> 64 (all ReLU) -> 1 */
    float *cur = xa, *nxt = xb;
    memcpy(cur, s, sizeof(s));
    for (int l = 0; l < 6; ++l) {
      orc_linear(nets->vw[l], nets->vb[l], cur, vdim[l], vdim[l + 1], l < 5, prec, nxt);
      float *tmp = cur; cur = nxt; nxt = tmp;
    }
    const float value = cur[0];

    /* 6-8. portfolio, barrier, diversity */
    float pnl, div, e;
    int hit, code;
    const int done = orc_env_step(p, &ep, a, t, prices[bar], prices[bar + 1], &pnl, &hit, &code,
                                  &div, &e);

    /* 9. curiosity: forward model on [state, one-hot(action)] predicts the
     * next bar's 51 features; bonus = coef * mean squared error */
    for (int i = 0; i < ORC_STATE_DIM; ++i) cin[i] = s[i];
    for (int i = 0; i < ORC_N_ACTIONS; ++i) cin[ORC_STATE_DIM + i] = (i == a) ? 1.0f : 0.0f;
    orc_linear(nets->cw[0], nets->cb[0], cin, ORC_STATE_DIM + ORC_N_ACTIONS, 128, 1, prec, ch);
    orc_linear(nets->cw[1], nets->cb[1], ch, 128, ORC_N_FEATURES, 0, prec, pred);
    const float *fn = features + (bar + 1) * ORC_N_FEATURES;
    float se = 0.0f;
    for (int j = 0; j < ORC_N_FEATURES; ++j) {
      const float dj = pred[j] - fn[j];
      se += dj * dj;
    }
    const float mse = se / (float)ORC_N_FEATURES;
    const float bonus = p->curiosity_coef * mse;

    /* 10. reward = pnl (1 + scale * hit) + diversity + curiosity - risk */
    const float reward =
        pnl * (1.0f + p->barrier_scale * (float)hit) + div + bonus - p->risk_coef * fabsf(e);

    /* 11. store */
    out->actions[o] = a;
    out->log_probs[o] = logp;
    out->values[o] = value;
    out->rewards[o] = reward;
    out->dones[o] = (uint8_t)done;
    out->barrier[o] = (uint8_t)code;

    /* 12. reset on done; the bar pointer keeps advancing, or with
     * recycling the episode restarts at a fresh random bar */
    if (done) orc_episode_reset(&ep);
    bar = (done && p->recycle && t + 1 < L)
              ? orc_recycle_bar(seed, (uint32_t)n, t, L, n_bars)
              : bar + 1;
  }

  /* Phase B: GAE over this episode's column, V(L) = 0 */
  if (out->adv || out->ret)
    gae_column(out->rewards, out->values, out->dones, 0.0f, L, N, n, p->gamma, p->lambda,
               prec == ORC_FP64 ? ORC_FP64 : ORC_FP32, out->adv, out->ret);
  return 0;
}

static float *bf16_copy(const float *w, int64_t count) {
  float *c = (float *)malloc((size_t)count * sizeof(float));
  if (!c) return NULL;
  for (int64_t i = 0; i < count; ++i) c[i] = orc_bf16_round(w[i]);
  return c;
}

int orc_rollout(const orc_params *p, const orc_nets *nets_in, const float *features,
                const float *prices, int64_t n_bars, const int32_t *starts, uint64_t seed,
                const int32_t *forced_actions, const int32_t *subset, int32_t n_subset,
                const orc_outputs *out, int32_t n_threads) {
  if (!p || !nets_in || !features || !prices || !starts || !out) return -1;
  if (p->n_episodes <= 0 || p->n_steps <= 0) return -1;
  if (p->div_window <= 0 || p->div_window > ORC_MAX_WINDOW) return -1;
  if (!out->states || !out->actions || !out->log_probs || !out->values || !out->rewards ||
      !out->dones || !out->barrier)
    return -1;
  const int32_t N = p->n_episodes, L = p->n_steps;
  for (int32_t n = 0; n < N; ++n)
    if (starts[n] < 0 || (int64_t)starts[n] + L >= n_bars) return -1;

  /* bf16 mode: weights rounded once (biases stay fp32) */
  orc_nets nets = *nets_in;
  float *owned[11] = {0};
  int n_owned = 0, failed = 0;
  if (p->precision == ORC_BF16) {
    static const int adim[4] = {54, 128, 64, 45};
    static const int vdim[7] = {54, 512, 384, 256, 128, 64, 1};
    static const int cdim[3] = {99, 128, 51};
    for (int l = 0; l < 3; ++l) {
      float *c = bf16_copy(nets_in->aw[l], (int64_t)adim[l] * adim[l + 1]);
      owned[n_owned++] = c; nets.aw[l] = c; failed |= !c;
    }
    for (int l = 0; l < 6; ++l) {
      float *c = bf16_copy(nets_in->vw[l], (int64_t)vdim[l] * vdim[l + 1]);
      owned[n_owned++] = c; nets.vw[l] = c; failed |= !c;
    }
    for (int l = 0; l < 2; ++l) {
      float *c = bf16_copy(nets_in->cw[l], (int64_t)cdim[l] * cdim[l + 1]);
      owned[n_owned++] = c; nets.cw[l] = c; failed |= !c;
    }
  }
  int rc = 0;
  if (!failed) {
    const int32_t count = subset ? n_subset : N;
#ifdef _OPENMP
    const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : rc)
#endif
    for (int32_t i = 0; i < count; ++i) {
      const int32_t n = subset ? subset[i] : i;
      if (n < 0 || n >= N) { rc |= 1; continue; }
      if (collect_episode(p, &nets, features, prices, n_bars, starts, seed, forced_actions, n, out))
        rc |= 1;
    }
  }
  (void)n_threads;
  for (int i = 0; i < n_owned; ++i) free(owned[i]);
  return (failed || rc) ? -1 : 0;
}

/* ======================================================================== */
/* DQN collection ([DQN] Data Flow steps 1-15, Kernel Components 1, 7, 8).   */
/* ======================================================================== */
void orc_dueling_q(const orc_qnet *net, const float *s, int precision, float *q) {
  float h1[256], h2[128], v1[64], a1[64], v, a[ORC_N_ACTIONS];
  orc_linear(net->w[0], net->b[0], s, ORC_STATE_DIM, 256, 1, precision, h1);
  orc_linear(net->w[1], net->b[1], h1, 256, 128, 1, precision, h2);
  orc_linear(net->w[2], net->b[2], h2, 128, 64, 1, precision, v1);
  orc_linear(net->w[3], net->b[3], v1, 64, 1, 0, precision, &v);
  orc_linear(net->w[4], net->b[4], h2, 128, 64, 1, precision, a1);
  orc_linear(net->w[5], net->b[5], a1, 64, ORC_N_ACTIONS, 0, precision, a);
  float sum = 0.0f;
  for (int i = 0; i < ORC_N_ACTIONS; ++i) sum += a[i];
  const float mean = sum / (float)ORC_N_ACTIONS;
  for (int i = 0; i < ORC_N_ACTIONS; ++i) q[i] = v + (a[i] - mean);
}

int orc_argmax_first(const float *x, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

int orc_random_action(float u) {
  /* u = m * 2^-24 with m < 2^24, so floor(45 u) = (45 m) >> 24 exactly */
  const uint32_t m = (uint32_t)(u * 16777216.0f);
  return (int)(((uint64_t)m * (uint64_t)ORC_N_ACTIONS) >> 24);
}

static int collect_dqn_episode(const orc_params *p, const orc_dqn_params *dq,
                               const orc_dqn_nets *nets, const float *features,
                               const float *prices, int64_t n_bars, const int32_t *starts,
                               uint64_t seed,
                               const int32_t *forced, int32_t n, const orc_dqn_outputs *out) {
  const int32_t N = p->n_episodes, L = p->n_steps;
  const int prec = p->precision;
  float s[ORC_STATE_DIM], sn[ORC_STATE_DIM], q[ORC_N_ACTIONS], qt[ORC_N_ACTIONS];
  float cin[ORC_STATE_DIM + ORC_N_ACTIONS], ch[128], pred[ORC_N_FEATURES];
  orc_episode ep;
  orc_episode_reset(&ep);
  const float V0 = 1.0f;

  int64_t bar = starts[n];
  for (int32_t t = 0; t < L; ++t) {
    const int64_t o = (int64_t)t * N + n;
    /* 1-3. state = 51 market features + normalised value, position, spread */
    const float *f = features + bar * ORC_N_FEATURES;
    for (int i = 0; i < ORC_N_FEATURES; ++i) s[i] = f[i];
    s[51] = ep.V / V0 - 1.0f;
    s[52] = ep.e_prev;
    s[53] = p->spread;
    memcpy(out->states + o * ORC_STATE_DIM, s, sizeof(s));

    /* 4. online dueling Q of the state */
    orc_dueling_q(&nets->online, s, prec, q);
    if (out->q_values) memcpy(out->q_values + o * ORC_N_ACTIONS, q, sizeof(q));

    /* 5. epsilon-greedy: stream 1 decides, stream 2 picks the random action */
    const float u_explore = orc_uniform(seed, (uint32_t)n, (uint32_t)t, 1u);
    const int explore = u_explore < dq->epsilon;
    const int greedy = orc_argmax_first(q, ORC_N_ACTIONS);
    int a = explore ? orc_random_action(orc_uniform(seed, (uint32_t)n, (uint32_t)t, 2u)) : greedy;
    if (forced) {
      a = forced[o];
      if (a < 0 || a >= ORC_N_ACTIONS) return -1;
    }
    if (out->explored) out->explored[o] = (uint8_t)explore;
    if (out->q_gap) {
      float second = -INFINITY;
      for (int i = 0; i < ORC_N_ACTIONS; ++i)
        if (i != greedy && q[i] > second) second = q[i];
      out->q_gap[o] = q[greedy] - second;
    }
    const float q_taken = q[a];

    /* 6-8. portfolio, barrier, diversity */
    float pnl, div, e;
    int hit, code;
    const int done = orc_env_step(p, &ep, a, t, prices[bar], prices[bar + 1], &pnl, &hit, &code,
                                  &div, &e);

    /* 9. curiosity on [state, one-hot(action)] against the next bar */
    for (int i = 0; i < ORC_STATE_DIM; ++i) cin[i] = s[i];
    for (int i = 0; i < ORC_N_ACTIONS; ++i) cin[ORC_STATE_DIM + i] = (i == a) ? 1.0f : 0.0f;
    orc_linear(nets->cw[0], nets->cb[0], cin, ORC_STATE_DIM + ORC_N_ACTIONS, 128, 1, prec, ch);
    orc_linear(nets->cw[1], nets->cb[1], ch, 128, ORC_N_FEATURES, 0, prec, pred);
    const float *fn = features + (bar + 1) * ORC_N_FEATURES;
    float se = 0.0f;
    for (int j = 0; j < ORC_N_FEATURES; ++j) {
      const float dj = pred[j] - fn[j];
      se += dj * dj;
    }
    const float bonus = p->curiosity_coef * (se / (float)ORC_N_FEATURES);

    /* 13. reward, as in the PPO collection */
    const float reward =
        pnl * (1.0f + p->barrier_scale * (float)hit) + div + bonus - p->risk_coef * fabsf(e);

    /* 10-12. next state (after the trade, before any reset), target Q, TD */
    for (int i = 0; i < ORC_N_FEATURES; ++i) sn[i] = fn[i];
    sn[51] = ep.V / V0 - 1.0f;
    sn[52] = ep.e_prev;
    sn[53] = p->spread;
    if (out->next_states) memcpy(out->next_states + o * ORC_STATE_DIM, sn, sizeof(sn));
    orc_dueling_q(&nets->target, sn, prec, qt);
    float qmax = qt[0];
    for (int i = 1; i < ORC_N_ACTIONS; ++i) qmax = qt[i] > qmax ? qt[i] : qmax;
    const float td = reward + p->gamma * qmax * (float)(1 - done) - q_taken;

    /* 14. store */
    out->actions[o] = a;
    out->q_taken[o] = q_taken;
    out->q_next_max[o] = qmax;
    out->rewards[o] = reward;
    out->dones[o] = (uint8_t)done;
    out->barrier[o] = (uint8_t)code;
    out->td[o] = td;
    out->priority[o] = powf(fabsf(td), dq->alpha);

    /* 15. reset on done; the bar pointer keeps advancing, or with
     * recycling the episode restarts at a fresh random bar */
    if (done) orc_episode_reset(&ep);
    bar = (done && p->recycle && t + 1 < L)
              ? orc_recycle_bar(seed, (uint32_t)n, t, L, n_bars)
              : bar + 1;
  }
  return 0;
}

int orc_dqn_rollout(const orc_params *p, const orc_dqn_params *dq, const orc_dqn_nets *nets,
                    const float *features, const float *prices, int64_t n_bars,
                    const int32_t *starts, uint64_t seed, const int32_t *forced_actions,
                    const int32_t *subset, int32_t n_subset, const orc_dqn_outputs *out,
                    int32_t n_threads) {
  if (!p || !dq || !nets || !features || !prices || !starts || !out) return -1;
  if (p->n_episodes <= 0 || p->n_steps <= 0) return -1;
  if (p->precision != ORC_FP32 && p->precision != ORC_FP64) return -1;
  if (p->div_window <= 0 || p->div_window > ORC_MAX_WINDOW) return -1;
  if (!out->states || !out->actions || !out->q_taken || !out->q_next_max || !out->rewards ||
      !out->dones || !out->barrier || !out->td || !out->priority)
    return -1;
  const int32_t N = p->n_episodes, L = p->n_steps;
  for (int32_t n = 0; n < N; ++n)
    if (starts[n] < 0 || (int64_t)starts[n] + L >= n_bars) return -1;
  int rc = 0;
  const int32_t count = subset ? n_subset : N;
#ifdef _OPENMP
  const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : rc)
#endif
  for (int32_t i = 0; i < count; ++i) {
    const int32_t n = subset ? subset[i] : i;
    if (n < 0 || n >= N) { rc |= 1; continue; }
    if (collect_dqn_episode(p, dq, nets, features, prices, n_bars, starts, seed, forced_actions, n,
                            out))
      rc |= 1;
  }
  (void)n_threads;
  return rc ? -1 : 0;
}

/* ======================================================================== */
/* Prioritized replay ("GPU-Resident Prioritized Experience Replay",         */
/* Sampling Kernels: proportional sampling, IS weights, priority update).    */
/* ======================================================================== */
double orc_per_uniform(uint64_t seed, uint32_t draw) {
  /* counter (draw, 0, 4, 0): 53 bits from the first two output words */
  const uint32_t ctr[4] = {draw, 0u, 4u, 0u};
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  const uint64_t m = ((uint64_t)out[0] << 21) | (uint64_t)(out[1] >> 11);
  return (double)m * (1.0 / 9007199254740992.0);
}

static double per_value(float p) { return (p > 0.0f) ? (double)p : 0.0; } /* NaN, <0 -> 0 */

int orc_per_sample(const float *priorities, int64_t n, int32_t batch, uint64_t seed, float beta,
                   int32_t *indices, float *weights, double *gap) {
  if (!priorities || !indices || !weights || n <= 0 || batch < 0) return -1;
  double *C = (double *)malloc((size_t)n * sizeof(double));
  double *w = (double *)malloc((size_t)(batch > 0 ? batch : 1) * sizeof(double));
  if (!C || !w) { free(C); free(w); return -1; }
  double run = 0.0;
  for (int64_t k = 0; k < n; ++k) {
    run += per_value(priorities[k]);
    C[k] = run;
  }
  const double T = run;
  const int uniform = !(T > 0.0) || isinf(T);
  double wmax = 0.0;
  for (int32_t b = 0; b < batch; ++b) {
    const double u = orc_per_uniform(seed, (uint32_t)b);
    int64_t k;
    if (uniform) {
      k = (int64_t)(u * (double)n);
      if (k >= n) k = n - 1;
      w[b] = 1.0;
      if (gap) gap[b] = 1.0;
    } else {
      const double target = u * T;
      int64_t lo = 0, hi = n - 1; /* first k with C[k] > target; C[n-1] = T > target */
      while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (C[mid] > target) hi = mid; else lo = mid + 1;
      }
      k = lo;
      /* only if rounding put u T at T itself: the last priority with weight */
      if (!(C[k] > target))
        while (k > 0 && per_value(priorities[k]) == 0.0) --k;
      w[b] = pow((double)n * per_value(priorities[k]) / T, -(double)beta);
      if (gap) {
        const double below = k > 0 ? target - C[k - 1] : target;
        const double above = C[k] - target;
        gap[b] = (below < above ? below : above) / T;
      }
    }
    indices[b] = (int32_t)k;
    if (w[b] > wmax) wmax = w[b];
  }
  for (int32_t b = 0; b < batch; ++b) weights[b] = (float)(w[b] / wmax);
  free(C);
  free(w);
  return 0;
}

int orc_per_update(float *priorities, int64_t n, const int32_t *indices, const float *td,
                   int32_t batch, float alpha, float epsilon, float max_priority) {
  if (!priorities || !indices || !td || batch < 0) return -1;
  for (int32_t b = 0; b < batch; ++b)
    if (indices[b] < 0 || (int64_t)indices[b] >= n) return -1;
  unsigned char *seen = (unsigned char *)calloc((size_t)(n > 0 ? n : 1), 1);
  if (!seen) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    float v = powf(fabsf(td[b]), alpha) + epsilon;
    if (!(v >= epsilon)) v = epsilon; /* NaN */
    if (v > max_priority) v = max_priority;
    const int32_t i = indices[b];
    if (!seen[i] || v > priorities[i]) priorities[i] = v; /* repeats keep the largest */
    seen[i] = 1;
  }
  free(seen);
  return 0;
}
