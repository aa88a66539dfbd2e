/*
 * Drives every entry point of the CPU oracle (test infrastructure) on small
 * inputs and on rejected arguments, for an AddressSanitizer +
 * UndefinedBehaviorSanitizer build: any out-of-bounds access, use of freed
 * memory or undefined operation aborts the program with a report.  Exit
 * status 0 means every call ran clean and returned what it must.
 * Built and run by tests/test_sanitizers.py (gcc, host only).
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* test data only: a 64-bit LCG */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss(void) {
  const double u = unif() + 1e-12, v = unif();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static float *rand_arr(size_t n, float scale) {
  float *a = (float *)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) a[i] = gauss() * scale;
  return a;
}
static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

static orc_params params(int N, int L, int precision, int recycle) {
  orc_params p;
  memset(&p, 0, sizeof(p));
  p.n_episodes = N; p.n_steps = L; p.precision = precision;
  p.gamma = 0.99f; p.lambda = 0.95f; p.profit_take = 0.02f; p.stop_loss = 0.01f;
  p.max_hold = 50; p.div_window = 20; p.div_threshold = 1.0f; p.div_penalty = -0.1f;
  p.curiosity_coef = 0.01f; p.risk_coef = 0.01f; p.spread = 0.0005f; p.barrier_scale = 0.5f;
  const float ex[5] = {-1.0f, -0.5f, 0.0f, 0.5f, 1.0f}, co[3] = {2e-4f, 5e-4f, 1e-3f};
  memcpy(p.exposure, ex, sizeof(ex));
  memcpy(p.cost, co, sizeof(co));
  p.urgency_mult = 0.5f; p.recycle = recycle;
  return p;
}

int main(void) {
  enum { N = 5, L = 30, BARS = 400 };
  /* market: AR(1) features, a geometric random walk of prices */
  float *F = (float *)malloc(sizeof(float) * BARS * 51), *P = (float *)malloc(sizeof(float) * BARS);
  for (int j = 0; j < 51; ++j) F[j] = gauss() * 2.3f;
  for (int b = 1; b < BARS; ++b)
    for (int j = 0; j < 51; ++j) F[b * 51 + j] = 0.9f * F[(b - 1) * 51 + j] + gauss();
  P[0] = 100.0f;
  for (int b = 1; b < BARS; ++b) P[b] = P[b - 1] * expf(0.01f * gauss());
  int32_t starts[N];
  for (int n = 0; n < N; ++n) starts[n] = (int32_t)(unif() * (BARS - L - 1));

  static const int adim[4] = {54, 128, 64, 45}, vdim[7] = {54, 512, 384, 256, 128, 64, 1},
                   cdim[3] = {99, 128, 51};
  orc_nets nets;
  float *owned[64];
  int no = 0;
  for (int l = 0; l < 3; ++l) {
    nets.aw[l] = owned[no++] = rand_arr((size_t)adim[l] * adim[l + 1], sqrtf(2.0f / adim[l]));
    nets.ab[l] = owned[no++] = rand_arr((size_t)adim[l + 1], 0.1f);
  }
  for (int l = 0; l < 6; ++l) {
    nets.vw[l] = owned[no++] = rand_arr((size_t)vdim[l] * vdim[l + 1], sqrtf(2.0f / vdim[l]));
    nets.vb[l] = owned[no++] = rand_arr((size_t)vdim[l + 1], 0.1f);
  }
  for (int l = 0; l < 2; ++l) {
    nets.cw[l] = owned[no++] = rand_arr((size_t)cdim[l] * cdim[l + 1], sqrtf(2.0f / cdim[l]));
    nets.cb[l] = owned[no++] = rand_arr((size_t)cdim[l + 1], 0.1f);
  }

  const size_t NL = (size_t)N * L;
  float *states = malloc(sizeof(float) * NL * 54), *logits = malloc(sizeof(float) * NL * 45);
  float *u = malloc(sizeof(float) * NL), *gap = malloc(sizeof(float) * NL);
  int32_t *actions = malloc(sizeof(int32_t) * NL), *forced = malloc(sizeof(int32_t) * NL);
  float *logp = malloc(sizeof(float) * NL), *val = malloc(sizeof(float) * NL);
  float *rew = malloc(sizeof(float) * NL), *adv = malloc(sizeof(float) * NL);
  float *ret = malloc(sizeof(float) * NL);
  uint8_t *dones = malloc(NL), *barrier = malloc(NL);
  orc_outputs out = {states, logits, u, gap, actions, logp, val, rew, dones, barrier, adv, ret};

  for (int prec = 0; prec < 3; ++prec)
    for (int rec = 0; rec < 2; ++rec) {
      orc_params p = params(N, L, prec, rec);
      CHECK(orc_rollout(&p, &nets, F, P, BARS, starts, 12345u, NULL, NULL, 0, &out, 2) == 0);
    }
  orc_params p = params(N, L, ORC_FP32, 0);
  for (size_t i = 0; i < NL; ++i) forced[i] = (int32_t)(i % 45);
  const int32_t subset[2] = {4, 1};
  CHECK(orc_rollout(&p, &nets, F, P, BARS, starts, 7u, forced, subset, 2, &out, 1) == 0);
  /* rejected arguments */
  forced[3] = 45;
  CHECK(orc_rollout(&p, &nets, F, P, BARS, starts, 7u, forced, NULL, 0, &out, 1) == -1);
  const int32_t bad_subset[1] = {N};
  CHECK(orc_rollout(&p, &nets, F, P, BARS, starts, 7u, NULL, bad_subset, 1, &out, 1) == -1);
  int32_t bad_starts[N];
  memcpy(bad_starts, starts, sizeof(bad_starts));
  bad_starts[2] = BARS - L;  /* start + L must stay below n_bars */
  CHECK(orc_rollout(&p, &nets, F, P, BARS, bad_starts, 7u, NULL, NULL, 0, &out, 1) == -1);
  CHECK(orc_rollout(NULL, &nets, F, P, BARS, starts, 7u, NULL, NULL, 0, &out, 1) == -1);
  orc_params pw = params(N, L, ORC_FP32, 0);
  pw.div_window = ORC_MAX_WINDOW + 1;
  CHECK(orc_rollout(&pw, &nets, F, P, BARS, starts, 7u, NULL, NULL, 0, &out, 1) == -1);

  /* GAE with and without bootstrap values, every precision */
  float lastv[N];
  for (int n = 0; n < N; ++n) lastv[n] = gauss();
  for (int prec = 0; prec < 3; prec += 2) {
    orc_gae(rew, val, dones, lastv, L, N, 0.99f, 0.95f, prec, adv, ret);
    orc_gae(rew, val, dones, NULL, L, N, 0.99f, 0.95f, prec, adv, NULL);
  }

#ifdef PLANT_OUT_OF_BOUNDS
  /* a planted mistake: one episode more than the buffers hold */
  orc_gae(rew, val, dones, NULL, L, N + 1, 0.99f, 0.95f, ORC_FP32, adv, ret);
#endif

  /* DQN collection */
  static const int qd[6][2] = {{54, 256}, {256, 128}, {128, 64}, {64, 1}, {128, 64}, {64, 45}};
  orc_dqn_nets dn;
  for (int net = 0; net < 2; ++net)
    for (int l = 0; l < 6; ++l) {
      float *w = owned[no++] = rand_arr((size_t)qd[l][0] * qd[l][1], sqrtf(2.0f / qd[l][0]));
      float *b = owned[no++] = rand_arr((size_t)qd[l][1], 0.1f);
      if (net == 0) { dn.online.w[l] = w; dn.online.b[l] = b; }
      else { dn.target.w[l] = w; dn.target.b[l] = b; }
    }
  for (int l = 0; l < 2; ++l) { dn.cw[l] = nets.cw[l]; dn.cb[l] = nets.cb[l]; }
  float *nstates = malloc(sizeof(float) * NL * 54), *qv = malloc(sizeof(float) * NL * 45);
  float *qgap = malloc(sizeof(float) * NL), *qt = malloc(sizeof(float) * NL);
  float *qn = malloc(sizeof(float) * NL), *td = malloc(sizeof(float) * NL);
  float *prio = malloc(sizeof(float) * NL);
  uint8_t *expl = malloc(NL);
  orc_dqn_outputs dout = {states, nstates, qv, actions, expl, qgap, qt, qn, rew, dones, barrier,
                          td, prio};
  orc_dqn_params dq = {0.1f, 0.6f};
  for (int rec = 0; rec < 2; ++rec) {
    orc_params pd = params(N, L, ORC_FP32, rec);
    CHECK(orc_dqn_rollout(&pd, &dq, &dn, F, P, BARS, starts, 99u, NULL, NULL, 0, &dout, 2) == 0);
  }
  orc_params pd = params(N, L, ORC_FP64, 0);
  for (size_t i = 0; i < NL; ++i) forced[i] = (int32_t)((i * 7) % 45);
  CHECK(orc_dqn_rollout(&pd, &dq, &dn, F, P, BARS, starts, 99u, forced, subset, 2, &dout, 1) == 0);
  CHECK(orc_dqn_rollout(&pd, &dq, &dn, F, P, BARS, bad_starts, 99u, NULL, NULL, 0, &dout, 1) == -1);

  /* building blocks at their edges */
  float lg[45];
  for (int i = 0; i < 45; ++i) lg[i] = (i == 44) ? -INFINITY : gauss();
  float lp, cdf[45], g;
  CHECK(orc_softmax_sample(lg, 45, 0.999999f, &lp, cdf, &g) >= 0);
  CHECK(orc_random_action(0.99999994f) == 44 && orc_random_action(0.0f) == 0);
  CHECK(orc_argmax_first(lg, 45) >= 0);
  CHECK(orc_entropy3(0, 0, 0) == 0.0f && orc_entropy3(20, 0, 0) == 0.0f);
  CHECK(isnan(orc_bf16_round(NAN)));
  for (int t = 0; t < 200; ++t)
    CHECK(orc_recycle_bar(5u, 3u, t % L, L, BARS) <= BARS - (L - (t % L) - 1) - 1);

  /* prioritized replay, with zero, negative and NaN priorities */
  enum { NP = 3000, B = 64 };
  float *pr = rand_arr(NP, 1.0f);
  for (int i = 0; i < NP; ++i) pr[i] = fabsf(pr[i]);
  pr[5] = 0.0f; pr[6] = -1.0f; pr[7] = NAN;
  int32_t idx[B];
  float w[B], tdb[B];
  double gaps[B];
  CHECK(orc_per_sample(pr, NP, B, 11u, 0.4f, idx, w, gaps) == 0);
  for (int b = 0; b < B; ++b) CHECK(idx[b] >= 0 && idx[b] < NP);
  for (int b = 0; b < B; ++b) tdb[b] = gauss();
  tdb[0] = NAN; tdb[1] = INFINITY;
  CHECK(orc_per_update(pr, NP, idx, tdb, B, 0.6f, 1e-3f, 100.0f) == 0);
  idx[3] = NP;
  CHECK(orc_per_update(pr, NP, idx, tdb, B, 0.6f, 1e-3f, 100.0f) == -1);
  float zero[4] = {0, 0, 0, 0};
  CHECK(orc_per_sample(zero, 4, B, 11u, 0.4f, idx, w, NULL) == 0);  /* uniform fallback */

  free(pr); free(F); free(P);
  for (int i = 0; i < no; ++i) free(owned[i]);
  free(states); free(logits); free(u); free(gap); free(actions); free(forced); free(logp);
  free(val); free(rew); free(adv); free(ret); free(dones); free(barrier);
  free(nstates); free(qv); free(qgap); free(qt); free(qn); free(td); free(prio); free(expl);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer run: clean\n");
  return 0;
}
